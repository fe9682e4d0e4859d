// stats.hip -- row statistics of the Sol-Attn forward pass (gfx950): the mean and population
// standard deviation of every query's proxy row and its selection threshold.
//
// Method (page "Sol-Attn: Accelerating Video Generation Inference via On-the-Fly Attention
// Sparsification", agihunt.info/papers/2607.24027): per query, a proxy score for every key block,
// a threshold tau = mu + beta * sigma over that query's proxy row (paragraph on the per-query
// threshold), exact attention on the kept blocks and an approximation for the unselected blocks,
// all inside one online-softmax pass (paragraphs on the fused operator).  Proxy and
// approximation are fixed here as q . mean(K_blk) / sqrt(d) and one pooled token per unselected
// block with logit s + ln(n_blk) and value mean(V_blk).
//
// Kernel
//   rowstats_kernel  mu_i = q_i . g / sqrt(d) and sigma_i^2 = q_i^T C q_i / d, where g and C are the
//                    mean and covariance of the pooled keys: the mean and population variance of
//                    the proxy row, exactly, without visiting its M entries.  mu in fp64.  C q is
//                    one bf16 matrix product per 32 rows over the hi + mid + lo pieces of C
//                    (fp32-accurate), after C's dominant directions, if any, are split off and
//                    taken in fp64 (see the pooled-key statistics).
//                    Writes tau_i = mu_i + beta * sigma_i (-inf for the fused kernel where
//                    sigma_i = 0: every proxy of such a row equals tau, so it keeps every block).
#include "tiles.hpp"

namespace solattn {

namespace {
// Row statistics: eight waves of 32 rows share the staged covariance pieces (two waves per SIMD
// hide each other's latency; the registers, and at d = 128 the pieces' 96 KB of LDS, allow one
// workgroup per CU), over up to kRowStatsPasses passes of 256 rows, each pass after the first
// reusing the staged pieces.  The pass count is chosen per launch (stats_passes).
constexpr int kRowStatsWaves = 8;
constexpr int kRowStatsThreads = 64 * kRowStatsWaves;
constexpr int kRowStatsRows = 32 * kRowStatsWaves;  // rows per pass
constexpr int kRowStatsPasses = 16;

// Passes per workgroup for `units` 256-row units over BH heads when `slots` workgroups run at
// once: the count that minimises rounds x (passes + 1), a round being one workgroup in every slot
// and the + 1 the staging of the pieces, which takes about as long as a pass; ties go to more
// passes.  (Wan, 40 x 296 units on 256 slots: 16 passes, 760 workgroups in three rounds; LTX,
// 32 x 24 units: 3 passes, 256 workgroups in one round, where 2 passes took two.)
int stats_passes(int64_t BH, int64_t units_per_head, int64_t slots) {
  int best = 1;
  int64_t best_cost = -1;
  for (int p = 1; p <= kRowStatsPasses; ++p) {
    const int64_t groups = BH * ((units_per_head + p - 1) / p);
    const int64_t cost = (groups + slots - 1) / slots * (p + 1);
    if (best_cost < 0 || cost <= best_cost) {
      best = p;
      best_cost = cost;
    }
    if (p >= units_per_head) break;  // more passes than units change nothing
  }
  return best;
}

// Workgroups of `kern` that run at once on the current device (CUs x workgroups per CU); the
// caller keeps the result per device (256 if the queries fail)
int64_t stats_slots(const void* kern, size_t smem) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kRowStatsThreads, smem) !=
          hipSuccess)
    return 256;
  return (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
}
}  // namespace

// ---------------------------------------------------------------------------------------------
// Row statistics: mu, sigma, tau of every query's proxy row
// ---------------------------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(kRowStatsThreads) void rowstats_kernel(RowStatsArgs a, int passes) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int64_t group_rows = (int64_t)kRowStatsRows * passes;
  const int64_t groups = (a.N + group_rows - 1) / group_rows;
  const int64_t bh = blockIdx.x / groups;
  const int64_t grp = blockIdx.x % groups;
  const int lane = threadIdx.x & 63, c = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform

  // C pieces (dominant directions removed) -> LDS, smallest first: tile p holds piece lo (p = 0),
  // mid (1), hi (2); then the mean pooled key and the dominant directions, both fp64
  const uint16_t* cbase = a.cp + bh * D * D;
  const int64_t piece = a.BH * D * D;
#pragma unroll
  for (int p = 0; p < 3; ++p)
    load_tile<D, D, kRowStatsThreads>(cbase + (2 - p) * piece, 0, D, smem + p * D * D * 2);
  double* kgl = (double*)(smem_raw + 3 * D * D * 2);
  double* ftl = kgl + D;  // [kFactorTop][D]
  const int ntop = __builtin_amdgcn_readfirstlane(a.ftop[bh]);
  for (int i = threadIdx.x; i < D; i += kRowStatsThreads) kgl[i] = a.kglob[bh * D + i];
  for (int i = threadIdx.x; i < kFactorTop * D; i += kRowStatsThreads)
    ftl[i] = i < ntop * D ? a.f64top[bh * kFactorTop * D + i] : 0.0;
  wait_vmcnt<0>();
  __syncthreads();

  // C operand of (piece p, k step kk, row tile ab): row 32 ab + c, chunk 2 kk + h.  The row swizzle
  // reads row bits below 5 only, so ab and p add whole tiles and kk flips chunk bits:
  // offset = p D D 2 + ab 32 2D + (crel ^ (kk << 5)).
  const int crel = c * (2 * D) + (swz<D>(c, h) << 4);
  const uint16_t* qhead = a.q + a.qs.base(bh);
  for (int pp = 0; pp < passes; ++pp) {
    const int64_t r0 = grp * group_rows + (int64_t)pp * kRowStatsRows;
    if (r0 >= a.N) break;
    const int64_t row0w = r0 + wave * 32;  // this wave's first row
    const int64_t row = row0w + c;
    const bool valid = row < a.N;
    // the wave's rows through a buffer resource that ends after its last valid row: rows past N
    // read as zeros without a branch per load
    const int64_t nrows = a.N - row0w < 32 ? a.N - row0w : 32;
    const uint32_t bytes = nrows > 0 ? (uint32_t)((nrows - 1) * a.qs.sn * 2 + D * 2) : 0u;
    const __amdgpu_buffer_rsrc_t qrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(qhead + row0w * a.qs.sn), (short)0, (int)bytes,
                                          0x00020000);
    const uint32_t qoff = (uint32_t)(c * a.qs.sn * 2);
    // B operand of k step kk, lane half h: q at d = 16 kk + 4 h + 0..3 and 16 kk + 8 + 4 h + 0..3 (the
    // pieces of C store their columns in the same order, see the pooled-key statistics).  These are
    // exactly the rows of C q this lane half receives, so the same registers serve q^T (C q):
    // element e of qf[kk] is q at d = 16 kk + 8 (e / 4) + 4 h + e % 4.
    bf16x8 qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const u32x2 lo = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(qrs, qoff + (16 * kk + 4 * h) * 2, 0, 0));
      const u32x2 hi = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(qrs, qoff + (16 * kk + 8 + 4 * h) * 2, 0, 0));
      qf[kk] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
    // all of the pass's loads are issued here, ahead of the matrix work that hides their latency
    __builtin_amdgcn_sched_barrier(0);
    // y[ab][v] = (C q)[32 ab + 8 (v/4) + 4 h + v%4]: D/32 independent accumulation chains,
    // pieces smallest first; the operand reads of step s + 1 are issued before step s's matrix
    // instructions
    constexpr int S = 3 * (D / 16);
    f32x16 y[D / 32];
#pragma unroll
    for (int ab = 0; ab < D / 32; ++ab) y[ab] = f32x16{};
    u32x4 ra[2][D / 32];
    auto read_step = [&](int s, u32x4 (&dst)[D / 32]) {
      const lds_u8* base = smem + (s / (D / 16)) * D * D * 2 + (crel ^ ((s % (D / 16)) << 5));
#pragma unroll
      for (int ab = 0; ab < D / 32; ++ab) dst[ab] = lds_read16(base + ab * 32 * 2 * D);
    };
    read_step(0, ra[0]);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (s + 1 < S) read_step(s + 1, ra[(s + 1) & 1]);
#pragma unroll
      for (int ab = 0; ab < D / 32; ++ab)
        y[ab] = mfma32(__builtin_bit_cast(bf16x8, ra[s & 1][ab]), qf[s % (D / 16)], y[ab]);
    }
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, D / 32, 0);
#pragma unroll
    for (int s = 0; s + 1 < S; ++s) {
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, D / 32, 0);
      __builtin_amdgcn_sched_group_barrier(kSgMfma, D / 32, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSgMfma, D / 32, 0);
    __builtin_amdgcn_sched_barrier(0);
    // q^T (C q) over this lane half's rows: y[ab][v] is row 32 ab + 8 g + 4 h + i (g = v / 4,
    // i = v % 4), whose query element is element 4 (g % 2) + i of qf[2 ab + g / 2]
    float vpart = 0.f;
#pragma unroll
    for (int ab = 0; ab < D / 32; ++ab)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        vpart = fmaf(y[ab][v], (float)qf[2 * ab + (v >> 3)][v & 7], vpart);
    // q . g over this lane half's D/2 elements, in fp64 (products and sums of the bf16 query
    // with the fp64 mean pooled key), and for heads with dominant directions (none for most) also
    // w_k . q in fp64, their squares summed into vtop.  Each query element is
    // converted where it is used, and the LDS offset is opaque to the optimiser, so that neither
    // the converted query nor the fp64 operands are held in registers across the pass loop.
    int hofs = 4 * h;
    __asm__ __volatile__("" : "+v"(hofs));
    double mpart = 0.0, vtop = 0.0;
    if (ntop == 0) {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          mpart = fma((double)(float)qf[kk][e], kgl[16 * kk + 8 * (e >> 2) + hofs + (e & 3)], mpart);
    } else {
      double z[kFactorTop] = {};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double qd = (double)(float)qf[kk][e];
          const int idx = 16 * kk + 8 * (e >> 2) + hofs + (e & 3);
          mpart = fma(qd, kgl[idx], mpart);
#pragma unroll
          for (int kt = 0; kt < kFactorTop; ++kt) z[kt] = fma(qd, ftl[kt * D + idx], z[kt]);
        }
#pragma unroll
      for (int kt = 0; kt < kFactorTop; ++kt) {  // rows past ntop are zero in LDS
        const double zz = z[kt] + __shfl_xor(z[kt], 32);
        vtop = fma(zz, zz, vtop);
      }
    }
    const double mu64 = (mpart + __shfl_xor(mpart, 32)) / sqrt((double)D);
    const float mu = (float)mu64;
    const float var = (float)((vtop + (double)pair_sum(vpart)) / (double)D);
    const float sigma = sqrtf(fmaxf(var, 0.f));
    const float tau = isinf(a.beta) ? a.beta : (float)fma((double)a.beta, (double)sigma, mu64);
    // sigma = 0 (one key block, q = 0, or identical pooled keys): every proxy of the row equals
    // mu = tau, so s >= tau keeps every block and the row is dense.  The fused kernel's s and this
    // mu are rounded along different paths and need not compare equal, so the threshold it reads
    // says so directly; the exported tau stays mu + beta * sigma.
    const float tau_sel = (!isinf(a.beta) && var <= 0.f) ? -INFINITY : tau;
    if (valid && h == 0) {
      a.tau[bh * a.N + row] = tau_sel;
      if (a.mu) a.mu[bh * a.N + row] = mu;
      if (a.sigma) a.sigma[bh * a.N + row] = sigma;
      if (a.tau_out) a.tau_out[bh * a.N + row] = tau;
    }
  }
}

template <int D>
static hipError_t launch_rowstats_t(const RowStatsArgs& a, hipStream_t stream) {
  const size_t smem = (size_t)3 * D * D * 2 + (size_t)(1 + kFactorTop) * D * sizeof(double);
  auto kern = rowstats_kernel<D>;
  hipError_t err = set_smem(kern, smem);
  if (err != hipSuccess) return err;
  // workgroups that run at once, per device (one cache per head dimension)
  static int64_t slots_of[64] = {};
  int dev = 0;
  err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  int64_t slots = dev >= 0 && dev < 64 ? slots_of[dev] : 0;
  if (slots <= 0) {
    slots = stats_slots((const void*)kern, smem);
    if (dev >= 0 && dev < 64) slots_of[dev] = slots;
  }
  const int passes = stats_passes(a.BH, (a.N + kRowStatsRows - 1) / kRowStatsRows, slots);
  const int64_t group_rows = (int64_t)kRowStatsRows * passes;
  const int64_t groups = (a.N + group_rows - 1) / group_rows;
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.BH * groups)), dim3(kRowStatsThreads), smem, stream, a,
                     passes);
  return hipGetLastError();
}

hipError_t launch_rowstats(int d, const RowStatsArgs& a, hipStream_t stream) {
  return d == 64 ? launch_rowstats_t<64>(a, stream) : launch_rowstats_t<128>(a, stream);
}

}  // namespace solattn
