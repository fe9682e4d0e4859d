// attn.hip -- the fused Sol-Attn forward kernel and the dense reference kernel (gfx950).
//
// Method (page "Sol-Attn: Accelerating Video Generation Inference via On-the-Fly Attention
// Sparsification", agihunt.info/papers/2607.24027): per query, a proxy score for every key block,
// a threshold tau = mu + beta * sigma over that query's proxy row (paragraph on the per-query
// threshold), exact attention on the kept blocks, and an approximation for the unselected blocks,
// all inside one online-softmax pass (paragraphs on the fused operator).  Proxy and
// approximation are fixed here as q . mean(K_blk) / sqrt(d) and one pooled token per unselected
// block with logit s + ln(n_blk) and value mean(V_blk).
//
// One workgroup = 4 waves = one tile of 128 query rows of one (batch, head); each wave owns 32
// rows, one row per lane pair (lanes c and c + 32).  Scores are computed transposed,
// S^T = K Q^T, with Q resident in registers as the B operand, so each lane sees its own query's
// scores.  Three sweeps:
//   1. proxy statistics: stream the pooled keys (as three bf16 pieces hi + mid + lo, whose bf16
//      products accumulate in fp32 to the fp32-accurate proxy) through LDS in chunks of 32 blocks;
//      accumulate sum (s - mu)^2 with mu = q . mean_j(Kbar_j) / sqrt(d) known up front, and the
//      largest pooled logit (an upper bound for the softmax max of the pooled tokens);
//   2. selection + pooled tokens: recompute the same proxies, set the per-row selection bits and
//      the tile's union of kept blocks in LDS, and fold every unselected block's pooled token into
//      the running softmax (P.Vbar on the matrix cores, Vbar as bf16);
//   3. exact attention: for each key block some row of the tile keeps, stage K (row-major) and V
//      (transposed) in LDS, S^T = K Q^T, mask the rows that did not keep the block, online
//      softmax update, O^T += V^T P^T.
// The proxy map is never written to memory; only the optional debug outputs leave the kernel.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace solattn {

namespace {

constexpr int kKeyTileDense = 128;  // keys per step of the dense kernel

// ---------------------------------------------------------------------------------------------
// LDS staging
// ---------------------------------------------------------------------------------------------

// K rows [r0, r0 + nrows) of one head -> ks (row-major, KT rows, 16-byte chunks swizzled).
// Rows >= nrows are zero-filled.
template <int D, int KT>
__device__ __forceinline__ void stage_k(const uint16_t* __restrict__ kb, int64_t r0, int nrows,
                                        u32x4* __restrict__ ks) {
  constexpr int kChunks = D / 8;
  constexpr int kIters = KT * kChunks / kThreads;
  const int t = threadIdx.x;
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int idx = it * kThreads + t;
    const int row = idx / kChunks;
    const int ch = idx % kChunks;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (row < nrows) val = *reinterpret_cast<const u32x4*>(kb + (r0 + row) * D + ch * 8);
    ks[swz16<kChunks>(row, ch)] = val;
  }
}

// V rows [r0, r0 + nrows) -> vt transposed: vt[d][key] in 8-byte slots of 4 keys, swizzled.
// Each thread moves a 4-key x 8-dim patch.  Rows >= nrows are zero-filled.
template <int D, int KT>
__device__ __forceinline__ void stage_vt(const uint16_t* __restrict__ vb, int64_t r0, int nrows,
                                         u32x2* __restrict__ vt) {
  constexpr int kChunks = D / 8;
  constexpr int kSlots = KT / 4;
  constexpr int kUnits = kSlots * kChunks;
  constexpr int kIters = (kUnits + kThreads - 1) / kThreads;
  const int t = threadIdx.x;
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int idx = it * kThreads + t;
    if (kUnits % kThreads != 0 && idx >= kUnits) break;
    const int kg = idx / kChunks;
    const int ch = idx % kChunks;
    u32x4 a[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 4 * kg + e;
      a[e] = u32x4{0u, 0u, 0u, 0u};
      if (row < nrows) a[e] = *reinterpret_cast<const u32x4*>(vb + (r0 + row) * D + ch * 8);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // dims 8ch + 2m (low halves) and 8ch + 2m + 1 (high halves)
      u32x2 lo, hi;
      lo[0] = (a[0][m] & 0xffffu) | (a[1][m] << 16);
      lo[1] = (a[2][m] & 0xffffu) | (a[3][m] << 16);
      hi[0] = (a[0][m] >> 16) | (a[1][m] & 0xffff0000u);
      hi[1] = (a[2][m] >> 16) | (a[3][m] & 0xffff0000u);
      vt[swz8<kSlots>(8 * ch + 2 * m, kg)] = lo;
      vt[swz8<kSlots>(8 * ch + 2 * m + 1, kg)] = hi;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Per-wave tile math
// ---------------------------------------------------------------------------------------------

// S^T for 32 keys (rows kr0 .. kr0 + 31 of the staged K tile) against this lane's query.
template <int D>
__device__ __forceinline__ f32x16 scores32(const u32x4* __restrict__ ks, int kr0,
                                           const bf16x8 (&qf)[D / 16]) {
  constexpr int kChunks = D / 8;
  const int lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
  f32x16 acc = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const u32x4 raw = ks[swz16<kChunks>(kr0 + c, 2 * kk + h)];
    acc = mfma32(__builtin_bit_cast(bf16x8, raw), qf[kk], acc);
  }
  return acc;
}

// The bf16 B operand holding probabilities 8*e2 .. 8*e2 + 7 of a 32-key score block, from the
// 8 packed words of that block.
__device__ __forceinline__ bf16x8 p_operand(const uint32_t* pk, int e2) {
  u32x4 w;
#pragma unroll
  for (int m = 0; m < 4; ++m) w[m] = pk[4 * e2 + m];
  return __builtin_bit_cast(bf16x8, w);
}

// Round 16 probabilities to bf16 pairs (pk[8]) and add the rounded values to `sum`.
__device__ __forceinline__ float round_p(const float* p, uint32_t* pk, float sum) {
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    pk[m] = pack_bf16x2(p[2 * m], p[2 * m + 1]);
    sum = add_bf16x2(pk[m], sum);
  }
  return sum;
}

// O^T[dsub] += V^T P^T for one 32-key score block kb (two 16-key steps), V^T staged in vt with
// kSlots 8-byte slots per d row.
template <int D, int kSlots>
__device__ __forceinline__ void pv32(const u32x2* __restrict__ vt, int kb, const uint32_t* pk,
                                     f32x16 (&o)[D / 32]) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
#pragma unroll
  for (int e2 = 0; e2 < 2; ++e2) {
    const bf16x8 b = p_operand(pk, e2);
    const int s0 = 8 * kb + 4 * e2 + h;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      const int row = 32 * ds + c;
      u32x4 raw;
      const u32x2 x0 = vt[swz8<kSlots>(row, s0)];
      const u32x2 x1 = vt[swz8<kSlots>(row, s0 + 2)];
      raw[0] = x0[0]; raw[1] = x0[1]; raw[2] = x1[0]; raw[3] = x1[1];
      o[ds] = mfma32(__builtin_bit_cast(bf16x8, raw), b, o[ds]);
    }
  }
}

// Key offset (within a 32-key score block) of result register v for lane half h.
__device__ __forceinline__ int key_of(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// One exact key tile (KT keys staged in ks / vt) folded into the running softmax of this lane.
// `active`: this lane's row takes part (kept block, valid row); `nvalid`: keys < N in the tile.
template <int D, int KT>
__device__ __forceinline__ void exact_tile(const u32x4* __restrict__ ks, const u32x2* __restrict__ vt,
                                           const bf16x8 (&qf)[D / 16], bool active, int nvalid,
                                           float sl2, float& mrun, float& lsum,
                                           f32x16 (&o)[D / 32]) {
  constexpr int NS = KT / 32;
  const int h = (threadIdx.x & 63) >> 5;
  f32x16 s[NS];
#pragma unroll
  for (int kb = 0; kb < NS; ++kb) s[kb] = scores32<D>(ks, 32 * kb, qf);

  float mt = -INFINITY;
  if (nvalid >= KT) {
#pragma unroll
    for (int kb = 0; kb < NS; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mt = fmaxf(mt, s[kb][v]);
  } else {
#pragma unroll
    for (int kb = 0; kb < NS; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (32 * kb + key_of(v, h) < nvalid) mt = fmaxf(mt, s[kb][v]);
  }
  mt = fmaxf(mt, swap_halves(mt));
  const float mnew = active ? fmaxf(mrun, mt * sl2) : mrun;
  const float alpha = exp2f(mrun - mnew);
  mrun = mnew;
  uint32_t pk[NS][8];
  float ps = 0.f;
#pragma unroll
  for (int kb = 0; kb < NS; ++kb) {
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const bool ok = active && (32 * kb + key_of(v, h) < nvalid);
      p[v] = ok ? exp2f(fmaf(s[kb][v], sl2, -mnew)) : 0.f;
    }
    ps = round_p(p, pk[kb], ps);
  }
  lsum = lsum * alpha + ps;
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[ds][v] *= alpha;
#pragma unroll
  for (int kb = 0; kb < NS; ++kb) pv32<D, KT / 4>(vt, kb, pk[kb], o);
}

// Write O = O^T / l for this lane's row (and its log-sum-exp if asked).
// out_f32 (optional): the same values before rounding to bf16.
template <int D>
__device__ __forceinline__ void epilogue(const f32x16 (&o)[D / 32], float mrun, float lsum,
                                         bool valid, uint16_t* __restrict__ orow, float* lse_out,
                                         float* __restrict__ frow = nullptr) {
  const int h = (threadIdx.x & 63) >> 5;
  const float l = lsum + swap_halves(lsum);
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  if (!valid) return;
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float x0 = o[ds][4 * g + 0] * inv, x1 = o[ds][4 * g + 1] * inv;
      const float x2 = o[ds][4 * g + 2] * inv, x3 = o[ds][4 * g + 3] * inv;
      u32x2 w;
      w[0] = pack_bf16x2(x0, x1);
      w[1] = pack_bf16x2(x2, x3);
      *reinterpret_cast<u32x2*>(orow + 32 * ds + 8 * g + 4 * h) = w;
      if (frow) *reinterpret_cast<f32x4*>(frow + 32 * ds + 8 * g + 4 * h) = f32x4{x0, x1, x2, x3};
    }
  if (lse_out && h == 0) *lse_out = l > 0.f ? (mrun + log2f(l)) * kLn2 : -INFINITY;
}

template <int D>
__device__ __forceinline__ void load_q(const uint16_t* __restrict__ qrow, bool valid,
                                       bf16x8 (&qf)[D / 16]) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (valid) raw = *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * h);
    qf[kk] = __builtin_bit_cast(bf16x8, raw);
  }
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// Fused Sol-Attn kernel
// ---------------------------------------------------------------------------------------------

template <int D, int BLK>
__global__ __launch_bounds__(kThreads) void sol_attn_kernel(SparseArgs a) {
  constexpr int kChunks = D / 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // region A: sweeps 1-2 (pooled chunk) or sweep 3 (K and V^T tiles)
  constexpr int kTileBytes = BLK * D * 2;
  constexpr int kChunkBytes = 3 * 32 * D * 2 + 2 * D * 32 * 2;
  constexpr int kRegionA = 2 * kTileBytes > kChunkBytes ? 2 * kTileBytes : kChunkBytes;
  const int W = (int)(a.Mp / 32);
  u32x4* ks = reinterpret_cast<u32x4*>(smem);
  u32x2* vt = reinterpret_cast<u32x2*>(smem + kTileBytes);
  u32x4* kpc = reinterpret_cast<u32x4*>(smem);                       // [3][32][D]
  u32x2* vbc = reinterpret_cast<u32x2*>(smem + 3 * 32 * D * 2);      // [D][32]
  uint32_t* rowmask = reinterpret_cast<uint32_t*>(smem + kRegionA);  // [128][W]
  uint32_t* umask = rowmask + kQTile * W;                            // [W]
  int* klist = reinterpret_cast<int*>(umask + W);                    // [Mp]
  int* nkept_s = klist + a.Mp;

  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, c = lane & 31, h = lane >> 5;
  const int64_t ntiles = (a.N + kQTile - 1) / kQTile;
  const int64_t bh = blockIdx.x / ntiles;
  const int64_t tile = blockIdx.x % ntiles;
  const int rloc = wave * 32 + c;                 // row within the tile
  const int64_t row = tile * kQTile + rloc;
  const bool rvalid = row < a.N;

  const uint16_t* qb = a.q + bh * a.N * D;
  const uint16_t* kb = a.k + bh * a.N * D;
  const uint16_t* vb = a.v + bh * a.N * D;

  bf16x8 qf[D / 16];
  load_q<D>(qb + row * D, rvalid, qf);

  const float inv_sqrt_d = 1.0f / sqrtf((float)D);
  const float sl2 = inv_sqrt_d * kLog2e;
  const int n_last = (int)(a.N - (a.M - 1) * (int64_t)a.block);
  const float l2n_full = log2f((float)a.block);
  const float l2n_last = log2f((float)n_last);

  // mu = q . kglob / sqrt(d): each lane half holds half of the head dimension.
  float mu;
  {
    const float* kg = a.kglob + bh * D;
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf((float)qf[kk][e], kg[16 * kk + 8 * h + e], part);
    mu = (part + swap_halves(part)) * inv_sqrt_d;
  }

  for (int w = t; w < W; w += kThreads) umask[w] = 0u;

  const int64_t nchunks = a.Mp / 32;
  const uint16_t* kp_hi = a.kp + ((0 * a.BH + bh) * a.Mp) * D;
  const uint16_t* kp_mid = a.kp + ((1 * a.BH + bh) * a.Mp) * D;
  const uint16_t* kp_lo = a.kp + ((2 * a.BH + bh) * a.Mp) * D;
  const uint16_t* vbt = a.vbt + bh * D * a.Mp;                  // Vbar^T, hi piece
  const uint16_t* vbt_lo = a.vbt + (a.BH + bh) * D * a.Mp;       // Vbar^T, lo piece

  auto stage_chunk = [&](int64_t cb, bool with_v) {
    constexpr int kPieceUnits = 32 * kChunks;
    for (int idx = t; idx < 3 * kPieceUnits; idx += kThreads) {
      const int p = idx / kPieceUnits;
      const int r = (idx % kPieceUnits) / kChunks;
      const int ch = idx % kChunks;
      const uint16_t* src = (p == 0 ? kp_lo : (p == 1 ? kp_mid : kp_hi)) + (cb * 32 + r) * D + ch * 8;
      kpc[p * 32 * kChunks + swz16<kChunks>(r, ch)] = *reinterpret_cast<const u32x4*>(src);
    }
    if (with_v) {
      // Vbar^T chunk, lo and hi pieces: D rows x 32 blocks = 8 slots of 4 blocks per row
      // (swizzled by row & 7)
      for (int idx = t; idx < 2 * D * 8; idx += kThreads) {
        const int piece = idx / (D * 8);
        const int r = (idx / 8) % D, sl = idx % 8;
        const uint16_t* src = (piece == 0 ? vbt_lo : vbt) + r * a.Mp + cb * 32 + sl * 4;
        vbc[piece * D * 8 + r * 8 + (sl ^ (r & 7))] = *reinterpret_cast<const u32x2*>(src);
      }
    }
  };
  // fp32-accurate proxies (raw dot products, not yet scaled) of this lane's query for the 32
  // blocks of the staged chunk: pieces accumulated smallest first.
  auto chunk_scores = [&]() {
    f32x16 acc = {};
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const u32x4 raw = kpc[p * 32 * kChunks + swz16<kChunks>(c, 2 * kk + h)];
        acc = mfma32(__builtin_bit_cast(bf16x8, raw), qf[kk], acc);
      }
    return acc;
  };

  // ---- sweep 1: sigma and the pooled-logit bound ----
  float ssq = 0.f;
  float pmax = -INFINITY;  // log2-domain pooled logit bound
  for (int64_t cb = 0; cb < nchunks; ++cb) {
    __syncthreads();
    stage_chunk(cb, false);
    __syncthreads();
    const f32x16 acc = chunk_scores();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t j = cb * 32 + key_of(v, h);
      if (j < a.M) {
        const float s = acc[v] * inv_sqrt_d;
        const float dl = s - mu;
        ssq = fmaf(dl, dl, ssq);
        pmax = fmaxf(pmax, fmaf(acc[v], sl2, j == a.M - 1 ? l2n_last : l2n_full));
      }
    }
  }
  ssq += swap_halves(ssq);
  pmax = fmaxf(pmax, swap_halves(pmax));
  const float sigma = sqrtf(ssq / (float)a.M);
  float tau;
  if (isinf(a.beta)) tau = a.beta;
  else tau = fmaf(a.beta, sigma, mu);
  if (!rvalid) tau = INFINITY;  // padding rows keep nothing

  // ---- sweep 2: selection bits, tile union, pooled tokens ----
  f32x16 o[D / 32];
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) o[ds] = f32x16{};
  float mrun = a.drop ? -1e30f : pmax;
  float lsum = 0.f;
  for (int64_t cb = 0; cb < nchunks; ++cb) {
    __syncthreads();
    stage_chunk(cb, !a.drop);
    __syncthreads();
    const f32x16 acc = chunk_scores();
    uint32_t bits = 0u;
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kj = key_of(v, h);
      const int64_t j = cb * 32 + kj;
      const bool valid = j < a.M;
      const bool sel = valid && (acc[v] * inv_sqrt_d >= tau);
      bits |= (sel ? 1u : 0u) << kj;
      p[v] = (valid && !sel && !a.drop)
                 ? exp2f(fmaf(acc[v], sl2, (j == a.M - 1 ? l2n_last : l2n_full) - mrun))
                 : 0.f;
    }
    const uint32_t word = bits | swap_halves_u(bits);
    if (h == 0) rowmask[rloc * W + cb] = word;
    if (h == 0 && a.mask && rvalid) a.mask[(bh * a.N + row) * W + cb] = word;
    uint32_t u = word;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) u |= (uint32_t)__shfl_xor((int)u, off, kWave);
    if (lane == 0 && u) atomicOr(&umask[cb], u);
    if (!a.drop) {
      uint32_t pk[8];
      lsum = round_p(p, pk, lsum);
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const bf16x8 bop = p_operand(pk, e2);
#pragma unroll
        for (int piece = 0; piece < 2; ++piece)  // Vbar lo, then hi
#pragma unroll
          for (int ds = 0; ds < D / 32; ++ds) {
            const int r = 32 * ds + c;
            const int s0 = 4 * e2 + h;
            const u32x2* vp = vbc + piece * D * 8;
            const u32x2 x0 = vp[r * 8 + (s0 ^ (r & 7))];
            const u32x2 x1 = vp[r * 8 + ((s0 + 2) ^ (r & 7))];
            u32x4 raw;
            raw[0] = x0[0]; raw[1] = x0[1]; raw[2] = x1[0]; raw[3] = x1[1];
            o[ds] = mfma32(__builtin_bit_cast(bf16x8, raw), bop, o[ds]);
          }
      }
    }
  }
  __syncthreads();

  // ---- kept-block list of the tile ----
  // each of the first W threads expands one union word at its prefix offset
  for (int w = t; w < W; w += kThreads) {
    int off = 0;
    for (int w2 = 0; w2 < w; ++w2) off += __builtin_popcount(umask[w2]);
    uint32_t u = umask[w];
    while (u) {
      const int b = __builtin_ctz(u);
      u &= u - 1u;
      klist[off++] = w * 32 + b;
    }
    if (w == W - 1) {
      *nkept_s = off;
      if (a.tile_kept) a.tile_kept[bh * ntiles + tile] = off;
    }
  }
  __syncthreads();
  const int nkept = *nkept_s;

  // ---- sweep 3: exact attention over the kept blocks ----
  for (int idx = 0; idx < nkept; ++idx) {
    const int j = klist[idx];
    const int64_t r0 = (int64_t)j * BLK;
    const int nrows = (int)((a.N - r0) < BLK ? (a.N - r0) : BLK);
    __syncthreads();
    stage_k<D, BLK>(kb, r0, nrows, ks);
    stage_vt<D, BLK>(vb, r0, nrows, vt);
    __syncthreads();
    const bool active = rvalid && ((rowmask[rloc * W + (j >> 5)] >> (j & 31)) & 1u);
    exact_tile<D, BLK>(ks, vt, qf, active, nrows, sl2, mrun, lsum, o);
  }

  epilogue<D>(o, mrun, lsum, rvalid, a.out + (bh * a.N + row) * D,
              a.lse ? a.lse + bh * a.N + row : nullptr,
              a.out_f32 ? a.out_f32 + (bh * a.N + row) * D : nullptr);
  if (h == 0 && rvalid) {
    if (a.mu) a.mu[bh * a.N + row] = mu;
    if (a.sigma) a.sigma[bh * a.N + row] = sigma;
    if (a.tau) a.tau[bh * a.N + row] = tau;
  }
}

// ---------------------------------------------------------------------------------------------
// Dense reference kernel: same tile machinery, every key, no routing.
// ---------------------------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(kThreads) void dense_attn_kernel(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v,
                                                              uint16_t* __restrict__ out,
                                                              float* __restrict__ lse, int64_t N) {
  constexpr int KT = kKeyTileDense;
  constexpr int kTileBytes = KT * D * 2;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  u32x4* ks = reinterpret_cast<u32x4*>(smem);
  u32x2* vt = reinterpret_cast<u32x2*>(smem + kTileBytes);

  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, c = lane & 31;
  const int64_t ntiles = (N + kQTile - 1) / kQTile;
  const int64_t bh = blockIdx.x / ntiles;
  const int64_t tile = blockIdx.x % ntiles;
  const int64_t row = tile * kQTile + wave * 32 + c;
  const bool rvalid = row < N;

  bf16x8 qf[D / 16];
  load_q<D>(q + (bh * N + row) * D, rvalid, qf);
  const float sl2 = kLog2e / sqrtf((float)D);

  f32x16 o[D / 32];
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) o[ds] = f32x16{};
  float mrun = -1e30f, lsum = 0.f;
  const uint16_t* kb = k + bh * N * D;
  const uint16_t* vb = v + bh * N * D;
  for (int64_t r0 = 0; r0 < N; r0 += KT) {
    const int nrows = (int)((N - r0) < KT ? (N - r0) : KT);
    __syncthreads();
    stage_k<D, KT>(kb, r0, nrows, ks);
    stage_vt<D, KT>(vb, r0, nrows, vt);
    __syncthreads();
    exact_tile<D, KT>(ks, vt, qf, true, nrows, sl2, mrun, lsum, o);
  }
  epilogue<D>(o, mrun, lsum, rvalid, out + (bh * N + row) * D, lse ? lse + bh * N + row : nullptr);
}

// ---------------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------------

static size_t sparse_smem_bytes(int d, int block, int64_t Mp) {
  const size_t tile = (size_t)block * d * 2;
  const size_t chunk = (size_t)3 * 32 * d * 2 + (size_t)2 * d * 32 * 2;
  const size_t regionA = 2 * tile > chunk ? 2 * tile : chunk;
  const size_t W = (size_t)(Mp / 32);
  return regionA + (size_t)kQTile * W * 4 + W * 4 + (size_t)Mp * 4 + 16;
}

template <int D, int BLK>
static hipError_t launch_sparse_t(const SparseArgs& a, hipStream_t stream) {
  const size_t smem = sparse_smem_bytes(D, BLK, a.Mp);
  auto kern = sol_attn_kernel<D, BLK>;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)smem);
  if (err != hipSuccess) return err;
  const int64_t ntiles = (a.N + kQTile - 1) / kQTile;
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.BH * ntiles)), dim3(kThreads), smem, stream, a);
  return hipGetLastError();
}

size_t sparse_lds_bytes(int d, int block, int64_t Mp) { return sparse_smem_bytes(d, block, Mp); }

hipError_t launch_sparse(int d, const SparseArgs& a, hipStream_t stream) {
  if (d == 64 && a.block == 64) return launch_sparse_t<64, 64>(a, stream);
  if (d == 64 && a.block == 128) return launch_sparse_t<64, 128>(a, stream);
  if (d == 128 && a.block == 64) return launch_sparse_t<128, 64>(a, stream);
  return launch_sparse_t<128, 128>(a, stream);
}

hipError_t launch_dense(int d, int64_t BH, int64_t N, const void* q, const void* k, const void* v,
                        void* out, float* lse, hipStream_t stream) {
  const int64_t ntiles = (N + kQTile - 1) / kQTile;
  const dim3 grid((unsigned)(BH * ntiles));
  if (d == 64) {
    const size_t smem = 2 * kKeyTileDense * 64 * 2;
    hipError_t err = hipFuncSetAttribute((const void*)dense_attn_kernel<64>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(dense_attn_kernel<64>, grid, dim3(kThreads), smem, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)out, lse, N);
  } else {
    const size_t smem = 2 * kKeyTileDense * 128 * 2;
    hipError_t err = hipFuncSetAttribute((const void*)dense_attn_kernel<128>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(dense_attn_kernel<128>, grid, dim3(kThreads), smem, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)out, lse, N);
  }
  return hipGetLastError();
}

}  // namespace solattn
