// attn.hip -- the fused Sol-Attn forward kernels (gfx950).
//
// Method (page "Sol-Attn: Accelerating Video Generation Inference via On-the-Fly Attention
// Sparsification", agihunt.info/papers/2607.24027): per query, a proxy score for every key block,
// a threshold tau = mu + beta * sigma over that query's proxy row (paragraph on the per-query
// threshold), exact attention on the kept blocks and an approximation for the unselected blocks,
// all inside one online-softmax pass (paragraphs on the fused operator).  Proxy and
// approximation are fixed here as q . mean(K_blk) / sqrt(d) and one pooled token per unselected
// block with logit s + ln(n_blk) and value mean(V_blk).
//
// Kernels
//   sol_attn_kernel  (head dimension 64) one workgroup = 4 waves = 128 query rows of one
//                    (batch, head); each wave owns
//                    32 rows, one row per lane pair (lanes c and c + 32).  Scores are computed
//                    transposed, S^T = K Q^T, with Q resident in registers as the B operand, so a
//                    lane sees its own query's scores.
//                    Sweep over the pooled keys in chunks of 32 blocks: fp32-accurate proxies from
//                    the three bf16 pieces of Kbar, the selection bits s >= tau (per row, to the
//                    row-mask buffer) and their union over the tile (LDS), and every unselected
//                    block's pooled token folded into the running softmax (P Vbar on the matrix
//                    cores).  The chunks are double buffered like the exact stages.
//                    Exact loop over the blocks in the union, in stages of 64 keys, double
//                    buffered: K and V rows go straight from memory to LDS (global_load_lds), the
//                    next stage's copy overlapping this stage's math; S^T = K Q^T, rows that did not
//                    keep the block are masked, online softmax, O^T += V^T P^T with V^T read from
//                    the row-major V tile by the LDS transpose read (ds_read_b64_tr_b16).
//   sol_attn16_kernel (head dimension 128) the same stages with eight waves of 16 rows per
//                    128-row tile on the 16x16x32 matrix instructions: a wave skips a stage when
//                    none of its 16 rows keeps the block, and two workgroups per CU give four
//                    waves per SIMD.  In the pooled sweep each lane row's proxies are 8
//                    consecutive blocks (selection bits by constant shifts, one 16-byte operand
//                    read per pooled product) and a wave's union word is one DPP OR and store.
//                    Stages are pipelined by hand.  Per-stage scalar work is kept to one wave
//                    where it can be (the CU has one scalar unit): wave 0 alone walks the union
//                    and publishes each stage as a word in an LDS ring, and the lowest wave
//                    without math issues the whole next-stage copy.  A head's tiles are dealt
//                    round-robin to the four XCDs of one half of the chip (work_item_quad), and
//                    each tile's walk starts at a point that lines up the tiles running together
//                    on an XCD.  Given the
//                    tokens' latent grid, a workgroup's eight 16-row segments come from 2 frames
//                    x 4 latent rows instead of 128 consecutive rows (seg_row): rows that keep
//                    similar blocks, so the union each workgroup copies is smaller.
//   tile_union_kernel  the debug output tile_kept (blocks kept by each contiguous 128-row tile)
//                    from the selection words, for launches whose workgroups are not such tiles.
// The proxy map is never written to memory; only the optional debug outputs leave the kernel.
#include "tiles.hpp"

namespace solattn {

// ---------------------------------------------------------------------------------------------
// Fused Sol-Attn kernel
// ---------------------------------------------------------------------------------------------

// WAVES waves (32 query rows each) share each staged K/V tile: 4 (one 128-row tile, two
// workgroups per CU; launched at d = 64) or 8 (two 128-row tiles, one workgroup per CU, every
// copy feeding twice the rows; d = 128 only, whose 32-row pooled-key chunks split into whole
// loads for 512 threads; measured slower and not launched).
// Four waves: at most 168 VGPRs, so that three workgroups fit a CU (their LDS does, 33 KB each at
// d = 64); with 178 only two did, and LTX's fused pass ran 10-18% slower.
template <int D, int BLK, int WAVES>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 ? 3 : 8 / WAVES) void sol_attn_kernel(SparseArgs a) {
  constexpr int NT = 64 * WAVES;       // threads
  constexpr int QT = 32 * WAVES;       // query rows per workgroup
  constexpr int HALVES = WAVES / 4;    // 128-row tiles per workgroup
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  constexpr int kTileBytes = kStage * D * 2;          // one 64-row tile
  constexpr int kStageBytes = 2 * kTileBytes;         // K + V
  constexpr int kChunkTile = 32 * D * 2;              // one 32-row pooled tile
  constexpr int kRouteBuf = 4 * kChunkTile;           // Kbar lo, mid, hi + Vbar^T
  constexpr int kRegionA = 2 * kStageBytes > 2 * kRouteBuf ? 2 * kStageBytes : 2 * kRouteBuf;
  constexpr int kStagesPerBlock = BLK / kStage;
  uint32_t* umask = (uint32_t*)(smem_raw + kRegionA);  // [HALVES][W]: union of each 128-row tile
  const int W = (int)(a.Mp / 32);

  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, c = lane & 31, h = lane >> 5;
  const int64_t ntiles = (a.N + QT - 1) / QT;
  int64_t w;
  if (!work_item(a.BH * ntiles, w)) return;
  const int64_t bh = w / ntiles;
  const int64_t tile = w % ntiles;
  const int64_t row0 = tile * QT + wave * 32;   // first row of this wave
  uint32_t* my_umask = umask + (wave >> 2) * W;  // this wave's 128-row tile
  const int64_t row = row0 + c;
  const bool rvalid = row < a.N;

  const uint16_t* qb = a.q + a.in.base(bh);
  const uint16_t* kb = a.k + a.in.base(bh);
  const uint16_t* vb = a.v + a.in.base(bh);
  const int64_t sn = a.in.sn;
  uint32_t* rmask = a.rowmask + bh * W * a.N;  // word w of row r at rmask[w * N + r]

  bf16x8 qf[D / 16];
  load_q<D>(qb + row * sn, rvalid, qf);
  // padding rows keep nothing; with a caller's selection the threshold is not used
  const float tau = (rvalid && !a.mask_in) ? a.tau[bh * a.N + row] : INFINITY;
  // s >= tau  <=>  raw dot product >= tau * sqrt(d)  (compared in fp32)
  const float tau_raw = tau * sqrtf((float)D);

  const float inv_sqrt_d = 1.0f / sqrtf((float)D);
  const float sl2 = inv_sqrt_d * kLog2e;
  const int n_last = (int)(a.N - (a.M - 1) * (int64_t)a.block);
  const float l2n_full = log2f((float)a.block);
  const float l2n_last = log2f((float)n_last);
  // blocks [0, full_end) hold `block` keys each; a partial last block ends the range early
  const int64_t full_end = a.M - (n_last < a.block ? 1 : 0);

  for (int i = t; i < HALVES * W; i += NT) umask[i] = 0u;

  // ---- pooled sweep: selection bits, tile union, pooled tokens ----
  // Chunks of 32 blocks, double buffered: chunk tiles 0..2 = lo, mid, hi pieces of Kbar,
  // tile 3 = Vbar^T (D rows x 32 blocks).
  const int64_t piece = a.BH * a.Mp * D;
  const uint16_t* kp0 = a.kp + bh * a.Mp * D;  // hi; mid at + piece, lo at + 2 piece
  const uint16_t* vt0 = a.vbt + bh * D * a.Mp;
  f32x16 o[D / 32];
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) o[ds] = f32x16{};
  float mrun = -1e30f;  // running max, log2 domain
  float lsum = 0.f;
  const int nchunks = (int)(a.Mp / 32);
  const TileOffsets<D, 32, NT> coff(D);
  const VbtOffsets<D, NT> voff(a.Mp);
  auto issue_chunk = [&](int cb, int b) {
    lds_u8* base = smem + b * kRouteBuf;
    load_dense_rows<D, 32, NT>(kp0 + 2 * piece, (int64_t)cb * 32, coff, base);
    load_dense_rows<D, 32, NT>(kp0 + 1 * piece, (int64_t)cb * 32, coff, base + kChunkTile);
    load_dense_rows<D, 32, NT>(kp0, (int64_t)cb * 32, coff, base + 2 * kChunkTile);
    load_vbt_buf<D, NT>(vt0, a.Mp, cb, voff, base + 3 * kChunkTile);
  };
  // the caller's selection word of this row for chunk cb (loaded one chunk ahead, with the copy)
  const bool has_in = a.mask_in != nullptr;  // wave-uniform
  const uint32_t* min_row = has_in ? a.mask_in + (bh * a.N + row) * W : nullptr;
  auto in_word = [&](int cb) -> uint32_t { return (has_in && rvalid) ? min_row[cb] : 0u; };
  issue_chunk(0, 0);
  uint32_t win_next = in_word(0);
  for (int cb = 0; cb < nchunks; ++cb) {
    const int b = cb & 1;
    wait_vmcnt<0>();
    bar();  // publishes chunk cb, retires chunk cb - 1's buffer
    const uint32_t win = win_next;
    if (cb + 1 < nchunks) {
      issue_chunk(cb + 1, b ^ 1);
      win_next = in_word(cb + 1);
    }
    const lds_u8* base = smem + b * kRouteBuf;
    f32x16 acc = {};
#pragma unroll
    for (int p = 0; p < 3; ++p) acc = scores32<D>(base + p * kChunkTile, 0, qf, acc);
    uint32_t bits = 0u;
    float x[16];
    float cmax = -INFINITY;
    const int nvalid = (int)(a.M - (int64_t)cb * 32);  // blocks of this chunk below M
    if ((int64_t)cb * 32 + 32 <= full_end) {  // wave-uniform: all 32 blocks exist, full-size
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kj = key_of(v, h);
        const bool sel = has_in ? ((win >> kj) & 1u) != 0u : acc[v] >= tau_raw;
        bits |= (sel ? 1u : 0u) << kj;
        x[v] = sel ? -INFINITY : fmaf(acc[v], sl2, l2n_full);
        cmax = fmaxf(cmax, x[v]);
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kj = key_of(v, h);
        const bool valid = kj < nvalid;
        const bool sel = valid & (has_in ? ((win >> kj) & 1u) != 0u : acc[v] >= tau_raw);
        bits |= (sel ? 1u : 0u) << kj;
        x[v] = (valid & !sel) ? fmaf(acc[v], sl2, kj == nvalid - 1 ? l2n_last : l2n_full)
                              : -INFINITY;
        cmax = fmaxf(cmax, x[v]);
      }
    }
    const uint32_t word = pair_or(bits);
    if (h == 0 && rvalid) {
      rmask[(int64_t)cb * a.N + row] = word;
      if (a.mask_out) a.mask_out[(bh * a.N + row) * W + cb] = word;
    }
    // tile union: one LDS atomic OR per row (no dependent cross-lane reduction)
    if (h == 0 && word) atomicOr(&my_umask[cb], word);
    if (!a.drop) {
      cmax = pair_max(cmax);
      const bool grow = cmax > mrun + kSlack;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float mnew = grow ? cmax : mrun;
        const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
        mrun = mnew;
        lsum *= alpha;
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[ds][v] *= alpha;
      }
      float p[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(x[v] - mrun);
      uint32_t pk[8];
      lsum = round_p(p, pk, lsum);
      pv_pooled<D>(base + 3 * kChunkTile, pk, o);
    }
  }
  __syncthreads();  // union complete and chunk buffers retired before the exact loop

  // ---- exact attention over the kept blocks, double-buffered 64-key stages ----
  // Stage iterator: blocks j in the tile's union (ascending), stages s of each block with keys
  // below N.  All values are wave-uniform.
  int it_w = -1;
  uint32_t it_u = 0u;
  int it_j = -1, it_s = kStagesPerBlock;
  auto next_stage = [&](int& j, int& s) -> bool {
    for (;;) {
      if (it_j >= 0 && it_s + 1 < kStagesPerBlock && it_j * BLK + (it_s + 1) * kStage < (int)a.N) {
        ++it_s;
        j = it_j;
        s = it_s;
        return true;
      }
      while (it_u == 0u) {
        if (++it_w >= W) return false;
        uint32_t u = umask[it_w];
#pragma unroll
        for (int hh = 1; hh < HALVES; ++hh) u |= umask[hh * W + it_w];
        it_u = __builtin_amdgcn_readfirstlane(u);
      }
      const int b = __builtin_ctz(it_u);
      it_u &= it_u - 1u;
      it_j = it_w * 32 + b;
      it_s = -1;
    }
  };
  const TileOffsets<D, kStage, NT> toff(sn);
  auto issue = [&](int j, int s, int buf) {
    const int64_t r0 = (int64_t)j * BLK + s * kStage;
    lds_u8* base = smem + buf * kStageBytes;
    load_rows<D, kStage, NT>(kb, r0, a.N, sn, toff, base);
    load_rows<D, kStage, NT>(vb, r0, a.N, sn, toff, base + kTileBytes);
  };

  // One barrier per stage: it publishes the stage's copy (each lane waited for its own loads)
  // and retires the previous stage's reads, so the next copy can go into that buffer.  A row's
  // selection word for the next stage's block is loaded together with that stage's copy, so the
  // wait at the top of the loop covers it.
  auto load_word = [&](int wd) -> uint32_t {
    return rvalid ? rmask[(int64_t)wd * a.N + row] : 0u;
  };
  int cur_j = -1, cur_s = 0;
  bool have = next_stage(cur_j, cur_s);
  int mask_w = -1;
  uint32_t mask_word = 0u;
  if (have) {
    issue(cur_j, cur_s, 0);
    mask_w = cur_j >> 5;
    mask_word = load_word(mask_w);
  }
  int buf = 0;
  while (have) {
    wait_vmcnt<0>();
    bar();
    int nj = -1, ns = 0;
    const bool more = next_stage(nj, ns);
    int next_w = mask_w;
    uint32_t next_word = mask_word;
    if (more) {
      issue(nj, ns, buf ^ 1);
      if ((nj >> 5) != mask_w) {
        next_w = nj >> 5;
        next_word = load_word(next_w);
      }
    }
    const bool active = (mask_word >> (cur_j & 31)) & 1u;
    const int r0 = cur_j * BLK + cur_s * kStage;
    const int nvalid = (int)a.N - r0 < kStage ? (int)a.N - r0 : kStage;
    const lds_u8* base = smem + buf * kStageBytes;
    // a wave none of whose rows keeps the block has nothing to add (every probability would be
    // 0): it skips the stage's math and only takes part in the copies and barriers
    if (__builtin_amdgcn_ballot_w64(active))
      exact_stage<D>(base, base + kTileBytes, qf, active, nvalid, sl2, mrun, lsum, o);
    buf ^= 1;
    cur_j = nj;
    cur_s = ns;
    mask_w = next_w;
    mask_word = next_word;
    have = more;
  }
  if (a.tile_kept && t < HALVES) {  // blocks kept by some row of each 128-row tile
    const int64_t nt128 = (a.N + kQTile - 1) / kQTile;
    const int64_t t128 = tile * HALVES + t;
    int kept = 0;
    for (int i = 0; i < W; ++i) kept += __builtin_popcount(umask[t * W + i]);
    if (t128 < nt128) a.tile_kept[bh * nt128 + t128] = kept;
  }
  bar();  // every wave is done with the stage buffers before the epilogue reuses them

  epilogue<D>(o, mrun, lsum, row0, a.N, a.out + a.outs.base(bh), a.outs.sn,
              a.out_f32 ? a.out_f32 + bh * a.N * D : nullptr, a.lse ? a.lse + bh * a.N : nullptr,
              smem + wave * 32 * D * 2);
}

// ---------------------------------------------------------------------------------------------
// Fused kernel with 16-row waves (head dimension 128).  A 128-row query tile is split over eight
// waves of 16 rows, on the 16x16x32 matrix instructions (lane row g = lane / 16 holds keys or
// blocks 4g .. 4g + 3 of every 16, lane q = lane % 16 is the query).  Against the 4-wave kernel:
//   * a wave skips a stage when none of its 16 rows keeps the block, so the math executed follows
//     the kept blocks at 16-row rather than 32-row granularity;
//   * two workgroups per CU give four waves per SIMD instead of two, to cover the latency of the
//     waves that do have work.
// The stage structure (routing sweep over 32-block chunks, then the tile union's 64-key stages,
// double buffered, one barrier per stage) is that of sol_attn_kernel.
// ---------------------------------------------------------------------------------------------
constexpr int kWaves16 = 8;
constexpr int kThreads16 = 64 * kWaves16;

// OR over lanes 0 .. kWaves16 - 1 of x (the other lanes hold 0), returned in every lane as a
// wave-uniform value: three DPP steps within each 8-lane group (swap neighbours, swap pairs,
// mirror the 8; all lanes active), then lane 0's result.  DPP moves are plain vector operations,
// where cross-lane shuffles would be three dependent LDS-unit round trips.
static_assert(kWaves16 == 8, "one 8-lane DPP group");
__device__ __forceinline__ uint32_t union_of_waves(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  return __builtin_amdgcn_readfirstlane(x);
}

// The lane index, opaque to the optimiser: LDS addresses derived from it inside a loop are
// recomputed each iteration (a few VALU operations) instead of being hoisted out and held in
// registers for the whole loop, which at four waves per SIMD (128 VGPRs) would spill.
__device__ __forceinline__ int fresh_lane() {
  int l = threadIdx.x & 63;
  __asm__ __volatile__("" : "+v"(l));
  return l;
}

// Q fragments of this lane's query row for the 16x16x32 S^T products.  Lane row g takes the
// head-dimension chunks kk + (D/32) g (d = 8 kk + (D/4) g ..) at step kk: the K reads of one step
// then hit chunks D/32 apart across the lane rows, which the LDS serves without bank conflicts
// (adjacent chunks per lane row, the other choice, run at half rate).
template <int D>
__device__ __forceinline__ void load_q16(const uint16_t* __restrict__ qrow, bool valid,
                                         bf16x8 (&qf)[D / 32]) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (valid) raw = *reinterpret_cast<const u32x4*>(qrow + 8 * (kk + (D / 32) * g));
    qf[kk] = __builtin_bit_cast(bf16x8, raw);
  }
}

// S^T of the 16 rows kr0 .. kr0 + 15 of a swizzled LDS tile against this lane's query.
template <int D>
__device__ __forceinline__ f32x4 scores16(const lds_u8* tile, int kr0, const bf16x8 (&qf)[D / 32],
                                          f32x4 acc, int lane) {
  const int q = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const u32x4 raw = lds_read16(tile + tile_off<D>(kr0 + q, kk + (D / 32) * g));
    acc = mfma16(__builtin_bit_cast(bf16x8, raw), qf[kk], acc);
  }
  return acc;
}

// Probabilities of one 32-key group as the B operand of O^T += V^T P^T: lane row g holds the
// keys 4g .. 4g + 3 (from the first 16-key score tile) and 16 + 4g .. 16 + 4g + 3 (second tile),
// which fixes the k order the A operand must follow.
__device__ __forceinline__ bf16x8 p_operand16(const uint32_t (&pk)[4]) {
  u32x4 w;
#pragma unroll
  for (int m = 0; m < 4; ++m) w[m] = pk[m];
  return __builtin_bit_cast(bf16x8, w);
}

// O^T[dt] += Vbar^T P^T for the 32 pooled blocks of a routing chunk.  Lane row g holds the
// probabilities of blocks 8g .. 8g + 7 (the proxy reads take the pooled-key rows in that order), so
// the A operand of lane (g, q) is row 16 dt + q of the Vbar^T chunk tile at blocks 8g .. 8g + 7:
// one 16-byte chunk, whose swizzle (vbt_off) is the same for every dt.
template <int D>
__device__ __forceinline__ void pv_pooled16(const lds_u8* vt, const bf16x8& b, f32x4 (&o)[D / 16],
                                            int lane) {
  const int q = lane & 15, g = lane >> 4;
  const lds_u8* base = vt + vbt_off<D>(q, g);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const u32x4 raw = lds_read16(base + dt * 16 * 64);
    o[dt] = mfma16(__builtin_bit_cast(bf16x8, raw), b, o[dt]);
  }
}

// Scale the running state by 2^(mrun - mt) when a taking-part row's new maximum mt exceeds the
// running one by more than kSlack (wave-uniform branch; see kSlack).
template <int D>
__device__ __forceinline__ void raise_max16(float mt, bool active, float& mrun, float& lsum,
                                            f32x4 (&o)[D / 16]) {
  const bool grow = active && mt > mrun + kSlack;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float mnew = grow ? mt : mrun;
    const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
    mrun = mnew;
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[dt][i] *= alpha;
  }
}

// One 64-key stage folded into this lane's running softmax (as exact_stage, 16-row layout).
// Every lane of a query row holds the same running max; lsum is this lane's share of the row's
// denominator (the four lane rows are added in the epilogue).
template <int D>
__device__ __forceinline__ void exact_stage16(const lds_u8* ktile, const lds_u8* vtile,
                                              const bf16x8 (&qf)[D / 32], bool active, int nvalid,
                                              float sl2, float& mrun, float& lsum,
                                              f32x4 (&o)[D / 16], int lane) {
  constexpr int NT16 = kStage / 16;  // 16-key score tiles per stage
  constexpr int KS = D / 32;         // k steps per tile
  static_assert(KS == 4, "the address arithmetic below assumes 16 chunks per row");
  const int q = lane & 15, g = lane >> 4;
  // Swizzled addresses without per-read arithmetic: row q's swizzle f(q) is shared by rows
  // 16 kt + q, and chunk kk + 4 g = kk ^ 4 g, so the K read (kt, kk) sits at
  // (q's row offset + ((4 g ^ f(q)) << 4)) ^ (kk << 4), plus kt * 16 rows.
  const int krel = q * (2 * D) + (((KS * g) ^ swz<D>(q, 0)) << 4);
  auto kaddr = [&](int kt, int kk) { return ktile + 16 * kt * (2 * D) + (krel ^ (kk << 4)); };
  // Q.K^T, software-pipelined by hand: the operand reads of tile kt + 1 are issued before tile
  // kt's matrix instructions, so two tiles' reads are in flight at most
  f32x4 s[NT16];
  u32x4 kr[2][KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) kr[0][kk] = lds_read16(kaddr(0, kk));
#pragma unroll
  for (int kt = 0; kt < NT16; ++kt) {
    if (kt + 1 < NT16) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) kr[(kt + 1) & 1][kk] = lds_read16(kaddr(kt + 1, kk));
    }
    s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) s[kt] = mfma16(__builtin_bit_cast(bf16x8, kr[kt & 1][kk]), qf[kk], s[kt]);
  }
  __builtin_amdgcn_sched_group_barrier(kSgDsRead, KS, 0);
#pragma unroll
  for (int kt = 0; kt + 1 < NT16; ++kt) {
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, KS, 0);
    __builtin_amdgcn_sched_group_barrier(kSgMfma, KS, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSgMfma, KS, 0);
  __builtin_amdgcn_sched_barrier(0);
  if (nvalid < kStage) {  // wave-uniform
#pragma unroll
    for (int kt = 0; kt < NT16; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * kt + 4 * g + i >= nvalid) s[kt][i] = -INFINITY;
  }
  float mt = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < NT16; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[kt][i]);
  mt = quad_max(mt) * sl2;
  raise_max16<D>(mt, active, mrun, lsum, o);
  // rows that do not take part subtract +inf: every probability is 0
  const float moff = active ? -mrun : -INFINITY;
  float ps = 0.f;
  uint32_t pk[NT16 / 2][4];
#pragma unroll
  for (int grp = 0; grp < NT16 / 2; ++grp) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const f32x4& sv = s[2 * grp + h2];
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[0], sl2, moff));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[1], sl2, moff));
      const float p2 = __builtin_amdgcn_exp2f(fmaf(sv[2], sl2, moff));
      const float p3 = __builtin_amdgcn_exp2f(fmaf(sv[3], sl2, moff));
      pk[grp][2 * h2] = pack_bf16x2(p0, p1);
      pk[grp][2 * h2 + 1] = pack_bf16x2(p2, p3);
      ps = add_bf16x2(pk[grp][2 * h2], ps);
      ps = add_bf16x2(pk[grp][2 * h2 + 1], ps);
    }
  }
  lsum += ps;
  // O^T[dt] += V^T P^T, 2 x D/16 matrix instructions, the reads of the next one issued before the
  // current one.  For 32-key group grp, the A operand of lane (g, q) is V^T[16 dt + q][keys
  // 4g .. 4g + 3 and 16 + 4g .. 16 + 4g + 3 of the group]: two LDS transpose reads, in which the
  // 16 lanes of row g point at the four key rows (lane / 4) and four column quads (lane % 4) and
  // lane q receives column q of those rows.
  const int j = q;
  constexpr int NPV = (NT16 / 2) * (D / 16);
  // lane j of row g points at key row 4g + j / 4 (+ 32 grp, + 16 for the second read; neither
  // changes the swizzle) and columns 16 dt + 4 (j % 4): chunk 2 dt + (j % 4) / 2 = 2 dt ^ x, so
  // the address is the dt = 0 one XOR (dt << 5)
  const int rr = 4 * g + (j >> 2);
  const int vrel = rr * (2 * D) + ((((j & 3) >> 1) ^ swz<D>(rr, 0)) << 4) + (j & 1) * 8;
  s16x4 vr[2][2];
  auto read_v = [&](int idx, s16x4 (&dst)[2]) {
    const int grp = idx / (D / 16), dt = idx % (D / 16);
    const lds_u8* p = vtile + 32 * grp * (2 * D) + (vrel ^ (dt << 5));
    dst[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
    dst[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p + 16 * (2 * D)));
  };
  read_v(0, vr[0]);
#pragma unroll
  for (int idx = 0; idx < NPV; ++idx) {
    if (idx + 1 < NPV) read_v(idx + 1, vr[(idx + 1) & 1]);
    const int grp = idx / (D / 16), dt = idx % (D / 16);
    u32x4 raw;
    raw[0] = __builtin_bit_cast(u32x2, vr[idx & 1][0])[0];
    raw[1] = __builtin_bit_cast(u32x2, vr[idx & 1][0])[1];
    raw[2] = __builtin_bit_cast(u32x2, vr[idx & 1][1])[0];
    raw[3] = __builtin_bit_cast(u32x2, vr[idx & 1][1])[1];
    o[dt] = mfma16(__builtin_bit_cast(bf16x8, raw), p_operand16(pk[grp]), o[dt]);
  }
  __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
#pragma unroll
  for (int idx = 0; idx + 1 < NPV; ++idx) {
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// Write O = O^T / l for the wave's 16 rows through LDS (row-major, swizzled) so that every global
// store writes whole rows; also the optional fp32 output and log-sum-exp.
template <int D>
__device__ __forceinline__ void epilogue16(const f32x4 (&o)[D / 16], float mrun, float lsum,
                                           int64_t row0, int64_t N, uint16_t* __restrict__ out,
                                           int64_t on, float* __restrict__ out_f32,
                                           float* __restrict__ lse, lds_u8* stage) {
  const int lane = threadIdx.x & 63;
  const int q = lane & 15, g = lane >> 4;
  const int64_t row = row0 + q;
  const float l = quad_sum(lsum);
  const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const float x0 = o[dt][0] * inv, x1 = o[dt][1] * inv, x2 = o[dt][2] * inv, x3 = o[dt][3] * inv;
    u32x2 w;
    w[0] = pack_bf16x2(x0, x1);
    w[1] = pack_bf16x2(x2, x3);
    // d = 16 dt + 4 g + (0..3): chunk 2 dt + g / 2, half g % 2
    *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
        stage + tile_off<D>(q, 2 * dt + (g >> 1)) + 8 * (g & 1)) = w;
    if (out_f32 && row < N)
      *reinterpret_cast<f32x4*>(out_f32 + row * D + 16 * dt + 4 * g) = f32x4{x0, x1, x2, x3};
  }
  if (lse && g == 0 && row < N) lse[row] = l > 0.f ? (mrun + log2f(l)) * kLn2 : -INFINITY;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int kChunks = D / 8;
#pragma unroll
  for (int i = 0; i < 16 * kChunks / 64; ++i) {
    const int idx = i * 64 + lane;
    const int r = idx / kChunks, ch = idx % kChunks;
    const u32x4 v = lds_read16(stage + tile_off<D>(r, ch));
    if (row0 + r < N) *reinterpret_cast<u32x4*>(out + (row0 + r) * on + ch * 8) = v;
  }
}

// First row of the 16-row query segment at position p of the workgroup order (workgroup tile,
// wave w: p = kWaves16 * tile + w).  Without a latent grid (gS = 0) the rows are consecutive.
// With a grid of T frames, H rows and S segments of 16 tokens per row, positions run over pairs
// of frames (the last one single when T is odd); inside a pair over the horizontal segment, then
// the row, then the frame.  Eight consecutive positions then cover 2 frames x 4 rows at one
// horizontal position (a workgroup at the end of a column takes the next column's first rows),
// rows whose selections overlap more than those of 128 consecutive rows, and consecutive
// workgroups are vertical neighbours.  Positions past the last segment give N.
__device__ __forceinline__ int64_t seg_row(const SparseArgs& a, int64_t p) {
  if (a.gS == 0) return p * 16;
  const uint32_t T = (uint32_t)a.gT, H = (uint32_t)a.gH, S = (uint32_t)a.gS;
  if (p >= (int64_t)T * H * S) return a.N;
  const uint32_t pp = (uint32_t)p;
  const uint32_t per_pair = 2u * H * S;
  const uint32_t tp = pp / per_pair;                        // frame pair
  const uint32_t p1 = pp - tp * per_pair;
  const uint32_t tq = T - 2u * tp < 2u ? T - 2u * tp : 2u;  // frames in the pair
  const uint32_t xs = p1 / (H * tq);                        // horizontal segment
  const uint32_t r = p1 - xs * H * tq;
  const uint32_t y = r / tq, tt = r - y * tq;               // row, frame within the pair
  return ((int64_t)((2u * tp + tt) * H + y) * S + xs) * 16;
}

template <int D, int BLK>
__global__ __launch_bounds__(kThreads16, 4) void sol_attn16_kernel(SparseArgs a) {
  static_assert(D == 128, "the 16-row kernel serves head dimension 128");
  constexpr int NT = kThreads16;
  constexpr int QT = kQTile;                          // 128 query rows, 16 per wave
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  constexpr int kTileBytes = kStage * D * 2;          // one 64-row tile
  constexpr int kStageBytes = 2 * kTileBytes;         // K + V
  constexpr int kChunkTile = 32 * D * 2;              // one 32-row pooled tile
  constexpr int kRouteBuf = 4 * kChunkTile;           // Kbar lo, mid, hi + Vbar^T
  constexpr int kRegionA = 2 * kStageBytes > 2 * kRouteBuf ? 2 * kStageBytes : 2 * kRouteBuf;
  static_assert(kWaves16 * 16 * D * 2 <= kRegionA, "epilogue staging fits in the stage buffers");
  constexpr int kStagesPerBlock = BLK / kStage;
  const int W = (int)(a.Mp / 32);
  uint32_t* wmask = (uint32_t*)(smem_raw + kRegionA);  // [kWaves16][W]: union of each wave's rows

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform, in scalar registers
  const int lane = t & 63, q = lane & 15, g = lane >> 4;
  const int64_t ntiles = (a.N + QT - 1) / QT;
  int64_t w;
  if (!work_item_quad(a.BH * ntiles, w)) return;
  const int64_t bh = w / ntiles;
  const int64_t tile = w % ntiles;
  const int64_t row0 = seg_row(a, tile * kWaves16 + wave);  // first row of this wave
  const int64_t row = row0 + q;
  const bool rvalid = row < a.N;

  const uint16_t* qb = a.q + a.in.base(bh);
  const uint16_t* kb = a.k + a.in.base(bh);
  const uint16_t* vb = a.v + a.in.base(bh);
  const int64_t sn = a.in.sn;
  uint32_t* rmask = a.rowmask + bh * W * a.N;  // word w of row r at rmask[w * N + r]

  bf16x8 qf[D / 32];
  load_q16<D>(qb + row * sn, rvalid, qf);
  // padding rows keep nothing; with a caller's selection the threshold is not used
  const float tau = (rvalid && !a.mask_in) ? a.tau[bh * a.N + row] : INFINITY;
  // s >= tau  <=>  raw dot product >= tau * sqrt(d)  (compared in fp32)
  const float tau_raw = tau * sqrtf((float)D);

  const float inv_sqrt_d = 1.0f / sqrtf((float)D);
  const float sl2 = inv_sqrt_d * kLog2e;
  const int n_last = (int)(a.N - (a.M - 1) * (int64_t)a.block);
  const float l2n_full = log2f((float)a.block);
  const float l2n_last = log2f((float)n_last);
  // blocks [0, full_end) hold `block` keys each; a partial last block ends the range early
  const int64_t full_end = a.M - (n_last < a.block ? 1 : 0);

  for (int i = t; i < kWaves16 * W; i += NT) wmask[i] = 0u;

  // ---- pooled sweep: selection bits, tile union, pooled tokens ----
  const int64_t piece = a.BH * a.Mp * D;
  const uint16_t* kp0 = a.kp + bh * a.Mp * D;  // hi; mid at + piece, lo at + 2 piece
  const uint16_t* vt0 = a.vbt + bh * D * a.Mp;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -1e30f;  // running max, log2 domain
  float lsum = 0.f;
  const int nchunks = (int)(a.Mp / 32);
  const TileOffsets<D, 32, NT, true> coff(D);
  const VbtOffsets<D, NT> voff(a.Mp);
  auto issue_chunk = [&](int cb, int b) {
    lds_u8* base = smem + b * kRouteBuf;
    load_dense_rows<D, 32, NT>(kp0 + 2 * piece, (int64_t)cb * 32, coff, base);
    load_dense_rows<D, 32, NT>(kp0 + 1 * piece, (int64_t)cb * 32, coff, base + kChunkTile);
    load_dense_rows<D, 32, NT>(kp0, (int64_t)cb * 32, coff, base + 2 * kChunkTile);
    load_vbt_buf<D, NT>(vt0, a.Mp, cb, voff, base + 3 * kChunkTile);
  };
  const bool has_in = a.mask_in != nullptr;  // wave-uniform
  const uint32_t* min_row = has_in ? a.mask_in + (bh * a.N + row) * W : nullptr;
  auto in_word = [&](int cb) -> uint32_t { return (has_in && rvalid) ? min_row[cb] : 0u; };
  issue_chunk(0, 0);
  uint32_t win_next = in_word(0);
  for (int cb = 0; cb < nchunks; ++cb) {
    const int b = cb & 1;
    wait_vmcnt<0>();
    bar();  // publishes chunk cb, retires chunk cb - 1's buffer
    const uint32_t win = win_next;
    const lds_u8* base = smem + b * kRouteBuf;
    const int lane_v = fresh_lane();
    const int qv = lane_v & 15, gv = lane_v >> 4;
    // proxies: 6 (piece, block tile) steps of D/32 matrix instructions, pieces smallest first; the
    // reads of step st + 1 are issued before step st's matrix instructions
    constexpr int KS = D / 32;
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    u32x4 kr[2][KS];
    // lane qv reads pooled-key row 8 (qv / 4) + 4 bt + qv % 4 (block tile bt = st & 1), so that the
    // result registers (bt, i) of lane row g are block 8g + 4bt + i; that row's swizzle is the same
    // for both bt, and chunk kk + 4 gv = kk ^ 4 gv (see exact_stage16)
    const int prow = 8 * (qv >> 2) + (qv & 3);
    const int krel = prow * (2 * D) + (swz_pk(prow, KS * gv) << 4);
    auto read_step = [&](int st, u32x4 (&dst)[KS]) {
      const lds_u8* tl = base + (st >> 1) * kChunkTile + 4 * (st & 1) * (2 * D);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) dst[kk] = lds_read16(tl + (krel ^ (kk << 4)));
    };
    read_step(0, kr[0]);
#pragma unroll
    for (int st = 0; st < 6; ++st) {
      if (st + 1 < 6) read_step(st + 1, kr[(st + 1) & 1]);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        acc[st & 1] = mfma16(__builtin_bit_cast(bf16x8, kr[st & 1][kk]), qf[kk], acc[st & 1]);
    }
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, KS, 0);
#pragma unroll
    for (int st = 0; st + 1 < 6; ++st) {
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, KS, 0);
      __builtin_amdgcn_sched_group_barrier(kSgMfma, KS, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSgMfma, KS, 0);
    __builtin_amdgcn_sched_barrier(0);
    // register (bt, i) of lane row g holds block 8g + e of the chunk, e = 4bt + i; lb collects the
    // lane row's 8 selection bits at bits e, and the row's word has them at 8g + e
    uint32_t lb = 0u;
    float x[2][4];
    if ((int64_t)cb * 32 + 32 <= full_end) {  // wave-uniform: all 32 blocks exist, full-size
#pragma unroll
      for (int bt = 0; bt < 2; ++bt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool sel = acc[bt][i] >= tau_raw;  // tau is +inf with a caller's selection
          lb |= sel ? (1u << (4 * bt + i)) : 0u;
          x[bt][i] = sel ? -INFINITY : fmaf(acc[bt][i], sl2, l2n_full);
        }
      if (has_in) {  // wave-uniform: the caller's words decide
        lb = (win >> (8 * g)) & 0xffu;
#pragma unroll
        for (int bt = 0; bt < 2; ++bt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((lb >> (4 * bt + i)) & 1u) x[bt][i] = -INFINITY;
      }
    } else {
      const int nvalid = (int)(a.M - (int64_t)cb * 32);  // blocks of this chunk below M
#pragma unroll
      for (int bt = 0; bt < 2; ++bt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kj = 8 * g + 4 * bt + i;
          const bool valid = kj < nvalid;
          const bool sel = valid & (has_in ? ((win >> kj) & 1u) != 0u : acc[bt][i] >= tau_raw);
          lb |= (sel ? 1u : 0u) << (4 * bt + i);
          x[bt][i] = (valid & !sel)
                         ? fmaf(acc[bt][i], sl2, kj == nvalid - 1 ? l2n_last : l2n_full)
                         : -INFINITY;
        }
    }
    float cmax = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
    const uint32_t word = quad_or(lb << (8 * g));
    if (g == 0 && rvalid) {
      rmask[(int64_t)cb * a.N + row] = word;
      if (a.mask_out) a.mask_out[(bh * a.N + row) * W + cb] = word;
    }
    // the wave's union: each wave owns its word, so one lane stores the OR of its 16 rows
    const uint32_t wword = row16_or(word);
    if (lane == 0) wmask[wave * W + cb] = wword;
    // the next chunk's copy: after the proxy matrix instructions (every wave has math here, so a
    // copy issued at the top of the chunk would hold back the whole workgroup) and after this
    // chunk's selection store (which would otherwise queue behind the copies)
    if (cb + 1 < nchunks) {
      issue_chunk(cb + 1, b ^ 1);
      win_next = in_word(cb + 1);
    }
    if (!a.drop) {
      cmax = quad_max(cmax);
      raise_max16<D>(cmax, true, mrun, lsum, o);
      uint32_t pk[4];
#pragma unroll
      for (int bt = 0; bt < 2; ++bt) {
        const float p0 = __builtin_amdgcn_exp2f(x[bt][0] - mrun);
        const float p1 = __builtin_amdgcn_exp2f(x[bt][1] - mrun);
        const float p2 = __builtin_amdgcn_exp2f(x[bt][2] - mrun);
        const float p3 = __builtin_amdgcn_exp2f(x[bt][3] - mrun);
        pk[2 * bt] = pack_bf16x2(p0, p1);
        pk[2 * bt + 1] = pack_bf16x2(p2, p3);
        lsum = add_bf16x2(pk[2 * bt], lsum);
        lsum = add_bf16x2(pk[2 * bt + 1], lsum);
      }
      pv_pooled16<D>(base + 3 * kChunkTile, p_operand16(pk), o, lane_v);
    }
  }
  __syncthreads();  // union complete and chunk buffers retired before the exact loop

  // ---- exact attention over the kept blocks, double-buffered 64-key stages ----
  // Stage iterator over the union, with the set of waves that have math in each stage (bit w:
  // some row of wave w keeps the block).  All values are wave-uniform; only wave 0 runs it (see
  // the descriptor ring below).
  // The walk over the union starts at block p0 and wraps around.  The i-th tile run on an XCD
  // starts at i * M / 64 (64 tiles run on an XCD at a time, started in turn): in the steady
  // state the tiles running together then sweep the same region of keys at the same time, so
  // the K/V blocks they share are read from HBM once and served from L2 to the others.
  const int p0 = (int)(((int64_t)(blockIdx.x / 8) * a.M / 64) % a.M);
  const int w0 = p0 >> 5;
  const uint32_t low0 = (1u << (p0 & 31)) - 1u;  // blocks of word w0 below p0: visited last
  int it_k = -1, it_w = -1;
  uint32_t it_u = 0u, it_act = 0u;
  uint32_t it_ww = 0u;  // lane w < kWaves16: wave w's selection word for union word it_w
  int it_j = -1, it_s = kStagesPerBlock;
  auto next_stage = [&](int& j, int& s, uint32_t& act) -> bool {
    for (;;) {
      if (it_j >= 0 && it_s + 1 < kStagesPerBlock && it_j * BLK + (it_s + 1) * kStage < (int)a.N) {
        ++it_s;
        j = it_j;
        s = it_s;
        act = it_act;
        return true;
      }
      while (it_u == 0u) {
        if (++it_k > W) return false;
        it_w = it_k < W ? (w0 + it_k < W ? w0 + it_k : w0 + it_k - W) : w0;  // (w0 + it_k) mod W
        it_ww = lane < kWaves16 ? wmask[lane * W + it_w] : 0u;
        it_u = union_of_waves(it_ww);
        if (it_k == 0) it_u &= ~low0;
        if (it_k == W) it_u &= low0;
      }
      const int b = __builtin_ctz(it_u);
      it_u &= it_u - 1u;
      it_j = it_w * 32 + b;
      it_s = -1;
      it_act = (uint32_t)__builtin_amdgcn_ballot_w64(((it_ww >> b) & 1u) != 0u);
    }
  };
  // The next stage's copy, issued during a stage whose waves with math are `act`: when some wave
  // has none, the lowest such wave issues the whole copy, so that the waves that compute do not
  // queue behind the copy's issue.  One issuing wave pays the copy's scalar set-up once; spread
  // over all idle waves, the set-up ran in each of them through the CU's one scalar unit (3%
  // slower at Wan).  Copy offsets are recomputed per stage (see fresh_lane).
  // The scalar work here runs in every wave right after each stage's barrier, through the CU's
  // one scalar unit, so a computing wave leaves before any of it, and the issuing waves make one
  // 64-bit product per stage (the head's end offset is fixed per tile).
  const int64_t end_bytes = (a.N - 1) * sn * 2 + D * 2;  // head start to the end of its last row
  const uint32_t sn2 = (uint32_t)(sn * 2);
  // imask: bit w set for the waves that issue; one bit (that wave issues the whole copy) or all
  // eight (every wave issues its own share)
  auto issue = [&](int j, int s, int buf, uint32_t imask) {
    if (!((imask >> wave) & 1u)) return;
    const int64_t roff = ((int64_t)j * BLK + s * kStage) * sn;  // first row, in elements
    const int64_t rest = end_bytes - 2 * roff;
    const uint32_t bytes = (uint32_t)(rest < 0xffffffffll ? rest : 0xffffffffll);
    const i32x4_t krs = make_rsrc(kb + roff, bytes);
    const i32x4_t vrs = make_rsrc(vb + roff, bytes);
    lds_u8* base = smem + buf * kStageBytes;
    const int lane_v = fresh_lane();
    if (imask == (1u << kWaves16) - 1u) {
      copy_share<D, kStage, NT>(krs, sn2, wave, lane_v, base);
      copy_share<D, kStage, NT>(vrs, sn2, wave, lane_v, base + kTileBytes);
      return;
    }
    for (int k = 0; k < kWaves16; ++k) {
      copy_share<D, kStage, NT>(krs, sn2, k, lane_v, base);
      copy_share<D, kStage, NT>(vrs, sn2, k, lane_v, base + kTileBytes);
    }
  };
  // selection words through a buffer resource over word row wd (N words, at most 16 MB): scalar
  // base, 32-bit lane offset
  const uint32_t wvoff = (uint32_t)(row * 4);
  auto load_word = [&](int wd) -> uint32_t {
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        rmask + (int64_t)wd * a.N, (short)0, (int)(a.N * 4), 0x00020000);
    return rvalid ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(wrsrc, wvoff, 0, 0) : 0u;
  };
  // Only wave 0 walks the union; it publishes each stage as one word in a 4-slot LDS ring, three
  // stages ahead of the stage being computed, and every wave reads the descriptor of the stage
  // after next during this one.  The walk's scalar work then runs once per workgroup instead of
  // in all eight waves, through the CU's one scalar unit, and no wave waits on the ring.
  // Descriptor: bit 31 the stage exists, bit 29 it runs past N, bits 17..24 the waves that issue
  // the next stage's copy during it (the lowest wave without math alone, or all eight when every
  // wave has math), bit 16 the stage within the block, bits 0..15 the block (M <= 2^16).
  uint32_t* ring = wmask + kWaves16 * W;
  auto walk = [&]() -> uint32_t {
    int j, s;
    uint32_t act;
    if (!next_stage(j, s, act)) return 0u;
    const uint32_t idle = ~act & ((1u << kWaves16) - 1u);
    const uint32_t imask = idle ? idle & (0u - idle) : (1u << kWaves16) - 1u;
    const uint32_t partial = j * BLK + (s + 1) * kStage > (int)a.N ? 1u : 0u;
    return (1u << 31) | (partial << 29) | (imask << 17) | ((uint32_t)s << 16) | (uint32_t)j;
  };
  auto d_j = [](uint32_t d) { return (int)(d & 0xffffu); };
  auto d_s = [](uint32_t d) { return (int)((d >> 16) & 1u); };
  auto d_imask = [](uint32_t d) { return (d >> 17) & 0xffu; };
  auto d_partial = [](uint32_t d) { return ((d >> 29) & 1u) != 0u; };
  auto read_ring = [&](int slot) { return __builtin_amdgcn_readfirstlane(ring[slot]); };
  if (wave == 0) {
    const uint32_t w0d = walk();
    const uint32_t w1d = w0d ? walk() : 0u;
    const uint32_t w2d = w1d ? walk() : 0u;
    if (lane == 0) {
      ring[0] = w0d;
      ring[1] = w1d;
      ring[2] = w2d;
    }
  }
  __syncthreads();
  uint32_t dcur = read_ring(0), dnxt = read_ring(1);
  int mask_w = -1;
  uint32_t mask_word = 0u;
  if (dcur) {
    issue(d_j(dcur), d_s(dcur), 0, (1u << kWaves16) - 1u);  // every wave takes its own share
    mask_w = d_j(dcur) >> 5;
    mask_word = load_word(mask_w);
  }
  int buf = 0;
  for (int i = 0; dcur; ++i) {
    wait_vmcnt<0>();
    bar();  // publishes this stage's copy and the ring word written during the previous stage
    // the descriptor of the stage after next: loaded now (the slot is read even when there is no
    // next stage; its word is then ignored), made scalar after the math, so that the LDS round
    // trip overlaps the stage
    const uint32_t dnn_v = ring[(i + 2) & 3];
    int next_w = mask_w;
    uint32_t next_word = mask_word;
    if (dnxt) {
      issue(d_j(dnxt), d_s(dnxt), buf ^ 1, d_imask(dcur));
      if ((d_j(dnxt) >> 5) != mask_w) {
        next_w = d_j(dnxt) >> 5;
        next_word = load_word(next_w);
      }
    }
    const int cur_j = d_j(dcur);
    const bool active = (mask_word >> (cur_j & 31)) & 1u;
    const int nvalid = d_partial(dcur) ? (int)a.N - (cur_j * BLK + d_s(dcur) * kStage) : kStage;
    const lds_u8* base = smem + buf * kStageBytes;
    // a wave none of whose 16 rows keeps the block skips the stage's math
    if (__builtin_amdgcn_ballot_w64(active))
      exact_stage16<D>(base, base + kTileBytes, qf, active, nvalid, sl2, mrun, lsum, o,
                       fresh_lane());
    const uint32_t dnn = dnxt ? __builtin_amdgcn_readfirstlane(dnn_v) : 0u;
    // three stages ahead, after the math; slot (i + 3) & 3 was last read three stages ago.  The
    // write has completed before wave 0 reaches the next barrier (bar() has no fence).
    if (wave == 0 && dnn) {
      const uint32_t d3 = walk();
      if (lane == 0) ring[(i + 3) & 3] = d3;
      wait_lgkmcnt0();
    }
    buf ^= 1;
    mask_w = next_w;
    mask_word = next_word;
    dcur = dnxt;
    dnxt = dnn;
  }
  // blocks kept by some row of the tile (with a latent grid the workgroup's rows are not a
  // contiguous tile: tile_union_kernel fills tile_kept instead)
  if (a.tile_kept && a.gS == 0 && wave == 0) {
    int kept = 0;
    for (int i = 0; i < W; ++i)
      kept += __builtin_popcount(union_of_waves(lane < kWaves16 ? wmask[lane * W + i] : 0u));
    if (lane == 0) a.tile_kept[bh * ntiles + tile] = kept;
  }
  bar();  // every wave is done with the stage buffers before the epilogue reuses them

  epilogue16<D>(o, mrun, lsum, row0, a.N, a.out + a.outs.base(bh), a.outs.sn,
                a.out_f32 ? a.out_f32 + bh * a.N * D : nullptr, a.lse ? a.lse + bh * a.N : nullptr,
                smem + wave * 16 * D * 2);
}

// ---------------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------------

static size_t sparse_smem_bytes(int d, int64_t Mp, int halves) {
  const size_t stage = (size_t)2 * kStage * d * 2;
  const size_t route = (size_t)4 * 32 * d * 2;
  const size_t regionA = 2 * stage > 2 * route ? 2 * stage : 2 * route;
  return regionA + (size_t)halves * (Mp / 32) * 4;
}

template <int D, int BLK, int WAVES>
static hipError_t launch_sparse_t(const SparseArgs& a, hipStream_t stream) {
  const size_t smem = sparse_smem_bytes(D, a.Mp, WAVES / 4);
  auto kern = sol_attn_kernel<D, BLK, WAVES>;
  hipError_t err = set_smem(kern, smem);
  if (err != hipSuccess) return err;
  const int64_t ntiles = (a.N + 32 * WAVES - 1) / (32 * WAVES);
  hipLaunchKernelGGL(kern, dim3(xcd_grid(a.BH * ntiles)), dim3(64 * WAVES), smem, stream, a);
  return hipGetLastError();
}

// The 16-row kernel: eight waves of 16 rows per 128-row tile, two workgroups per CU (four waves
// per SIMD).  Dynamic LDS: the stage / routing-chunk region, the waves' union words and the
// 4-slot stage descriptor ring.
template <int D, int BLK>
static hipError_t launch_sparse16_t(const SparseArgs& a, hipStream_t stream) {
  const size_t smem = sparse_smem_bytes(D, a.Mp, 0) + (size_t)kWaves16 * (a.Mp / 32) * 4 + 4 * 4;
  auto kern = sol_attn16_kernel<D, BLK>;
  hipError_t err = set_smem(kern, smem);
  if (err != hipSuccess) return err;
  const int64_t ntiles = (a.N + kQTile - 1) / kQTile;
  hipLaunchKernelGGL(kern, dim3(xcd_grid(a.BH * ntiles)), dim3(kThreads16), smem, stream, a);
  return hipGetLastError();
}

// tile_kept of the debug outputs when the fused kernel's workgroups are not contiguous tiles: one
// wave per (head, 128-row tile) ORs the tile's selection words, word by word, and counts the bits.
__global__ __launch_bounds__(64) void tile_union_kernel(const uint32_t* __restrict__ rowmask,
                                                        int64_t N, int64_t W, int64_t ntiles,
                                                        int32_t* __restrict__ tile_kept) {
  const int64_t bh = blockIdx.x / ntiles, t = blockIdx.x % ntiles;
  const int lane = threadIdx.x;
  const uint32_t* rm = rowmask + bh * W * N;
  const int64_t r0 = t * kQTile + lane, r1 = r0 + 64;
  int kept = 0;
  for (int64_t w = 0; w < W; ++w) {
    uint32_t x = (r0 < N ? rm[w * N + r0] : 0u) | (r1 < N ? rm[w * N + r1] : 0u);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x |= (uint32_t)__shfl_xor((int)x, o);
    kept += __builtin_popcount(x);
  }
  if (lane == 0) tile_kept[bh * ntiles + t] = kept;
}

hipError_t launch_tile_union(int64_t BH, int64_t N, int64_t W, const uint32_t* rowmask,
                             int32_t* tile_kept, hipStream_t stream) {
  const int64_t ntiles = (N + kQTile - 1) / kQTile;
  hipLaunchKernelGGL(tile_union_kernel, dim3((unsigned)(BH * ntiles)), dim3(64), 0, stream, rowmask,
                     N, W, ntiles, tile_kept);
  return hipGetLastError();
}

hipError_t launch_sparse(int d, const SparseArgs& a, hipStream_t stream) {
  if (d == 64 && a.block == 64) return launch_sparse_t<64, 64, 4>(a, stream);
  if (d == 64 && a.block == 128) return launch_sparse_t<64, 128, 4>(a, stream);
  if (d == 128 && a.block == 64) return launch_sparse16_t<128, 64>(a, stream);
  return launch_sparse16_t<128, 128>(a, stream);
}

}  // namespace solattn
