// attn.hip -- row statistics, the fused Sol-Attn forward kernel and the dense reference kernel
// (gfx950).
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
//   rowstats_kernel  mu_i = q_i . g / sqrt(d) and sigma_i^2 = q_i^T C q_i / d, where g and C are the
//                    mean and covariance of the pooled keys: the mean and population variance of
//                    the proxy row, exactly, without visiting its M entries.  mu in fp64.  C q is
//                    one bf16 matrix product per 32 rows over the hi + mid + lo pieces of C
//                    (fp32-accurate), after C's dominant directions, if any, are split off and
//                    taken in fp64 (see the pooled-key statistics).
//                    Writes tau_i = mu_i + beta * sigma_i (-inf for the fused kernel where
//                    sigma_i = 0: every proxy of such a row equals tau, so it keeps every block).
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
//                    without math issues the whole next-stage copy.  Each tile's walk starts at
//                    a point that lines up the tiles running together on an XCD.
//   dense_attn_kernel the exact loop over every key: the reference the speedup is measured against.
// The proxy map is never written to memory; only the optional debug outputs leave the kernel.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace solattn {

namespace {

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kStage = 64;  // keys per pipeline stage
// Row statistics: eight waves of 32 rows share the staged covariance pieces (two waves per SIMD
// hide each other's latency; the pieces' 96 KB of LDS at d = 128 allow one workgroup per CU),
// over kRowStatsPasses passes of 256 rows.
constexpr int kRowStatsWaves = 8;
constexpr int kRowStatsThreads = 64 * kRowStatsWaves;
constexpr int kRowStatsRows = 32 * kRowStatsWaves;  // rows per pass
constexpr int kRowStatsPasses = 8;

// ---------------------------------------------------------------------------------------------
// LDS tiles: row-major [rows][D] bf16, 16-byte chunks XOR-swizzled per row.  The swizzle makes
// the access patterns conflict-free on a 256-byte-wide LDS: 16 consecutive rows read at one
// logical chunk (the K / Kbar A operand) land on 16 distinct 16-byte bank groups, and the
// transpose reads of V land on distinct chunks per 32 lanes -- 4 consecutive rows x 4 adjacent
// chunks (32x32 layout), or two 4-row groups x 2 chunks (16x16 layout, where bit 2 of the row
// goes to chunk bit 1 so that the two groups differ in a bit the read does not cover).
// ---------------------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz(int row, int ch) {
  if constexpr (D == 128)
    return ch ^ (((row & 3) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1));
  else return ch ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
// Pooled-key chunk tiles of the 16-row kernel (D = 128, 32 rows): the proxy reads take rows in
// the order 8 (q / 4) + 4 bt + q % 4 for lane q and block tile bt (so that lane row g's scores are
// blocks 8g .. 8g + 7), which leaves row bit 2 fixed across the 16 lanes of a read; the swizzle
// takes row bits 0, 1, 3 and 4, distinct for those 16 rows.
__device__ __forceinline__ int swz_pk(int row, int ch) {
  return ch ^ (((row & 3) << 2) | ((row >> 3) & 3));
}
template <int D>
__device__ __forceinline__ int tile_off(int row, int ch) {  // byte offset of a 16-byte chunk
  return row * (2 * D) + (swz<D>(row, ch) << 4);
}

// Copy rows [row0, row0 + ROWS) of a row-major [*, D] bf16 matrix into an LDS tile with
// global_load_lds (16 bytes per lane, no registers).  Rows >= limit read row limit - 1 instead
// (finite data; such keys are masked).  Every thread of an NT-thread workgroup issues
// ROWS * D / 8 / NT loads.
template <int D, int ROWS, int NT = kThreads>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ src, int64_t row0,
                                          int64_t limit, lds_u8* tile) {
  constexpr int kChunks = D / 8;
  constexpr int kIters = ROWS * kChunks / NT;
  static_assert(ROWS * kChunks % NT == 0, "tile must split into whole wave loads");
  const int t = threadIdx.x;
  const int wave = t >> 6;
#pragma unroll
  for (int i = 0; i < kIters; ++i) {
    const int p = i * NT + t;  // physical slot written by this lane
    const int row = p / kChunks;
    const int ch = swz<D>(row, p % kChunks);  // logical chunk stored in that slot (XOR involution)
    int64_t grow = row0 + row;
    if (grow >= limit) grow = limit - 1;
    const uint16_t* g = src + grow * D + ch * 8;
    lds_u8* dst = tile + (i * NT + wave * 64) * 16;  // wave-uniform; lane l lands at +16 l
    __builtin_amdgcn_global_load_lds((const void*)g, (__attribute__((address_space(3))) void*)dst,
                                     16, 0, 0);
  }
}
template <int D, int ROWS, int NT = kThreads>
constexpr int tile_loads() { return ROWS * (D / 8) / NT; }

// Buffer resource descriptor over `bytes` bytes at `base` (raw buffer: stride 0, 32-bit dword
// data format): loads past `bytes` return zeros.  Built from wave-uniform values, so it lives in
// scalar registers.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t addr = (uint64_t)(uintptr_t)base;
  i32x4_t r;
  r[0] = (int)__builtin_amdgcn_readfirstlane((uint32_t)addr);
  r[1] = (int)__builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32) & 0xffffu);
  r[2] = (int)__builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000;
  return r;
}

// Per-lane byte offsets, within a ROWS-row tile of a bf16 matrix with rows of D contiguous
// elements sn elements apart, of the 16 bytes each lane copies so that the LDS tile comes out
// swizzled (see load_tile).
// PK: the pooled-key tile swizzle (swz_pk) instead of swz.
template <int D, int ROWS, int NT = kThreads, bool PK = false>
struct TileOffsets {
  static_assert(!PK || D == 128, "the pooled-key swizzle covers 16 chunks per row");
  uint32_t v[tile_loads<D, ROWS, NT>()];
  __device__ __forceinline__ explicit TileOffsets(int64_t sn, int tid = (int)threadIdx.x) {
    constexpr int kChunks = D / 8;
#pragma unroll
    for (int i = 0; i < tile_loads<D, ROWS, NT>(); ++i) {
      const int p = i * NT + tid;
      const int row = p / kChunks;
      const int ch = PK ? swz_pk(row, p % kChunks) : swz<D>(row, p % kChunks);
      v[i] = (uint32_t)(row * sn * 2 + ch * 16);
    }
  }
};

// Copy the first ROWS rows of the buffer `rsrc` into LDS with buffer loads (16 bytes per lane,
// straight to LDS).  Rows past the buffer end read as zeros: the range check covers the per-lane
// offset, so callers start the resource at the tile (soff stays 0; a scalar offset would bypass
// the check).
//
// The copy is issued as an asm statement rather than through the compiler's LDS-DMA builtin: the
// compiler cannot tell which LDS buffer such a copy writes, and would make every LDS transpose
// read wait for all copies in flight -- including the next stage's prefetch, serialising copy and
// math.  The instruction has no register result (its destination is LDS), its address operands
// are consumed at issue, and the callers order the LDS traffic themselves: wait_vmcnt before the
// barrier that publishes a tile, and a barrier before a buffer is refilled.
// One copy of 16 bytes per lane from the buffer `rsrc` (at byte voff + soff) to LDS; lane l lands
// at dst + 16 l, dst wave-uniform.  The LDS destination base goes in m0 as an operand bound to
// that register, so the compiler sets m0 itself (one scalar move; it knows m0's value afterwards)
// and knows this statement writes LDS.  These copies sit in every stage's scalar-bound
// bookkeeping, where a save and restore of m0 around each would cost two more scalar
// instructions per copy.
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t voff, uint32_t soff, lds_u8* dst) {
  __asm__ __volatile__("buffer_load_dwordx4 %[voff], %[rsrc], %[soff] offen lds"
                       :
                       : "{m0}"(dst), [voff] "v"(voff), [rsrc] "s"(rsrc), [soff] "s"(soff)
                       : "memory");
}

template <int D, int ROWS, int NT = kThreads, bool PK = false>
__device__ __forceinline__ void load_tile_buf(i32x4_t rsrc, uint32_t soff,
                                              const TileOffsets<D, ROWS, NT, PK>& off, lds_u8* tile) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < tile_loads<D, ROWS, NT>(); ++i)
    dma16(rsrc, off.v[i], soff, tile + (i * NT + wave * 64) * 16);
}

// Rows [row0, row0 + ROWS) of a row-major [*, D] bf16 matrix whose rows all exist (pooled-key
// pieces, padded to Mp rows), copied as load_tile does but without the compiler's LDS-DMA builtin
// (see load_tile_buf): a builtin copy in flight makes the compiler wait for every outstanding
// memory operation before the next LDS write, which stalls the routing sweep once per chunk.
template <int D, int ROWS, int NT = kThreads, bool PK = false>
__device__ __forceinline__ void load_dense_rows(const uint16_t* src, int64_t row0,
                                                const TileOffsets<D, ROWS, NT, PK>& off, lds_u8* tile) {
  load_tile_buf<D, ROWS, NT, PK>(make_rsrc(src + row0 * D, ROWS * D * 2), 0u, off, tile);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt lgkmcnt(0) alone (gfx9 encoding: vmcnt and expcnt left at their maxima).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

// Rows [r0, r0 + ROWS) of a row-strided bf16 matrix (row r at base + r * sn, rows below `limit`)
// into an LDS tile; rows at or beyond `limit` read as zeros (the buffer ends after the last valid
// row, and every later row starts at or beyond that end since sn >= D).  The buffer covers all
// the remaining valid rows, not just this tile's: measured on gfx950, a resource cut to the tile
// made the dense loop fetch 3.7x more bytes from beyond L2.
template <int D, int ROWS, int NT = kThreads>
__device__ __forceinline__ void load_rows(const uint16_t* base, int64_t r0, int64_t limit, int64_t sn,
                                          const TileOffsets<D, ROWS, NT>& off, lds_u8* tile) {
  const int64_t rest = (limit - r0 - 1) * sn * 2 + D * 2;
  const uint32_t bytes = (uint32_t)(rest < 0xffffffffll ? rest : 0xffffffffll);
  load_tile_buf<D, ROWS, NT>(make_rsrc(base + r0 * sn, bytes), 0u, off, tile);
}

// Share k of the copy load_rows makes of rows [r0, r0 + ROWS) (the loads lane l of wave k issues
// there), issued by the calling wave instead; k is wave-uniform.  rsrc starts at row r0 and ends
// after the head's last valid row (load_rows' range); sn2 is the row stride in bytes.
template <int D, int ROWS, int NT>
__device__ __forceinline__ void copy_share(i32x4_t rsrc, uint32_t sn2, int k, int lane,
                                           lds_u8* tile) {
  constexpr int kChunks = D / 8;
  static_assert(64 % kChunks == 0 && NT % kChunks == 0, "a wave's slots cover whole rows");
  // The offsets TileOffsets would give, split into a wave-uniform and a per-lane part: slot
  // i NT + 64 k + lane holds row rs + rl (rs = (i NT + 64 k) / kChunks, a multiple of
  // 64 / kChunks, and rl = lane / kChunks < 64 / kChunks) and logical chunk
  // (lane % kChunks) ^ f(rs + rl).  The swizzle f only permutes row bits, so
  // f(rs + rl) = f(rs) ^ f(rl).
  const int rl = lane / kChunks;
  const uint32_t lane_row = (uint32_t)rl * sn2;
  const int cl = swz<D>(rl, lane % kChunks);
#pragma unroll
  for (int i = 0; i < tile_loads<D, ROWS, NT>(); ++i) {
    const int rs = (i * NT + 64 * k) / kChunks;  // wave-uniform
    const uint32_t voff = (uint32_t)rs * sn2 + lane_row + ((uint32_t)(cl ^ swz<D>(rs, 0)) << 4);
    dma16(rsrc, voff, 0u, tile + (i * NT + k * 64) * 16);
  }
}

// Workgroup barrier without the memory fence of __syncthreads: the pipelined loops order their
// LDS traffic themselves (explicit vmcnt waits for the LDS-bound copies; LDS reads are consumed
// before the barrier), so the fence's wait for every outstanding load -- including the next
// stage's prefetch -- is not wanted.  The empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void bar() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

__device__ __forceinline__ u32x4 lds_read16(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
}

// ---------------------------------------------------------------------------------------------
// Per-wave tile math
// ---------------------------------------------------------------------------------------------

// S^T (32 keys = tile rows kr0 .. kr0 + 31) x (this lane's query): D/16 MFMAs.
template <int D>
__device__ __forceinline__ f32x16 scores32(const lds_u8* tile, int kr0, const bf16x8 (&qf)[D / 16],
                                           f32x16 acc) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const u32x4 raw = lds_read16(tile + tile_off<D>(kr0 + c, 2 * kk + h));
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

// O^T[ds] += V^T P^T for one 32-key score block (tile rows kr0 .. kr0 + 31 of a V tile).
// Score register v of lane half h belongs to key 8*(v/4) + 4*h + v%4; the probabilities of
// registers 8*e2 .. 8*e2 + 7 form the B operand of one MFMA, whose A operand (V^T restricted to
// those 8 keys, this lane's d column) comes from two LDS transpose reads.  In each 16-lane group
// the source lane j points at key row (e = j/4 of the 4 keys) and 4 columns (j%4); the hardware
// hands lane i column i of each of the 4 rows.
template <int D>
__device__ __forceinline__ void pv32(const lds_u8* vtile, int kr0, const uint32_t* pk,
                                     f32x16 (&o)[D / 32]) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, j = lane & 15;
  const int h = grp >> 1, cg = grp & 1;
#pragma unroll
  for (int e2 = 0; e2 < 2; ++e2) {
    const bf16x8 b = p_operand(pk, e2);
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      const int d0 = 32 * ds + 16 * cg + 4 * (j & 3);
      s16x4 x[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = kr0 + 16 * e2 + 8 * r + 4 * h + (j >> 2);
        const lds_u8* p = vtile + tile_off<D>(row, d0 >> 3) + ((d0 >> 2) & 1) * 8;
        x[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(p));
      }
      u32x4 raw;
      raw[0] = __builtin_bit_cast(u32x2, x[0])[0];
      raw[1] = __builtin_bit_cast(u32x2, x[0])[1];
      raw[2] = __builtin_bit_cast(u32x2, x[1])[0];
      raw[3] = __builtin_bit_cast(u32x2, x[1])[1];
      o[ds] = mfma32(__builtin_bit_cast(bf16x8, raw), b, o[ds]);
    }
  }
}

// Vbar^T chunk tile: D rows (head dimension) x 32 blocks, 64-byte rows of four 16-byte chunks,
// chunk index XOR (row / 4) % 4 so that 16 consecutive rows read at one position are spread over
// the banks.  Copied from vbt [D][Mp] (block index contiguous).
template <int D>
__device__ __forceinline__ int vbt_off(int row, int ch) { return row * 64 + ((ch ^ ((row >> 2) & 3)) << 4); }

// Per-lane byte offsets of the Vbar^T chunk copy (relative to the chunk's first column): lane
// slot p of the tile holds row p / 4, logical chunk (p % 4) XOR the row's swizzle.
template <int D, int NT = kThreads>
struct VbtOffsets {
  static_assert(D * 4 % NT == 0, "tile must split into whole wave loads");
  uint32_t v[D * 4 / NT];
  __device__ __forceinline__ explicit VbtOffsets(int64_t Mp) {
#pragma unroll
    for (int i = 0; i < D * 4 / NT; ++i) {
      const int p = i * NT + (int)threadIdx.x;
      const int row = p >> 2;
      const int ch = (p & 3) ^ ((row >> 2) & 3);
      v[i] = (uint32_t)(((int64_t)row * Mp + ch * 8) * 2);
    }
  }
};

// The Vbar^T tile of chunk cb (blocks 32 cb .. 32 cb + 31) into LDS, with buffer loads issued from
// asm (see load_dense_rows for why).
template <int D, int NT = kThreads>
__device__ __forceinline__ void load_vbt_buf(const uint16_t* vt, int64_t Mp, int cb,
                                             const VbtOffsets<D, NT>& off, lds_u8* tile) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const i32x4_t rsrc = make_rsrc(vt + (int64_t)cb * 32, (uint32_t)(((D - 1) * Mp + 32) * 2));
#pragma unroll
  for (int i = 0; i < D * 4 / NT; ++i) dma16(rsrc, off.v[i], 0u, tile + (i * NT + wave * 64) * 16);
}

// O^T[ds] += Vbar^T P^T for the 32 pooled blocks of a chunk (probability registers as in pv32).
// The A operand for blocks {16 e2 + 4 h + 0..3} and {16 e2 + 8 + 4 h + 0..3} of this lane's d row
// is two 8-byte reads of the transposed tile.
template <int D>
__device__ __forceinline__ void pv_pooled(const lds_u8* vt, const uint32_t* pk, f32x16 (&o)[D / 32]) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
#pragma unroll
  for (int e2 = 0; e2 < 2; ++e2) {
    const bf16x8 b = p_operand(pk, e2);
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      const int row = 32 * ds + c;
      const u32x2 x0 = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(
          vt + vbt_off<D>(row, 2 * e2) + 8 * h);
      const u32x2 x1 = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(
          vt + vbt_off<D>(row, 2 * e2 + 1) + 8 * h);
      u32x4 raw;
      raw[0] = x0[0]; raw[1] = x0[1]; raw[2] = x1[0]; raw[3] = x1[1];
      o[ds] = mfma32(__builtin_bit_cast(bf16x8, raw), b, o[ds]);
    }
  }
}

// Key offset (within a 32-key score block) of result register v for lane half h.
__device__ __forceinline__ int key_of(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// The running max is only raised when a row's new scores exceed it by more than kSlack (log2
// units); otherwise probabilities up to 2^kSlack are accumulated against the old max.  With
// N <= 2^22 keys, sums stay below 2^54 times the largest |v|, far inside fp32 range, and bf16
// probabilities keep their relative precision.  Rescaling the accumulators is then rare, and is
// skipped by the whole wave when no lane needs it.
constexpr float kSlack = 32.0f;

// One 64-key stage (K and V tiles in LDS) folded into this lane's running softmax.
// active: this row takes part; nvalid: keys of the stage below N.
template <int D>
__device__ __forceinline__ void exact_stage(const lds_u8* ktile, const lds_u8* vtile,
                                            const bf16x8 (&qf)[D / 16], bool active, int nvalid,
                                            float sl2, float& mrun, float& lsum,
                                            f32x16 (&o)[D / 32]) {
  constexpr int NS = kStage / 32;
  const int h = (threadIdx.x & 63) >> 5;
  f32x16 s[NS];
#pragma unroll
  for (int kb = 0; kb < NS; ++kb) s[kb] = scores32<D>(ktile, 32 * kb, qf, f32x16{});

  const bool partial = nvalid < kStage;  // wave-uniform
  if (partial) {
#pragma unroll
    for (int kb = 0; kb < NS; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (32 * kb + key_of(v, h) >= nvalid) s[kb][v] = -INFINITY;
  }
  float mt = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NS; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) mt = fmaxf(mt, s[kb][v]);
  mt = pair_max(mt) * sl2;
  const bool grow = active && mt > mrun + kSlack;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float mnew = grow ? mt : mrun;
    const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
    mrun = mnew;
    lsum *= alpha;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[ds][v] *= alpha;
  }
  // rows that do not take part subtract +inf: every probability is 0
  const float moff = active ? -mrun : -INFINITY;
  uint32_t pk[NS][8];
  float ps = 0.f;
#pragma unroll
  for (int kb = 0; kb < NS; ++kb) {
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(fmaf(s[kb][v], sl2, moff));
    ps = round_p(p, pk[kb], ps);
  }
  lsum += ps;
#pragma unroll
  for (int kb = 0; kb < NS; ++kb) pv32<D>(vtile, 32 * kb, pk[kb], o);
}

// ---------------------------------------------------------------------------------------------
// Software-pipelined exact loop, in steps of 32 keys (half a 64-key stage).  A wave keeps two
// score blocks live: while the matrix cores compute S^T of the next 32 keys (phase A), the vector
// ALU turns the current 32 keys' scores into probabilities; while the matrix cores accumulate
// O^T += V^T P^T for the current 32 keys (phase B), the vector ALU takes the next block's row
// maximum.  K and V tiles are double buffered separately, each with its own barrier, so the next
// stage's keys can be in use while this stage's values still are.  Instruction groups are
// interleaved with sched_group_barrier so that every MFMA has independent vector work behind it.
// ---------------------------------------------------------------------------------------------
constexpr int kSgMfma = 0x008, kSgValu = 0x002 | 0x400, kSgDsRead = 0x100;

// Phase A: (QK) sn = S^T of the 32 keys at rows kr0.. of ktile, and the probabilities of the
// current block sc (offset moff = -running max, or -inf for rows that do not take part) packed
// into pk, with their rounded sum added to ps.
template <int D, bool QK>
__device__ __forceinline__ void phase_a(const lds_u8* ktile, int kr0, const bf16x8 (&qf)[D / 16],
                                        f32x16& sn, const f32x16& sc, float sl2, float moff,
                                        uint32_t (&pk)[8], float& ps) {
  constexpr int NM = D / 16;        // MFMAs
  constexpr int PER = 16 / NM;      // probabilities per MFMA slot (even)
  const int lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
  if constexpr (QK) sn = f32x16{};
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    if constexpr (QK) {
      const u32x4 raw = lds_read16(ktile + tile_off<D>(kr0 + c, 2 * i + h));
      sn = mfma32(__builtin_bit_cast(bf16x8, raw), qf[i], sn);
    }
#pragma unroll
    for (int u = 0; u < PER; u += 2) {
      const int v = i * PER + u;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[v], sl2, moff));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[v + 1], sl2, moff));
      pk[v / 2] = pack_bf16x2(p0, p1);
      ps = add_bf16x2(pk[v / 2], ps);
    }
  }
  if constexpr (QK) {
    // K operand reads run three MFMAs ahead
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 3, 0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + 3 < NM) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgValu, 3 * PER, 0);
    }
  }
}

// Phase B: O^T += V^T P^T for the 32 keys at rows vr0.. of vtile and, when MX, the maximum of the
// next block's scores sn (raw, before scaling).
template <int D, bool MX>
__device__ __forceinline__ float phase_b(const lds_u8* vtile, int vr0, const uint32_t (&pk)[8],
                                         const f32x16& sn, f32x16 (&o)[D / 32]) {
  constexpr int NM = 2 * (D / 32);  // MFMAs
  constexpr int PER = 16 / NM;      // maxima per MFMA slot
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, j = lane & 15;
  const int h = grp >> 1, cg = grp & 1;
  float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
  for (int e2 = 0; e2 < 2; ++e2) {
    const bf16x8 b = p_operand(pk, e2);
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      const int d0 = 32 * ds + 16 * cg + 4 * (j & 3);
      s16x4 x[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = vr0 + 16 * e2 + 8 * r + 4 * h + (j >> 2);
        const lds_u8* p = vtile + tile_off<D>(row, d0 >> 3) + ((d0 >> 2) & 1) * 8;
        x[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(p));
      }
      u32x4 raw;
      raw[0] = __builtin_bit_cast(u32x2, x[0])[0];
      raw[1] = __builtin_bit_cast(u32x2, x[0])[1];
      raw[2] = __builtin_bit_cast(u32x2, x[1])[0];
      raw[3] = __builtin_bit_cast(u32x2, x[1])[1];
      o[ds] = mfma32(__builtin_bit_cast(bf16x8, raw), b, o[ds]);
      if constexpr (MX) {
        const int step = e2 * (D / 32) + ds;
#pragma unroll
        for (int u = 0; u < PER; u += 2) {
          m0 = fmaxf(m0, sn[step * PER + u]);
          m1 = fmaxf(m1, sn[step * PER + u + 1]);
        }
      }
    }
  }
  __builtin_amdgcn_sched_group_barrier(kSgDsRead, 4, 0);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    if (i + 2 < NM) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    if constexpr (MX) __builtin_amdgcn_sched_group_barrier(kSgValu, PER, 0);
  }
  return fmaxf(m0, m1);
}

// Keys of a 32-key block at or beyond nvalid (counted from the block's first key) get -inf.
__device__ __forceinline__ void mask_tail(f32x16& s, int nvalid) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int v = 0; v < 16; ++v)
    if (key_of(v, h) >= nvalid) s[v] = -INFINITY;
}

// Raise the running max to the block maximum mt_raw (raw score units) when it exceeds it by more
// than kSlack, rescaling the accumulators; rows that do not take part never raise it.
template <int D>
__device__ __forceinline__ void raise_max(float mt_raw, bool active, float sl2, float& mrun,
                                          float& lsum, f32x16 (&o)[D / 32]) {
  const float mt = pair_max(mt_raw) * sl2;
  const bool grow = active && mt > mrun + kSlack;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float mnew = grow ? mt : mrun;
    const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
    mrun = mnew;
    lsum *= alpha;
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[ds][v] *= alpha;
  }
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

// Write O = O^T / l for the wave's 32 rows: through LDS (row-major, swizzled) so that each global
// store instruction writes whole rows.  stage: this wave's 32 x D bf16 LDS area.  Also the
// optional fp32 output and log-sum-exp.  Called by every lane of the wave.
template <int D>
__device__ __forceinline__ void epilogue(const f32x16 (&o)[D / 32], float mrun, float lsum,
                                         int64_t row0, int64_t N, uint16_t* __restrict__ out,
                                         int64_t on, float* __restrict__ out_f32,
                                         float* __restrict__ lse, lds_u8* stage) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 31, h = lane >> 5;
  const int64_t row = row0 + c;
  const float l = pair_sum(lsum);
  const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float x0 = o[ds][4 * g + 0] * inv, x1 = o[ds][4 * g + 1] * inv;
      const float x2 = o[ds][4 * g + 2] * inv, x3 = o[ds][4 * g + 3] * inv;
      u32x2 w;
      w[0] = pack_bf16x2(x0, x1);
      w[1] = pack_bf16x2(x2, x3);
      // d = 32 ds + 8 g + 4 h + (0..3): chunk 4 ds + g, half h
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
          stage + tile_off<D>(c, 4 * ds + g) + 8 * h) = w;
      if (out_f32 && row < N)
        *reinterpret_cast<f32x4*>(out_f32 + row * D + 32 * ds + 8 * g + 4 * h) = f32x4{x0, x1, x2, x3};
    }
  if (lse && h == 0 && row < N) lse[row] = l > 0.f ? (mrun + log2f(l)) * kLn2 : -INFINITY;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int kChunks = D / 8;
#pragma unroll
  for (int i = 0; i < 32 * kChunks / 64; ++i) {
    const int idx = i * 64 + lane;
    const int r = idx / kChunks, ch = idx % kChunks;
    const u32x4 v = lds_read16(stage + tile_off<D>(r, ch));
    if (row0 + r < N) *reinterpret_cast<u32x4*>(out + (row0 + r) * on + ch * 8) = v;
  }
}

// Work item of this workgroup, XCD-aware: workgroup i runs on XCD i % 8, so XCD x is given the
// contiguous range of (head, query tile) items x*P .. x*P + P - 1 and the tiles of one head that
// run at the same time share that XCD's L2.  Returns false for the padding workgroups.
__device__ __forceinline__ bool work_item(int64_t total, int64_t& w) {
  const int64_t per = (total + 7) / 8;
  w = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  return w < total;
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// Row statistics: mu, sigma, tau of every query's proxy row
// ---------------------------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(kRowStatsThreads) void rowstats_kernel(RowStatsArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  constexpr int64_t kGroupRows = (int64_t)kRowStatsRows * kRowStatsPasses;
  const int64_t groups = (a.N + kGroupRows - 1) / kGroupRows;
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
  for (int pp = 0; pp < kRowStatsPasses; ++pp) {
    const int64_t r0 = grp * kGroupRows + (int64_t)pp * kRowStatsRows;
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
  if (!work_item(a.BH * ntiles, w)) return;
  const int64_t bh = w / ntiles;
  const int64_t tile = w % ntiles;
  const int64_t row0 = tile * QT + wave * 16;  // first row of this wave
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
  if (a.tile_kept && wave == 0) {  // blocks kept by some row of the tile
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

// Half HB of stage n of the pipelined exact loop over consecutive stages (dense kernel); B = n & 1.
// NEXT: a next 32-key block exists (it may be partial).  sc holds the current block's scores,
// sn receives the next block's.  K tiles live at kbuf + b * tile, V tiles at vbuf + b * tile.
// Copies are issued K0, V0, K1 (prologue), then V_{n+1} at half 0 and K_{n+2} at half 1 of stage n.
template <int D, int B, int HB, bool NEXT, int NT>
__device__ __forceinline__ void dense_half(int n, int nst, int64_t N, const uint16_t* kb,
                                           const uint16_t* vb, int64_t rs, lds_u8* kbuf,
                                           lds_u8* vbuf, const TileOffsets<D, kStage, NT>& toff,
                                           const bf16x8 (&qf)[D / 16], float sl2,
                                           const f32x16& sc, f32x16& sn, float& mrun,
                                           float& lsum, f32x16 (&o)[D / 32]) {
  constexpr int kTileBytes = kStage * D * 2;
  constexpr int L = tile_loads<D, kStage, NT>();
  auto issue = [&](const uint16_t* src, int st, lds_u8* dst) {
    load_rows<D, kStage, NT>(src, (int64_t)st * kStage, N, rs, toff, dst);
  };
  const bool more = n + 1 < nst;
  if constexpr (HB == 0) {
    // V_n has landed (only K_{n+1}, issued after it, may be in flight); after the barrier every
    // wave is done with V_{n-1}, whose buffer takes V_{n+1}
    if (more) wait_vmcnt<L>();
    else wait_vmcnt<0>();
    bar();
    if (more) issue(vb, n + 1, vbuf + (B ^ 1) * kTileBytes);
  } else {
    // K_{n+1} has landed (only V_{n+1} may be in flight); after the barrier every wave is done
    // with K_n, whose buffer takes K_{n+2}
    if (more) wait_vmcnt<L>();
    bar();
    if (n + 2 < nst) issue(kb, n + 2, kbuf + B * kTileBytes);
  }
  uint32_t pk[8];
  float ps = 0.f;
  const lds_u8* knext = HB == 0 ? kbuf + B * kTileBytes : kbuf + (B ^ 1) * kTileBytes;
  phase_a<D, NEXT>(knext, HB == 0 ? 32 : 0, qf, sn, sc, sl2, -mrun, pk, ps);
  if constexpr (NEXT) {
    const int nv = (int)(N - (int64_t)n * kStage) - (HB == 0 ? 32 : 64);
    if (nv < 32) mask_tail(sn, nv);
  }
  lsum += ps;
  if constexpr (NEXT) {
    const float mt = phase_b<D, true>(vbuf + B * kTileBytes, 32 * HB, pk, sn, o);
    raise_max<D>(mt, true, sl2, mrun, lsum, o);
  } else {
    phase_b<D, false>(vbuf + B * kTileBytes, 32 * HB, pk, sn, o);
  }
}

// ---------------------------------------------------------------------------------------------
// Full proxy map (the prior-art routing's input): s_map[bh][i][j] = q_i . Kbar_j / sqrt(d) for
// every row and block, written to memory -- the round trip the fused kernel avoids.  The same
// fp32-accurate three-piece product as the fused kernel's routing sweep, one workgroup per
// 128-row tile, pooled-key chunks double buffered.  Row-major: a wave's 32 x 32 chunk of scores is
// transposed through LDS so that every store writes whole 128-byte row segments.
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 2) void proxy_map_kernel(const uint16_t* __restrict__ q,
                                                                Strides qs,
                                                                const uint16_t* __restrict__ kp,
                                                                int64_t BH, int64_t N, int64_t M,
                                                                int64_t Mp, float* __restrict__ smap) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  constexpr int kChunkTile = 32 * D * 2;
  constexpr int kBuf = 3 * kChunkTile;
  constexpr int kStageStride = 33;  // floats per staged row (33: conflict-free column writes)
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, c = lane & 31, h = lane >> 5;
  const int64_t ntiles = (N + kQTile - 1) / kQTile;
  int64_t w;
  if (!work_item(BH * ntiles, w)) return;
  const int64_t bh = w / ntiles;
  const int64_t tile = w % ntiles;
  const int64_t row = tile * kQTile + wave * 32 + c;
  const bool rvalid = row < N;
  bf16x8 qf[D / 16];
  load_q<D>(q + qs.base(bh) + row * qs.sn, rvalid, qf);
  const float inv_sqrt_d = 1.0f / sqrtf((float)D);
  const int64_t piece = BH * Mp * D;
  const uint16_t* kp0 = kp + bh * Mp * D;
  const int64_t row0 = tile * kQTile + wave * 32;
  float* stage = (float*)(smem_raw + 2 * kBuf) + wave * 32 * kStageStride;  // this wave's 32 x 32
  const int nchunks = (int)(Mp / 32);
  const TileOffsets<D, 32> coff(D);
  auto issue_chunk = [&](int cb, int b) {
    lds_u8* base = smem + b * kBuf;
    load_dense_rows<D, 32>(kp0 + 2 * piece, (int64_t)cb * 32, coff, base);
    load_dense_rows<D, 32>(kp0 + 1 * piece, (int64_t)cb * 32, coff, base + kChunkTile);
    load_dense_rows<D, 32>(kp0, (int64_t)cb * 32, coff, base + 2 * kChunkTile);
  };
  issue_chunk(0, 0);
  for (int cb = 0; cb < nchunks; ++cb) {
    const int b = cb & 1;
    wait_vmcnt<0>();
    bar();
    if (cb + 1 < nchunks) issue_chunk(cb + 1, b ^ 1);
    const lds_u8* base = smem + b * kBuf;
    f32x16 acc = {};
#pragma unroll
    for (int p = 0; p < 3; ++p) acc = scores32<D>(base + p * kChunkTile, 0, qf, acc);
    // stage[r][kj] = score of row r, block kj of the chunk; then each store instruction writes
    // two rows' 32 consecutive scores (lane l: block l % 32 of rows l / 32 + 2 i)
#pragma unroll
    for (int v = 0; v < 16; ++v) stage[c * kStageStride + key_of(v, h)] = acc[v] * inv_sqrt_d;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t j = (int64_t)cb * 32 + c;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = h + 2 * i;
      const int64_t grow = row0 + r;
      if (grow < N && j < M) smap[(bh * N + grow) * M + j] = stage[r * kStageStride + c];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ---------------------------------------------------------------------------------------------
// Dense reference kernel: the exact loop over every key, no routing.
// ---------------------------------------------------------------------------------------------

// WAVES waves of 32 rows per workgroup: 4 (two workgroups per CU) or 8 (one workgroup per CU,
// every K/V stage copied into LDS feeding 256 rows).
template <int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void dense_attn_kernel(const uint16_t* __restrict__ q,
                                                                 const uint16_t* __restrict__ k,
                                                                 const uint16_t* __restrict__ v,
                                                                 Strides in,
                                                                 uint16_t* __restrict__ out,
                                                                 Strides outs,
                                                                 float* __restrict__ lse,
                                                                 int64_t BH, int64_t N) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  constexpr int kTileBytes = kStage * D * 2;
  constexpr int NT = 64 * WAVES;
  constexpr int QT = 32 * WAVES;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, c = lane & 31;
  const int64_t ntiles = (N + QT - 1) / QT;
  int64_t w;
  if (!work_item(BH * ntiles, w)) return;
  const int64_t bh = w / ntiles;
  const int64_t tile = w % ntiles;
  const int64_t row0 = tile * QT + wave * 32;
  const int64_t row = row0 + c;
  const bool rvalid = row < N;
  const uint16_t* kb = k + in.base(bh);
  const uint16_t* vb = v + in.base(bh);
  const int64_t sn = in.sn;

  bf16x8 qf[D / 16];
  load_q<D>(q + in.base(bh) + row * sn, rvalid, qf);
  const float sl2 = kLog2e / sqrtf((float)D);
  f32x16 o[D / 32];
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) o[ds] = f32x16{};
  float mrun = -1e30f, lsum = 0.f;

  const int nst = (int)((N + kStage - 1) / kStage);
  const TileOffsets<D, kStage, NT> toff(sn);
  lds_u8* kbuf = smem;                        // K tiles: kbuf + b * kTileBytes
  lds_u8* vbuf = smem + 2 * kTileBytes;       // V tiles
  auto issue = [&](const uint16_t* src, int st, lds_u8* dst) {
    load_rows<D, kStage, NT>(src, (int64_t)st * kStage, N, sn, toff, dst);
  };

  // prologue: K0, V0, K1 in LDS; scores and max of the first 32 keys
  issue(kb, 0, kbuf);
  issue(vb, 0, vbuf);
  if (nst > 1) issue(kb, 1, kbuf + kTileBytes);
  wait_vmcnt<0>();
  bar();
  f32x16 sa = scores32<D>(kbuf, 0, qf, f32x16{}), sb;
  if (N < 32) mask_tail(sa, (int)N);
  {
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) m = fmaxf(m, sa[v]);
    mrun = pair_max(m) * sl2;
  }
  // stages n (buffers 0) and n + 1 (buffers 1) per iteration; the last stage's half 1 has no
  // next block
  int n = 0;
  for (; n + 2 < nst; n += 2) {
    dense_half<D, 0, 0, true, NT>(n, nst, N, kb, vb, sn, kbuf, vbuf, toff, qf, sl2, sa, sb, mrun, lsum, o);
    dense_half<D, 0, 1, true, NT>(n, nst, N, kb, vb, sn, kbuf, vbuf, toff, qf, sl2, sb, sa, mrun, lsum, o);
    dense_half<D, 1, 0, true, NT>(n + 1, nst, N, kb, vb, sn, kbuf, vbuf, toff, qf, sl2, sa, sb, mrun, lsum, o);
    dense_half<D, 1, 1, true, NT>(n + 1, nst, N, kb, vb, sn, kbuf, vbuf, toff, qf, sl2, sb, sa, mrun, lsum, o);
  }
  if (n + 1 < nst) {
    dense_half<D, 0, 0, true, NT>(n, nst, N, kb, vb, sn, kbuf, vbuf, toff, qf, sl2, sa, sb, mrun, lsum, o);
    dense_half<D, 0, 1, true, NT>(n, nst, N, kb, vb, sn, kbuf, vbuf, toff, qf, sl2, sb, sa, mrun, lsum, o);
    dense_half<D, 1, 0, true, NT>(n + 1, nst, N, kb, vb, sn, kbuf, vbuf, toff, qf, sl2, sa, sb, mrun, lsum, o);
    dense_half<D, 1, 1, false, NT>(n + 1, nst, N, kb, vb, sn, kbuf, vbuf, toff, qf, sl2, sb, sa, mrun, lsum, o);
  } else {
    dense_half<D, 0, 0, true, NT>(n, nst, N, kb, vb, sn, kbuf, vbuf, toff, qf, sl2, sa, sb, mrun, lsum, o);
    dense_half<D, 0, 1, false, NT>(n, nst, N, kb, vb, sn, kbuf, vbuf, toff, qf, sl2, sb, sa, mrun, lsum, o);
  }
  bar();  // stage buffers free for the epilogue
  epilogue<D>(o, mrun, lsum, row0, N, out + outs.base(bh), outs.sn, nullptr,
              lse ? lse + bh * N : nullptr,
              smem + wave * 32 * D * 2);
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

template <typename K>
static hipError_t set_smem(K kern, size_t bytes) {
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

static unsigned xcd_grid(int64_t total) { return (unsigned)(((total + 7) / 8) * 8); }

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

hipError_t launch_sparse(int d, const SparseArgs& a, hipStream_t stream) {
  if (d == 64 && a.block == 64) return launch_sparse_t<64, 64, 4>(a, stream);
  if (d == 64 && a.block == 128) return launch_sparse_t<64, 128, 4>(a, stream);
  if (d == 128 && a.block == 64) return launch_sparse16_t<128, 64>(a, stream);
  return launch_sparse16_t<128, 128>(a, stream);
}

template <int D>
static hipError_t launch_rowstats_t(const RowStatsArgs& a, hipStream_t stream) {
  const size_t smem = (size_t)3 * D * D * 2 + (size_t)(1 + kFactorTop) * D * sizeof(double);
  auto kern = rowstats_kernel<D>;
  hipError_t err = set_smem(kern, smem);
  if (err != hipSuccess) return err;
  constexpr int64_t kGroupRows = (int64_t)kRowStatsRows * kRowStatsPasses;
  const int64_t groups = (a.N + kGroupRows - 1) / kGroupRows;
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.BH * groups)), dim3(kRowStatsThreads), smem, stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_proxy_map_t(const uint16_t* q, const Strides& qs, const uint16_t* kp,
                                     int64_t BH, int64_t N, int64_t M, int64_t Mp, float* s_map,
                                     hipStream_t stream) {
  const size_t smem = (size_t)2 * 3 * 32 * D * 2 + (size_t)4 * 32 * 33 * sizeof(float);
  auto kern = proxy_map_kernel<D>;
  hipError_t err = set_smem(kern, smem);
  if (err != hipSuccess) return err;
  const int64_t ntiles = (N + kQTile - 1) / kQTile;
  hipLaunchKernelGGL(kern, dim3(xcd_grid(BH * ntiles)), dim3(kThreads), smem, stream, q, qs, kp, BH,
                     N, M, Mp, s_map);
  return hipGetLastError();
}

hipError_t launch_proxy_map(int d, const uint16_t* q, const Strides& qs, const uint16_t* kp,
                            int64_t BH, int64_t N, int64_t M, int64_t Mp, float* s_map,
                            hipStream_t stream) {
  return d == 64 ? launch_proxy_map_t<64>(q, qs, kp, BH, N, M, Mp, s_map, stream)
                 : launch_proxy_map_t<128>(q, qs, kp, BH, N, M, Mp, s_map, stream);
}

hipError_t launch_rowstats(int d, const RowStatsArgs& a, hipStream_t stream) {
  return d == 64 ? launch_rowstats_t<64>(a, stream) : launch_rowstats_t<128>(a, stream);
}

// Eight waves (256 rows, one workgroup per CU) at d = 128: each K/V stage feeds twice the rows,
// 2% faster at the Wan2.1-14B shape (109 vs 111 ms, interleaved); four waves (two workgroups per
// CU) at d = 64, where eight were 10% slower on LTX's smaller grid.
template <int D>
static hipError_t launch_dense_t(int64_t BH, int64_t N, const void* q, const void* k,
                                 const void* v, const Strides& in, void* out, const Strides& outs,
                                 float* lse, hipStream_t stream) {
  constexpr int kDenseWaves = D == 128 ? 8 : 4;
  const size_t smem = (size_t)4 * kStage * D * 2;
  auto kern = dense_attn_kernel<D, kDenseWaves>;
  hipError_t err = set_smem(kern, smem);
  if (err != hipSuccess) return err;
  const int64_t ntiles = (N + 32 * kDenseWaves - 1) / (32 * kDenseWaves);
  hipLaunchKernelGGL(kern, dim3(xcd_grid(BH * ntiles)), dim3(64 * kDenseWaves), smem, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, in,
                     (uint16_t*)out, outs, lse, BH, N);
  return hipGetLastError();
}

hipError_t launch_dense(int d, int64_t BH, int64_t N, const void* q, const void* k, const void* v,
                        const Strides& in, void* out, const Strides& outs, float* lse,
                        hipStream_t stream) {
  return d == 64 ? launch_dense_t<64>(BH, N, q, k, v, in, out, outs, lse, stream)
                 : launch_dense_t<128>(BH, N, q, k, v, in, out, outs, lse, stream);
}

}  // namespace solattn
