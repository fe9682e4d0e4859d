// tiles.hpp -- LDS tile copies, matrix-core tile math and the online-softmax pieces shared by
// the gfx950 attention kernels of libsolattn (fused, dense, row statistics, proxy map).
// Internal: every translation unit that includes it gets its own copies (anonymous namespace).
#pragma once

#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace solattn {

namespace {

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kStage = 64;  // keys per pipeline stage

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

// Instruction-group masks for sched_group_barrier: matrix instructions, LDS reads.
constexpr int kSgMfma = 0x008, kSgDsRead = 0x100;

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

// Work item of this workgroup with the items split between the two halves of the chip: XCDs
// 0-3 walk the first half of the items and XCDs 4-7 the second, each quad interleaving its items
// round by round (XCD x of the quad takes every fourth item).  A head's query tiles are then
// spread over four L2s instead of one, so two heads have their K/V in flight instead of eight,
// few enough for the memory-side cache to hold, and a K/V row one XCD of the quad fetched can be
// served from there to the other three.  Every item in 0 .. 8*ceil(total/8) - 1 is hit once;
// returns false for the padding workgroups.
__device__ __forceinline__ bool work_item_quad(int64_t total, int64_t& w) {
  const int64_t per = (total + 7) / 8;
  const int64_t x = blockIdx.x % 8;
  w = (x / 4) * 4 * per + (int64_t)(blockIdx.x / 8) * 4 + (x % 4);
  return w < total;
}

template <typename K>
hipError_t set_smem(K kern, size_t bytes) {
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

// Grid of `total` work items rounded up to whole rounds over the 8 XCDs (see work_item).
inline unsigned xcd_grid(int64_t total) { return (unsigned)(((total + 7) / 8) * 8); }

}  // namespace

}  // namespace solattn
