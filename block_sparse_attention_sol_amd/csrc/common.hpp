// common.hpp -- shared device helpers for the gfx950 kernels of libsolattn.
//
// Matrix-core conventions (CDNA4 v_mfma_f32_32x32x16_bf16, one wave of 64 lanes):
//   lane l = 32*h + c  (h = l >> 5 is the lane half, c = l & 31).
//   A operand (32 x 16): lane l holds 8 bf16 of row c; B operand (16 x 32): 8 bf16 of column c.
//   Both operands use the same (half, slot) -> k assignment, so any consistent choice of which 8 of
//   the 16 k indices a half holds gives the same product; the kernels pick the k indices per half
//   to suit their data (contiguous head-dim chunks for Q.K, and the score layout for P.V).
//   Result (32 x 32, 16 fp32 per lane): lane l holds column c, rows 8*(v/4) + 4*h + (v%4), v=0..15.
// The attention kernels compute S^T = K Q^T so that one lane owns one query (column): the
// softmax row statistics are then lane-local plus one exchange with the other lane half.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace solattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kQTile = 128;           // query rows per workgroup tile
constexpr int kWaves = 4;             // waves per workgroup; each wave owns 32 query rows
constexpr int kThreads = kWave * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16: lane l = 16*g + q (g = l >> 4 the lane row, q = l & 15).
//   A operand (16 x 32): lane l holds A[q][8g .. 8g + 7]; B operand (32 x 16): B[8g .. 8g + 7][q].
//   Result (16 x 16, 4 fp32 per lane): lane l holds D[4g + i][q], i = 0..3.
// As with the 32x32 form, A and B only have to agree on which k indices lane row g holds.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 <-> fp32 bit helpers (round to nearest even; inputs here are finite).
__device__ __forceinline__ uint32_t f32_bits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bits_f32(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return bits_f32(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return bits_f32(packed & 0xffff0000u); }
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = f32_bits(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// acc + lo + hi of a packed bf16 pair, in fp32 (one v_dot2_f32_bf16 against (1, 1)): sums
// exactly the rounded values that enter the matrix product.
__device__ __forceinline__ float add_bf16x2(uint32_t packed, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
}

// Element strides of a [B][H][N][d] bf16 view whose d elements are contiguous: the start of row
// n of head (b, h) is b * sb + h * sh + n * sn.  The kernels take the combined index bh = b*H + h.
struct Strides {
  int64_t H, sb, sh, sn;
  __host__ __device__ int64_t base(int64_t bh) const { return (bh / H) * sb + (bh % H) * sh; }
  static Strides contiguous(int64_t H, int64_t N, int64_t d) { return Strides{H, H * N * d, N * d, d}; }
};

// Lane-pair combines across the two halves of the wave (lane l with lane l ^ 32), with the
// gfx950 v_permlane32_swap (a VALU op, no LDS round trip).  Swapping a register with itself
// leaves lanes 0-31 of the first result and lanes 32-63 of the second holding x, the other
// halves holding the partner's x, so any symmetric combine of the two results is the pair value.
__device__ __forceinline__ void pair_values(uint32_t x, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ float pair_max(float x) {
  uint32_t a, b;
  pair_values(__builtin_bit_cast(uint32_t, x), a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float pair_sum(float x) {
  uint32_t a, b;
  pair_values(__builtin_bit_cast(uint32_t, x), a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ uint32_t pair_or(uint32_t x) {
  uint32_t a, b;
  pair_values(x, a, b);
  return a | b;
}

// Combines over the four 16-lane rows holding one column of a 16x16 result (lanes q, q + 16,
// q + 32, q + 48): v_permlane16_swap pairs lane l with l ^ 16 the way permlane32_swap pairs l with
// l ^ 32, so two swaps give the four-way value in every lane.
__device__ __forceinline__ void row_pair_values(uint32_t x, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ float quad_max(float x) {
  uint32_t a, b;
  row_pair_values(__builtin_bit_cast(uint32_t, x), a, b);
  return pair_max(fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)));
}
__device__ __forceinline__ float quad_sum(float x) {
  uint32_t a, b;
  row_pair_values(__builtin_bit_cast(uint32_t, x), a, b);
  return pair_sum(__builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
}
__device__ __forceinline__ uint32_t quad_or(uint32_t x) {
  uint32_t a, b;
  row_pair_values(x, a, b);
  return pair_or(a | b);
}
// OR over the 16 lanes of each 16-lane row, every lane of the row receiving the value (DPP moves:
// swap neighbours, swap neighbour pairs, mirror within 8 lanes, mirror within 16; all lanes active).
__device__ __forceinline__ uint32_t row16_or(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false);  // row_mirror
  return x;
}

}  // namespace solattn
