// route.hip -- prior-art routing for comparison: top-k and top-p block selection from a fully
// materialised proxy map (gfx950).
//
// The page "Sol-Attn: Accelerating Video Generation Inference via On-the-Fly Attention
// Sparsification" (agihunt.info/papers/2607.24027), paragraph on routing, describes the two
// routings Sol-Attn replaces: top-k keeps a fixed number of key blocks per query, top-p keeps
// blocks until their cumulative probability reaches a threshold, and both need the whole proxy
// map in memory first.  Definitions used here (the same proxy as the fused kernel):
//   top-k: the k blocks with the largest s_ij; equal scores keep the lower block index first.
//   top-p: pi_j = softmax over the row of the pooled logits s_ij + ln n_j; blocks are taken in
//          decreasing order of pi (equal values: lower index first) and a block is kept while the
//          probability of the blocks before it is below p.
//
// One wave per query row.  The row's M scores (row-major map) are read once, coalesced, into
// registers (block j in lane j % 64, slot j / 64; M <= 2048).  Both rules keep a prefix of
// the decreasing order, so the last kept value is found by a 32-step bitwise search over an
// order-preserving 32-bit key: the largest x with mass(key > x) >= target, where the mass counts
// blocks (top-k, target k) or probabilities (top-p, target p * sum), summed per lane and across the
// wave by a fixed butterfly.  The kept set is then every key above x + 1 and, among keys equal to
// it, the lowest indices while the mass before them is below the target.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace solattn {

namespace {

constexpr int kMaxSlots = 32;        // scores per lane: M <= 2048
constexpr int kRowsPerGroup = 4;     // rows (waves) per workgroup

// Order-preserving key of a float (larger float -> larger key; -0 taken as +0).  Every finite or
// infinite float maps above 0.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = f32_bits(x == 0.f ? 0.f : x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// kSlots: scores per lane (the launch picks the smallest multiple of 4 with 64 * kSlots >= M)
template <int MODE, int kSlots>
__global__ __launch_bounds__(64 * kRowsPerGroup) void route_select_kernel(
    const float* __restrict__ smap, int64_t BH, int64_t N, int64_t M, int block, int64_t kk,
    float p, uint32_t* __restrict__ mask) {
  const int lane = threadIdx.x & 63;
  const int64_t grow = (int64_t)blockIdx.x * kRowsPerGroup + (threadIdx.x >> 6);  // bh * N + row
  if (grow >= BH * N) return;  // whole wave
  const float* srow = smap + grow * M;
  const int64_t W = (M + 31) / 32;
  uint32_t* mrow = mask + grow * W;
  const int n_last = (int)(N - (M - 1) * (int64_t)block);
  const float ln_full = logf((float)block), ln_last = logf((float)n_last);

  float u[kSlots];
  uint32_t key[kSlots];
#pragma unroll
  for (int r = 0; r < kSlots; ++r) {
    const int64_t j = (int64_t)r * 64 + lane;
    float x = -INFINITY;
    if (j < M) {
      x = srow[j];
      if (MODE == 1) x += (j == M - 1) ? ln_last : ln_full;
    }
    u[r] = x;
    key[r] = j < M ? order_key(x) : 0u;  // padding slots: key 0, below every real key
  }

  bool all = false, none = false;
  float target = 0.f, mx = 0.f;
  if (MODE == 0) {
    none = kk <= 0;
    all = kk >= M;
    target = (float)kk;
  } else {
    none = !(p > 0.f);
    all = p >= 1.f;
    if (!none && !all) {
      float m = -INFINITY;
#pragma unroll
      for (int r = 0; r < kSlots; ++r) m = fmaxf(m, u[r]);
      mx = wave_max(m);
      float z = 0.f;
#pragma unroll
      for (int r = 0; r < kSlots; ++r) z += key[r] ? expf(u[r] - mx) : 0.f;
      target = p * wave_sum(z);
    }
  }
  float w[kSlots];
#pragma unroll
  for (int r = 0; r < kSlots; ++r) w[r] = key[r] == 0u ? 0.f : (MODE == 0 ? 1.f : expf(u[r] - mx));

  uint32_t t = 0u;       // key of the last kept value
  float above = 0.f;     // mass of the keys above t
  if (!all && !none) {
    uint32_t x = 0u;     // largest x with mass(key > x) >= target (x = 0 qualifies)
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = x | (1u << b);
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < kSlots; ++r) m += key[r] > cand ? w[r] : 0.f;
      if (wave_sum(m) >= target) x = cand;
    }
    t = x + 1u;
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < kSlots; ++r) m += key[r] > t ? w[r] : 0.f;
    above = wave_sum(m);
  }

  // keep: above t; equal to t in index order while the mass before is below the target
  float cum = above;
#pragma unroll
  for (int r = 0; r < kSlots; ++r) {
    if ((int64_t)r * 64 >= M) break;
    bool keep = all && (int64_t)r * 64 + lane < M;
    if (!all && !none) {
      keep = key[r] > t;
      uint64_t ties = __builtin_amdgcn_ballot_w64(key[r] == t);
      while (ties) {  // wave-uniform loop over the equal keys of this slot, lowest lane first
        const int l = __builtin_ctzll(ties);
        ties &= ties - 1;
        const float wl = __shfl(w[r], l, 64);
        if (lane == l) keep = cum < target;
        cum += wl;
      }
    }
    const uint64_t bits = __builtin_amdgcn_ballot_w64(keep);
    const int64_t w0 = (int64_t)r * 2;
    if (lane == 0 && w0 < W) mrow[w0] = (uint32_t)bits;
    if (lane == 1 && w0 + 1 < W) mrow[w0 + 1] = (uint32_t)(bits >> 32);
  }
}

template <int MODE, int kSlots>
hipError_t launch_route_r(const float* s_map, int64_t BH, int64_t N, int64_t M, int block,
                          int64_t kk, float p, uint32_t* mask, hipStream_t stream) {
  const int64_t groups = (BH * N + kRowsPerGroup - 1) / kRowsPerGroup;
  hipLaunchKernelGGL((route_select_kernel<MODE, kSlots>), dim3((unsigned)groups),
                     dim3(64 * kRowsPerGroup), 0, stream, s_map, BH, N, M, block, kk, p, mask);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_route_t(const float* s_map, int64_t BH, int64_t N, int64_t M, int block,
                          int64_t kk, float p, uint32_t* mask, hipStream_t stream) {
  const int slots = (int)((M + 63) / 64);
  switch ((slots + 3) / 4) {
    case 1: return launch_route_r<MODE, 4>(s_map, BH, N, M, block, kk, p, mask, stream);
    case 2: return launch_route_r<MODE, 8>(s_map, BH, N, M, block, kk, p, mask, stream);
    case 3: return launch_route_r<MODE, 12>(s_map, BH, N, M, block, kk, p, mask, stream);
    case 4: return launch_route_r<MODE, 16>(s_map, BH, N, M, block, kk, p, mask, stream);
    case 5: return launch_route_r<MODE, 20>(s_map, BH, N, M, block, kk, p, mask, stream);
    case 6: return launch_route_r<MODE, 24>(s_map, BH, N, M, block, kk, p, mask, stream);
    case 7: return launch_route_r<MODE, 28>(s_map, BH, N, M, block, kk, p, mask, stream);
    default: return launch_route_r<MODE, 32>(s_map, BH, N, M, block, kk, p, mask, stream);
  }
}

}  // namespace

int64_t route_max_blocks() { return 64 * kMaxSlots; }

hipError_t launch_route_select(int mode, const float* s_map, int64_t BH, int64_t N, int64_t M,
                               int block, int64_t k, float p, uint32_t* mask, hipStream_t stream) {
  return mode == 0 ? launch_route_t<0>(s_map, BH, N, M, block, k, p, mask, stream)
                   : launch_route_t<1>(s_map, BH, N, M, block, k, p, mask, stream);
}

}  // namespace solattn
