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
// One lane per query row, 64 rows per workgroup, reading the block-major map [BH][M][N] (each
// load instruction reads 64 consecutive rows of one block).  The k-th largest score / the
// probability-p point is found by radix selection on an order-preserving 32-bit key of the
// ordering value: four passes of 8 bits, each summing counts (top-k) or probabilities (top-p) of
// the row's values under the current prefix into the lane's own 256-bin LDS histogram
// (bins x lanes, so lanes never share a bank).  A last pass keeps every value above the selected
// key and, among values equal to it, the lowest indices while the mass before them is below the
// target.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace solattn {

namespace {

constexpr int kRouteRows = 64;
constexpr int kBins = 256;

// Order-preserving key of a float (larger float -> larger key; -0 taken as +0).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = f32_bits(x == 0.f ? 0.f : x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int MODE>
__global__ __launch_bounds__(kRouteRows) void route_select_kernel(const float* __restrict__ smap,
                                                                  int64_t BH, int64_t N, int64_t M,
                                                                  int block, int64_t kk, float p,
                                                                  uint32_t* __restrict__ mask) {
  extern __shared__ __attribute__((aligned(16))) float hist[];  // [kBins][kRouteRows]
  const int lane = threadIdx.x;
  const int64_t groups = (N + kRouteRows - 1) / kRouteRows;
  const int64_t bh = blockIdx.x / groups;
  const int64_t row = (blockIdx.x % groups) * kRouteRows + lane;
  const bool valid = row < N;
  const float* col = smap + bh * M * N + (valid ? row : 0);
  const int64_t W = (M + 31) / 32;
  uint32_t* mrow = mask + (bh * N + (valid ? row : 0)) * W;
  const int n_last = (int)(N - (M - 1) * (int64_t)block);
  const float ln_full = logf((float)block), ln_last = logf((float)n_last);

  // the ordering value of block j: s_ij (top-k) or the pooled logit s_ij + ln n_j (top-p)
  auto value = [&](int64_t j) -> float {
    float x = col[j * N];
    if (MODE == 1) x += (j == M - 1) ? ln_last : ln_full;
    return x;
  };

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
      mx = -INFINITY;
      for (int64_t j = 0; j < M; ++j) mx = fmaxf(mx, value(j));
      float z = 0.f;
      for (int64_t j = 0; j < M; ++j) z += expf(value(j) - mx);
      target = p * z;
    }
  }
  auto weight = [&](float x) -> float { return MODE == 0 ? 1.f : expf(x - mx); };

  uint32_t prefix = 0u, pmask = 0u;
  float above = 0.f;  // mass of the values strictly above the current key range
  if (!none && !all) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int b = 0; b < kBins; ++b) hist[b * kRouteRows + lane] = 0.f;
      for (int64_t j = 0; j < M; ++j) {
        const float x = value(j);
        const uint32_t key = order_key(x);
        if ((key & pmask) == prefix) atomicAdd(&hist[((key >> shift) & 255u) * kRouteRows + lane], weight(x));
      }
      // the highest bin at which the mass from the top reaches the target; if rounding leaves it
      // short, the lowest non-empty bin (every value of the range is then kept)
      int pick = -1;
      float acc = above, acc_pick = above;
      for (int b = kBins - 1; b >= 0; --b) {
        const float hb = hist[b * kRouteRows + lane];
        if (hb > 0.f) {
          pick = b;
          acc_pick = acc;
          if (acc + hb >= target) break;
          acc += hb;
        }
      }
      if (pick < 0) pick = 0;
      above = acc_pick;
      prefix |= (uint32_t)pick << shift;
      pmask |= 255u << shift;
    }
  }

  // marking pass: above the selected key -> kept; equal -> kept in index order while the mass
  // before them is below the target
  float cum = above;
  uint32_t word = 0u;
  for (int64_t j = 0; j < M; ++j) {
    bool keep = all;
    if (!all && !none) {
      const float x = value(j);
      const uint32_t key = order_key(x);
      if (key > prefix) {
        keep = true;
      } else if (key == prefix) {
        keep = cum < target;
        cum += weight(x);
      }
    }
    word |= (keep ? 1u : 0u) << (j & 31);
    if ((j & 31) == 31 || j == M - 1) {
      if (valid) mrow[j >> 5] = word;
      word = 0u;
    }
  }
}

template <int MODE>
hipError_t launch_route_t(const float* s_map, int64_t BH, int64_t N, int64_t M, int block,
                          int64_t kk, float p, uint32_t* mask, hipStream_t stream) {
  const size_t smem = (size_t)kBins * kRouteRows * sizeof(float);
  auto kern = route_select_kernel<MODE>;
  hipError_t err = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  const int64_t groups = (N + kRouteRows - 1) / kRouteRows;
  hipLaunchKernelGGL(kern, dim3((unsigned)(BH * groups)), dim3(kRouteRows), smem, stream, s_map,
                     BH, N, M, block, kk, p, mask);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_select(int mode, const float* s_map, int64_t BH, int64_t N, int64_t M,
                               int block, int64_t k, float p, uint32_t* mask, hipStream_t stream) {
  return mode == 0 ? launch_route_t<0>(s_map, BH, N, M, block, k, p, mask, stream)
                   : launch_route_t<1>(s_map, BH, N, M, block, k, p, mask, stream);
}

}  // namespace solattn
