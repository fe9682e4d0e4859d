// pool.hip -- K/V mean pooling per key block (HBM-bound), and the mean pooled key per head.
//
// Pooled keys and values: Kbar_j = (1/n_j) sum_{t in block j} K_t, likewise Vbar_j.  The proxy
// score of the Sol-Attn page's routing paragraph is q . Kbar_j / sqrt(d), and Vbar_j is the value
// of block j's pooled token.
//
// One workgroup pools one key block of one (batch, head) for both K and V: 256 threads read the
// block's rows as 16-byte chunks (consecutive threads -> consecutive chunks of a row, so each
// load instruction covers whole rows), accumulate fp32 partial sums over a strided subset of rows,
// then combine the partials through LDS in a fixed order (deterministic).  Besides the fp32
// means it writes the layouts the attention kernel consumes:
//   kp   [3][BH][Mp][d] bf16: Kbar split into hi + mid + lo bf16 pieces whose sum is the fp32
//        value, so a bf16 matrix product over the three pieces reproduces fp32 proxies;
//   vbt  [BH][d][Mp] bf16: Vbar transposed (block index contiguous), the A operand of the
//        pooled tokens' P Vbar product;
// where Mp = M rounded up to a multiple of 32; padding blocks are written as zeros.
// Two small per-head kernels follow: the mean pooled key (fp32 and fp64) and the covariance
// matrix of the pooled keys as three bf16 pieces, from which the attention kernel gets every
// query's proxy standard deviation as a quadratic form.
#include "common.hpp"
#include "kernels.hpp"

namespace solattn {

template <int D>
__global__ __launch_bounds__(kThreads) void pool_kv_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t N, int block, int64_t M,
    int64_t Mp, float* __restrict__ kbar, float* __restrict__ vbar, uint16_t* __restrict__ kp,
    uint16_t* __restrict__ vbt) {
  constexpr int kChunks = D / 8;               // 16-byte chunks per row
  constexpr int kGroups = kThreads / kChunks;  // row groups
  __shared__ float part[2][kGroups][D];

  const int64_t j = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int t = threadIdx.x;
  const int cc = t % kChunks;
  const int rg = t / kChunks;

  if (j >= M) {  // padding block of the split layouts
    if (t < D) {
      if (kp) {
        for (int p = 0; p < 3; ++p) kp[((p * gridDim.y + bh) * Mp + j) * D + t] = 0;
      }
      if (vbt) vbt[(bh * D + t) * Mp + j] = 0;
    }
    return;
  }

  const int64_t lo = j * (int64_t)block;
  const int64_t hi = (lo + block < N) ? lo + block : N;
  const uint16_t* kb = k + bh * N * D;
  const uint16_t* vb = v + bh * N * D;

  float sk[8], sv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sk[e] = sv[e] = 0.f;
  for (int64_t r = lo + rg; r < hi; r += kGroups) {
    u32x4 a = *reinterpret_cast<const u32x4*>(kb + r * D + cc * 8);
    u32x4 b = *reinterpret_cast<const u32x4*>(vb + r * D + cc * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sk[2 * e] += bf16_lo(a[e]);
      sk[2 * e + 1] += bf16_hi(a[e]);
      sv[2 * e] += bf16_lo(b[e]);
      sv[2 * e + 1] += bf16_hi(b[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    part[0][rg][cc * 8 + e] = sk[e];
    part[1][rg][cc * 8 + e] = sv[e];
  }
  __syncthreads();

  if (t < 2 * D) {
    const int which = t / D;  // 0: K, 1: V
    const int c = t % D;
    float s = 0.f;
    for (int g = 0; g < kGroups; ++g) s += part[which][g][c];
    const float mean = s / (float)(hi - lo);
    if (which == 0) {
      if (kbar) kbar[(bh * M + j) * D + c] = mean;
      if (kp) {
        const uint16_t h16 = f32_to_bf16_rne(mean);
        const float r1 = mean - bits_f32((uint32_t)h16 << 16);
        const uint16_t m16 = f32_to_bf16_rne(r1);
        const float r2 = r1 - bits_f32((uint32_t)m16 << 16);
        const uint16_t l16 = f32_to_bf16_rne(r2);
        const int64_t BH = gridDim.y;
        kp[((0 * BH + bh) * Mp + j) * D + c] = h16;
        kp[((1 * BH + bh) * Mp + j) * D + c] = m16;
        kp[((2 * BH + bh) * Mp + j) * D + c] = l16;
      }
    } else {
      if (vbar) vbar[(bh * M + j) * D + c] = mean;
      if (vbt) vbt[(bh * D + c) * Mp + j] = f32_to_bf16_rne(mean);
    }
  }
}

// Mean of the pooled keys of each head, accumulated in fp64: kglob[bh][c] = (1/M) sum_j Kbar_j[c].
// The mean proxy score of a query is then q . kglob / sqrt(d) (the mean is linear).
template <int D>
__global__ __launch_bounds__(kThreads) void kglob_kernel(const float* __restrict__ kbar, int64_t M,
                                                         float* __restrict__ kglob,
                                                         double* __restrict__ kglob64) {
  constexpr int kGroups = kThreads / D;
  __shared__ double part[kGroups][D];
  const int64_t bh = blockIdx.x;
  const int t = threadIdx.x;
  const int c = t % D;
  const int g = t / D;
  double s = 0.0;
  for (int64_t j = g; j < M; j += kGroups) s += (double)kbar[(bh * M + j) * D + c];
  part[g][c] = s;
  __syncthreads();
  if (t < D) {
    double tot = 0.0;
    for (int q = 0; q < kGroups; ++q) tot += part[q][t];
    kglob[bh * D + t] = (float)(tot / (double)M);
    kglob64[bh * D + t] = tot / (double)M;
  }
}

// Covariance of the pooled keys of each head, in fp64:
//   C[a][b] = (1/M) sum_j (Kbar_j[a] - g[a]) (Kbar_j[b] - g[b]),  g = mean_j Kbar_j.
// For the proxy row s_ij = q_i . Kbar_j / sqrt(d), the population variance over j is exactly
// q_i^T C q_i / d.  C is rounded to fp32 and written as hi + mid + lo bf16 pieces
// cp [3][BH][D][D] (their sum is the fp32 value), so a bf16 matrix product with fp32
// accumulation evaluates C q to fp32 accuracy.  One workgroup computes 8 rows of C.
template <int D>
__global__ __launch_bounds__(kThreads) void kcov_kernel(const float* __restrict__ kbar, int64_t M,
                                                        const double* __restrict__ kglob64,
                                                        uint16_t* __restrict__ cp) {
  constexpr int kRows = 8;
  constexpr int kPer = kRows * D / kThreads;  // entries per thread
  const int64_t bh = blockIdx.x;
  const int a0 = blockIdx.y * kRows;
  const int t = threadIdx.x;
  const float* kb = kbar + bh * M * D;
  const double* g = kglob64 + bh * D;
  double acc[kPer];
  int ra[kPer], cb[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int idx = e * kThreads + t;
    ra[e] = a0 + idx / D;
    cb[e] = idx % D;
    acc[e] = 0.0;
  }
  for (int64_t j = 0; j < M; ++j) {
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      acc[e] += ((double)kb[j * D + ra[e]] - g[ra[e]]) * ((double)kb[j * D + cb[e]] - g[cb[e]]);
  }
  const int64_t BH = gridDim.x;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const float c = (float)(acc[e] / (double)M);
    const uint16_t h16 = f32_to_bf16_rne(c);
    const float r1 = c - bits_f32((uint32_t)h16 << 16);
    const uint16_t m16 = f32_to_bf16_rne(r1);
    const uint16_t l16 = f32_to_bf16_rne(r1 - bits_f32((uint32_t)m16 << 16));
    const int64_t off = (bh * D + ra[e]) * D + cb[e];
    cp[0 * BH * D * D + off] = h16;
    cp[1 * BH * D * D + off] = m16;
    cp[2 * BH * D * D + off] = l16;
  }
}

hipError_t launch_pool(int d, int64_t BH, int64_t N, int block, const void* k, const void* v,
                       float* kbar, float* vbar, uint16_t* kp, uint16_t* vbt, int64_t Mp,
                       hipStream_t stream) {
  const int64_t M = (N + block - 1) / block;
  const int64_t gx = (kp || vbt) ? Mp : M;
  dim3 grid((unsigned)gx, (unsigned)BH);
  if (d == 64)
    hipLaunchKernelGGL(pool_kv_kernel<64>, grid, dim3(kThreads), 0, stream,
                       (const uint16_t*)k, (const uint16_t*)v, N, block, M, Mp, kbar, vbar, kp, vbt);
  else
    hipLaunchKernelGGL(pool_kv_kernel<128>, grid, dim3(kThreads), 0, stream,
                       (const uint16_t*)k, (const uint16_t*)v, N, block, M, Mp, kbar, vbar, kp, vbt);
  return hipGetLastError();
}

hipError_t launch_kstats(int d, int64_t BH, int64_t M, const float* kbar, float* kglob,
                         double* kglob64, uint16_t* cp, hipStream_t stream) {
  if (d == 64) {
    hipLaunchKernelGGL(kglob_kernel<64>, dim3((unsigned)BH), dim3(kThreads), 0, stream, kbar, M,
                       kglob, kglob64);
    hipLaunchKernelGGL(kcov_kernel<64>, dim3((unsigned)BH, 64 / 8), dim3(kThreads), 0, stream, kbar,
                       M, kglob64, cp);
  } else {
    hipLaunchKernelGGL(kglob_kernel<128>, dim3((unsigned)BH), dim3(kThreads), 0, stream, kbar, M,
                       kglob, kglob64);
    hipLaunchKernelGGL(kcov_kernel<128>, dim3((unsigned)BH, 128 / 8), dim3(kThreads), 0, stream,
                       kbar, M, kglob64, cp);
  }
  return hipGetLastError();
}

}  // namespace solattn
