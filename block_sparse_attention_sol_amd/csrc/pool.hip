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
// A small per-head kernel follows: the mean pooled key (fp32 and fp64) and the covariance matrix
// of the pooled keys as three bf16 pieces, from which every query's proxy standard deviation is a
// quadratic form.
#include "common.hpp"
#include "kernels.hpp"

namespace solattn {

template <int D>
__global__ __launch_bounds__(kThreads) void pool_kv_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, Strides kv, int64_t N, int block,
    int64_t M, int64_t Mp, float* __restrict__ kbar, float* __restrict__ vbar,
    uint16_t* __restrict__ kp, uint16_t* __restrict__ vbt) {
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
  const uint16_t* kb = k + kv.base(bh);
  const uint16_t* vb = v + kv.base(bh);

  float sk[8], sv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sk[e] = sv[e] = 0.f;
  for (int64_t r = lo + rg; r < hi; r += kGroups) {
    u32x4 a = *reinterpret_cast<const u32x4*>(kb + r * kv.sn + cc * 8);
    u32x4 b = *reinterpret_cast<const u32x4*>(vb + r * kv.sn + cc * 8);
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

// Mean and covariance of the pooled keys of each head, in fp64:
//   g[a] = (1/M) sum_j Kbar_j[a],   C[a][b] = (1/M) sum_j Kbar_j[a] Kbar_j[b] - g[a] g[b].
// The mean proxy score of a query is q . g / sqrt(d) (the mean is linear), and for the proxy row
// s_ij = q_i . Kbar_j / sqrt(d) the population variance over j is exactly q_i^T C q_i / d.  C is
// rounded to fp32 and written as hi + mid + lo bf16 pieces cp [3][BH][D][D] (their sum is the fp32
// value), so a bf16 matrix product with fp32 accumulation evaluates C q to fp32 accuracy.
// One workgroup computes a 32 x 32 tile of C: pooled keys are staged through LDS in chunks of 64
// blocks, each thread accumulates a 2 x 2 block of products and the two column sums.  The diagonal
// tiles (ai == bi) also write g (fp32 and fp64).
template <int D>
__global__ __launch_bounds__(kThreads) void kstats_kernel(const float* __restrict__ kbar, int64_t M,
                                                          float* __restrict__ kglob,
                                                          double* __restrict__ kglob64,
                                                          uint16_t* __restrict__ cp) {
  constexpr int kT = D / 32;  // tiles per dimension
  constexpr int kChunk = 64;
  __shared__ double sa[kChunk][32];
  __shared__ double sb[kChunk][32];
  const int64_t bh = blockIdx.x / (kT * kT);
  const int ai = (int)(blockIdx.x % (kT * kT)) / kT;
  const int bi = (int)(blockIdx.x % (kT * kT)) % kT;
  const int t = threadIdx.x;
  const int ta = t / 16, tb = t % 16;  // rows 2 ta + {0,1}, columns 2 tb + {0,1} of the tile
  const float* kb = kbar + bh * M * D;
  double c00 = 0.0, c01 = 0.0, c10 = 0.0, c11 = 0.0;
  double s1a = 0.0, s1b = 0.0;  // column sums (threads t < 32: a column t, b column t)
  for (int64_t j0 = 0; j0 < M; j0 += kChunk) {
    const int n = (int)((M - j0) < kChunk ? (M - j0) : kChunk);
    __syncthreads();
    for (int idx = t; idx < kChunk * 32; idx += kThreads) {
      const int r = idx / 32, col = idx % 32;
      sa[r][col] = r < n ? (double)kb[(j0 + r) * D + 32 * ai + col] : 0.0;
      sb[r][col] = r < n ? (double)kb[(j0 + r) * D + 32 * bi + col] : 0.0;
    }
    __syncthreads();
    for (int r = 0; r < n; ++r) {
      const double a0 = sa[r][2 * ta], a1 = sa[r][2 * ta + 1];
      const double b0 = sb[r][2 * tb], b1 = sb[r][2 * tb + 1];
      c00 = fma(a0, b0, c00);
      c01 = fma(a0, b1, c01);
      c10 = fma(a1, b0, c10);
      c11 = fma(a1, b1, c11);
    }
    if (t < 32) {
      for (int r = 0; r < n; ++r) {
        s1a += sa[r][t];
        s1b += sb[r][t];
      }
    }
  }
  __shared__ double ga[32], gb[32];
  if (t < 32) {
    ga[t] = s1a / (double)M;
    gb[t] = s1b / (double)M;
    if (ai == bi) {
      kglob[bh * D + 32 * ai + t] = (float)(s1a / (double)M);
      kglob64[bh * D + 32 * ai + t] = s1a / (double)M;
    }
  }
  __syncthreads();
  const int64_t BH = gridDim.x / (kT * kT);
  const double inv_m = 1.0 / (double)M;
  const double cv[2][2] = {{c00, c01}, {c10, c11}};
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int ra = 2 * ta + x, rb = 2 * tb + y;
      const float c = (float)(cv[x][y] * inv_m - ga[ra] * gb[rb]);
      const uint16_t h16 = f32_to_bf16_rne(c);
      const float r1 = c - bits_f32((uint32_t)h16 << 16);
      const uint16_t m16 = f32_to_bf16_rne(r1);
      const uint16_t l16 = f32_to_bf16_rne(r1 - bits_f32((uint32_t)m16 << 16));
      const int64_t off = (bh * D + 32 * ai + ra) * D + 32 * bi + rb;
      cp[0 * BH * D * D + off] = h16;
      cp[1 * BH * D * D + off] = m16;
      cp[2 * BH * D * D + off] = l16;
    }
}

hipError_t launch_pool(int d, int64_t BH, int64_t N, int block, const void* k, const void* v,
                       const Strides& kv,
                       float* kbar, float* vbar, uint16_t* kp, uint16_t* vbt, int64_t Mp,
                       hipStream_t stream) {
  const int64_t M = (N + block - 1) / block;
  const int64_t gx = (kp || vbt) ? Mp : M;
  dim3 grid((unsigned)gx, (unsigned)BH);
  if (d == 64)
    hipLaunchKernelGGL(pool_kv_kernel<64>, grid, dim3(kThreads), 0, stream,
                       (const uint16_t*)k, (const uint16_t*)v, kv, N, block, M, Mp, kbar, vbar, kp,
                       vbt);
  else
    hipLaunchKernelGGL(pool_kv_kernel<128>, grid, dim3(kThreads), 0, stream,
                       (const uint16_t*)k, (const uint16_t*)v, kv, N, block, M, Mp, kbar, vbar, kp,
                       vbt);
  return hipGetLastError();
}

hipError_t launch_kstats(int d, int64_t BH, int64_t M, const float* kbar, float* kglob,
                         double* kglob64, uint16_t* cp, hipStream_t stream) {
  if (d == 64)
    hipLaunchKernelGGL(kstats_kernel<64>, dim3((unsigned)(BH * 4)), dim3(kThreads), 0, stream,
                       kbar, M, kglob, kglob64, cp);
  else
    hipLaunchKernelGGL(kstats_kernel<128>, dim3((unsigned)(BH * 16)), dim3(kThreads), 0, stream,
                       kbar, M, kglob, kglob64, cp);
  return hipGetLastError();
}

}  // namespace solattn
