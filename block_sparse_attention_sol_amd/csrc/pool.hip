// pool.hip -- K/V mean pooling per key block (HBM-bound), and the mean pooled key per head.
//
// Pooled keys and values: Kbar_j = (1/n_j) sum_{t in block j} K_t, likewise Vbar_j.  The proxy
// score of the Sol-Attn page's routing paragraph is q . Kbar_j / sqrt(d), and Vbar_j is the value
// of block j's pooled token.
//
// One workgroup pools 32 (small heads: 8) consecutive key blocks of one (batch, head) for both K
// and V: each wave reads its blocks' rows as 16-byte chunks (consecutive lanes -> consecutive
// chunks of a row, so each load instruction covers whole rows), accumulates fp32 sums and combines
// the lanes sharing a chunk with cross-lane operations in a fixed order (deterministic).  Besides the fp32 means it
// writes the layouts the attention kernel consumes:
//   kp   [3][BH][Mp][d] bf16: Kbar split into hi + mid + lo bf16 pieces whose sum is the fp32
//        value, so a bf16 matrix product over the three pieces reproduces fp32 proxies;
//   vbt  [BH][d][Mp] bf16: Vbar transposed (block index contiguous), the A operand of the
//        pooled tokens' P Vbar product;
// where Mp = M rounded up to a multiple of 32; padding blocks are written as zeros.
// Two small per-head kernels follow: the mean pooled key and the covariance matrix C of the pooled
// keys (fp64), from which every query's proxy variance is the quadratic form q^T C q / d; then the
// removal of C's dominant directions, if any, so that the form stays well conditioned.
#include "common.hpp"
#include "kernels.hpp"

namespace solattn {

constexpr int kPoolWaves = 8;                // waves per pooling workgroup
// key blocks per pooling workgroup: 32, or 8 (one per wave) when 32 would give fewer than
// kPoolMinGroups workgroups (small heads: more workgroups in flight, one round trip per wave)
constexpr int kPoolBlocks = 32;
constexpr int kPoolBlocksSmall = 8;
constexpr int64_t kPoolMinGroups = 512;

// Sum of x over the lanes that hold the same 16-byte chunk of a row: lanes l, l + C, l + 2C, ...
// for C = D / 8 chunks per row (D = 128: four lanes, D = 64: eight), every lane receiving the sum.
// DPP within a 16-lane row, then the permlane swaps of the 16x16 layout helpers.
template <int D>
__device__ __forceinline__ float chunk_sum(float x) {
  if constexpr (D == 64)
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128,
                                                               0xF, 0xF, false));  // row_ror:8
  return quad_sum(x);
}

// One workgroup pools BLOCKS consecutive key blocks of one (batch, head), for K and V; each wave
// takes BLOCKS / kPoolWaves of them.  A wave loads whole rows (lane l: 16-byte chunk l % C of rows
// l / C, l / C + 64 / C, ...), keeps fp32 sums of its chunk, and combines the lanes that share a
// chunk with cross-lane operations (fixed order: deterministic).  The mean divides by n_j.  Vbar^T
// is staged in LDS and written as one 2 x BLOCKS-byte run per head-dimension row.  K and V
// are streamed with non-temporal loads (each byte is read once; the attention kernel that follows
// reads the heads again from the first, long after these lines would have left the caches).
template <int D, int BLOCKS>
__global__ __launch_bounds__(64 * kPoolWaves) void pool_kv_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, Strides kv, int64_t N, int block,
    int64_t M, int64_t Mp, float* __restrict__ kbar, float* __restrict__ vbar,
    uint16_t* __restrict__ kp, uint16_t* __restrict__ vbt) {
  constexpr int C = D / 8;           // 16-byte chunks per row
  constexpr int RS = 64 / C;         // rows per wave load instruction
  constexpr int U = 8;               // row sets in flight per tensor
  constexpr int kPerWave = BLOCKS / kPoolWaves;
  __shared__ __attribute__((aligned(16))) uint16_t vt[D][BLOCKS];
  const int64_t bh = blockIdx.y;
  const int64_t BH = gridDim.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cc = lane % C, rs = lane / C;
  const uint16_t* kb = k + kv.base(bh);
  const uint16_t* vb = v + kv.base(bh);
  const int64_t jlast = (kp || vbt) ? Mp : M;  // blocks written (padding blocks: zeros)
  for (int bl = 0; bl < kPerWave; ++bl) {
    const int jl = wave * kPerWave + bl;  // block within the group
    const int64_t j = (int64_t)blockIdx.x * BLOCKS + jl;
    if (j >= jlast) break;
    float sk[8], sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sk[e] = sv[e] = 0.f;
    const int64_t lo = j * (int64_t)block;
    const int64_t hi = lo + block < N ? lo + block : N;
    if (j < M) {
      for (int64_t r0 = lo; r0 < hi; r0 += RS * U) {
        u32x4 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t r = r0 + u * RS + rs;
          a[u] = b[u] = u32x4{0u, 0u, 0u, 0u};
          if (r < hi) {  // read once here: non-temporal loads
            a[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + r * kv.sn + cc * 8));
            b[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + r * kv.sn + cc * 8));
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sk[2 * e] += bf16_lo(a[u][e]);
            sk[2 * e + 1] += bf16_hi(a[u][e]);
            sv[2 * e] += bf16_lo(b[u][e]);
            sv[2 * e + 1] += bf16_hi(b[u][e]);
          }
      }
    }
    float mk[8], mv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // true division by n_j (the reciprocal is not used: n_j need not be a power of two)
      mk[e] = j < M ? chunk_sum<D>(sk[e]) / (float)(hi - lo) : 0.f;
      mv[e] = j < M ? chunk_sum<D>(sv[e]) / (float)(hi - lo) : 0.f;
    }
    if (rs == 0) {  // lanes 0 .. C - 1 hold the block's means at d = 8 cc .. 8 cc + 7
      if (j < M) {
        if (kbar) {
          float* kr = kbar + (bh * M + j) * D + cc * 8;
          *reinterpret_cast<f32x4*>(kr) = f32x4{mk[0], mk[1], mk[2], mk[3]};
          *reinterpret_cast<f32x4*>(kr + 4) = f32x4{mk[4], mk[5], mk[6], mk[7]};
        }
        if (vbar) {
          float* vr = vbar + (bh * M + j) * D + cc * 8;
          *reinterpret_cast<f32x4*>(vr) = f32x4{mv[0], mv[1], mv[2], mv[3]};
          *reinterpret_cast<f32x4*>(vr + 4) = f32x4{mv[4], mv[5], mv[6], mv[7]};
        }
      }
      if (kp) {
        u32x4 ph, pm, pl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t h2[2], m2[2], l2[2];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const float m = mk[2 * e + x];
            const uint16_t h16 = f32_to_bf16_rne(m);
            const float r1 = m - bits_f32((uint32_t)h16 << 16);
            const uint16_t m16 = f32_to_bf16_rne(r1);
            const uint16_t l16 = f32_to_bf16_rne(r1 - bits_f32((uint32_t)m16 << 16));
            h2[x] = h16;
            m2[x] = m16;
            l2[x] = l16;
          }
          ph[e] = h2[0] | (h2[1] << 16);
          pm[e] = m2[0] | (m2[1] << 16);
          pl[e] = l2[0] | (l2[1] << 16);
        }
        const int64_t off = (bh * Mp + j) * D + cc * 8;
        *reinterpret_cast<u32x4*>(kp + off) = ph;
        *reinterpret_cast<u32x4*>(kp + BH * Mp * D + off) = pm;
        *reinterpret_cast<u32x4*>(kp + 2 * BH * Mp * D + off) = pl;
      }
      if (vbt) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vt[cc * 8 + e][jl] = f32_to_bf16_rne(mv[e]);
      }
    }
  }
  if (vbt) {
    __syncthreads();
    // row d of the group's Vbar^T tile: BLOCKS bf16 = BLOCKS / 8 chunks of 16 bytes
    const int64_t j0 = (int64_t)blockIdx.x * BLOCKS;
    for (int i = threadIdx.x; i < D * (BLOCKS / 8); i += 64 * kPoolWaves) {
      const int d = i / (BLOCKS / 8), ch = i % (BLOCKS / 8);
      if (j0 + ch * 8 < Mp)
        *reinterpret_cast<u32x4*>(vbt + (bh * D + d) * Mp + j0 + ch * 8) =
            *reinterpret_cast<const u32x4*>(&vt[d][ch * 8]);
    }
  }
}

// Mean and covariance of the pooled keys of each head, in fp64:
//   g[a] = (1/M) sum_j Kbar_j[a],   C[a][b] = (1/M) sum_j Kbar_j[a] Kbar_j[b] - g[a] g[b].
// The mean proxy score of a query is q . g / sqrt(d) (the mean is linear), and for the proxy row
// s_ij = q_i . Kbar_j / sqrt(d) the population variance over j is exactly q_i^T C q_i / d.
// Writes g and C (fp64; C as [BH][D][D]) for the factorisation below.
// One workgroup computes a 32 x 32 tile of C: pooled keys are staged through LDS in chunks of 64
// blocks, each thread accumulates a 2 x 2 block of products and, from the same operands, the sums
// of its two a columns and two b columns (the threads of row 0 / column 0 of the thread grid
// publish them).  The diagonal tiles (ai == bi) also write g.
template <int D>
__global__ __launch_bounds__(kThreads) void kstats_kernel(const float* __restrict__ kbar, int64_t M,
                                                          double* __restrict__ kglob,
                                                          double* __restrict__ c64) {
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
  double sa0 = 0.0, sa1 = 0.0, sb0 = 0.0, sb1 = 0.0;  // sums of a columns 2 ta + {0,1}, b 2 tb + {0,1}
  // the next chunk's pooled keys are loaded into registers while this chunk is multiplied
  constexpr int kPer = kChunk * 32 / kThreads;  // elements of each of sa, sb per thread
  static_assert(kPer * kThreads == kChunk * 32, "whole chunk per pass");
  float na[kPer], nb[kPer];
  auto fetch = [&](int64_t j0) {
    const int n = (int)((M - j0) < kChunk ? (M - j0) : kChunk);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int idx = t + e * kThreads;
      const int r = idx / 32, col = idx % 32;
      na[e] = r < n ? kb[(j0 + r) * D + 32 * ai + col] : 0.f;
      nb[e] = r < n ? kb[(j0 + r) * D + 32 * bi + col] : 0.f;
    }
  };
  fetch(0);
  for (int64_t j0 = 0; j0 < M; j0 += kChunk) {
    const int n = (int)((M - j0) < kChunk ? (M - j0) : kChunk);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int idx = t + e * kThreads;
      const int r = idx / 32, col = idx % 32;
      sa[r][col] = (double)na[e];
      sb[r][col] = (double)nb[e];
    }
    __syncthreads();
    if (j0 + kChunk < M) fetch(j0 + kChunk);
    for (int r = 0; r < n; ++r) {
      const double a0 = sa[r][2 * ta], a1 = sa[r][2 * ta + 1];
      const double b0 = sb[r][2 * tb], b1 = sb[r][2 * tb + 1];
      c00 = fma(a0, b0, c00);
      c01 = fma(a0, b1, c01);
      c10 = fma(a1, b0, c10);
      c11 = fma(a1, b1, c11);
      sa0 += a0;
      sa1 += a1;
      sb0 += b0;
      sb1 += b1;
    }
  }
  __shared__ double ga[32], gb[32];
  if (tb == 0) {
    ga[2 * ta] = sa0 / (double)M;
    ga[2 * ta + 1] = sa1 / (double)M;
    if (ai == bi) {
      kglob[bh * D + 32 * ai + 2 * ta] = sa0 / (double)M;
      kglob[bh * D + 32 * ai + 2 * ta + 1] = sa1 / (double)M;
    }
  }
  if (ta == 0) {
    gb[2 * tb] = sb0 / (double)M;
    gb[2 * tb + 1] = sb1 / (double)M;
  }
  __syncthreads();
  const double inv_m = 1.0 / (double)M;
  const double cv[2][2] = {{c00, c01}, {c10, c11}};
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int ra = 2 * ta + x, rb = 2 * tb + y;
      c64[(bh * D + 32 * ai + ra) * D + 32 * bi + rb] = cv[x][y] * inv_m - ga[ra] * gb[rb];
    }
}

// Dominant directions of each head's pooled-key covariance, removed before the quadratic form.
// The row statistics evaluate sigma_i^2 d = q^T C q on the matrix cores (fp32-accurate), whose
// rounding error scales with |q|^T |C| |q| rather than with q^T C q: when C has a direction far
// stronger than the others and q is nearly orthogonal to it, the relative error grows by the ratio
// of the two.  Such directions are split off by steps of Cholesky with diagonal pivoting in fp64,
//   C = sum_{k<T} w_k w_k^T + S_T,
// and q^T C q = sum_k (w_k . q)^2 + q^T S_T q, the w_k . q taken in fp64 by the row statistics and
// the well-conditioned remainder S_T on the matrix cores.  Step k (pivot: the largest remaining
// diagonal entry, lowest index on ties) is taken only while its row is dominant, |w_k|^2 >
// kDominant * trace(S_{k+1}) / D, and at most kFactorTop times.  On the synthetic video-token
// workloads this ratio is 4-11 (no step taken); one strong key direction gives ~10^5.
// Writes w_k (fp64) to f64top [BH][kFactorTop][D], T to ftop [BH], and S_T as three bf16 pieces
// (hi, mid, lo; their sum is the fp32 value) to cp [3][BH][D][D], each row's columns in the order
// the row statistics take the query in: column b at position b with bits 2 and 3 swapped (so the
// 16-byte chunk 2 kk + h of a row holds columns 16 kk + 4 h + 0..3 and 16 kk + 8 + 4 h + 0..3).
// One workgroup per head: thread t owns the TB x TB block (t / 16, t % 16) of S in registers.
template <int D>
__global__ __launch_bounds__(kThreads) void kdeflate_kernel(const double* __restrict__ c64,
                                                            uint16_t* __restrict__ cp,
                                                            double* __restrict__ f64top,
                                                            int32_t* __restrict__ ftop, int64_t BH) {
  constexpr int TB = D / 16;  // block edge
  static_assert(kThreads == 256, "a 16 x 16 grid of blocks");
  __shared__ double dg[D];    // remaining diagonal (-inf once pivoted)
  __shared__ double col[D];   // pivot column
  const int64_t bh = blockIdx.x;
  const int t = threadIdx.x;
  const int br = t / 16, bc = t % 16;
  const int lane = t & 63;
  const double* C = c64 + bh * D * D;
  double S[TB][TB];
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j) S[i][j] = C[(br * TB + i) * D + bc * TB + j];
  uint32_t piv_r = 0u, piv_c = 0u;  // pivoted rows / columns among this thread's TB
  if (br == bc) {
#pragma unroll
    for (int i = 0; i < TB; ++i) dg[br * TB + i] = S[i][i];
  }
  __syncthreads();
  double* F64 = f64top + bh * kFactorTop * D;
  int k = 0;
  for (; k < kFactorTop; ++k) {
    // pivot: argmax of the remaining diagonal, lowest index on ties (each wave reduces all D)
    double bv = -INFINITY;
    int bi = D;
    for (int i = lane; i < D; i += 64) {
      const double x = dg[i];
      if (x > bv) { bv = x; bi = i; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    const int p = __builtin_amdgcn_readfirstlane(bi);
    const double dmax = bv;
    if (!(dmax > 0.0)) break;  // uniform: every wave reduced the same values
    if (bc == p / TB) {
#pragma unroll
      for (int i = 0; i < TB; ++i) col[br * TB + i] = S[i][p % TB];
    }
    __syncthreads();
    // |w|^2 and the remaining trace: each wave sums all D entries, lane-strided and then by a
    // butterfly, in the same order in every wave, so every wave takes the same decision
    const double rs = 1.0 / sqrt(dmax);
    double nw = 0.0, tr = 0.0;
    for (int i = lane; i < D; i += 64) {
      const double di = dg[i];
      if (di != -INFINITY) {
        const double wi = i == p ? sqrt(dmax) : col[i] * rs;
        nw = fma(wi, wi, nw);
        tr += di;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      nw += __shfl_xor(nw, off);
      tr += __shfl_xor(tr, off);
    }
    if (!(nw > kDominant * (tr - nw) / (double)D)) break;  // uniform
    double wr[TB], wc[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      const int r = br * TB + i, c = bc * TB + i;
      wr[i] = ((piv_r >> i) & 1u) ? 0.0 : (r == p ? sqrt(dmax) : col[r] * rs);
      wc[i] = ((piv_c >> i) & 1u) ? 0.0 : (c == p ? sqrt(dmax) : col[c] * rs);
    }
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
      for (int j = 0; j < TB; ++j) S[i][j] = fma(-wr[i], wc[j], S[i][j]);
    if (br == p / TB) piv_r |= 1u << (p % TB);
    if (bc == p / TB) piv_c |= 1u << (p % TB);
    __syncthreads();  // every thread has read dg and col of this step
    if (br == bc) {
#pragma unroll
      for (int i = 0; i < TB; ++i) dg[br * TB + i] = ((piv_r >> i) & 1u) ? -INFINITY : S[i][i];
    }
    if (bc == 0) {
#pragma unroll
      for (int i = 0; i < TB; ++i) F64[k * D + br * TB + i] = wr[i];
    }
    __syncthreads();
  }
  if (t == 0) ftop[bh] = k;
  // S_T in three bf16 pieces; pivoted rows and columns are exactly zero in exact arithmetic and
  // are written as zero
  const int64_t piece = BH * D * D;
  uint16_t* P = cp + bh * D * D;
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const bool zero = ((piv_r >> i) & 1u) || ((piv_c >> j) & 1u);
      const float x = zero ? 0.f : (float)S[i][j];
      const uint16_t h16 = f32_to_bf16_rne(x);
      const float r1 = x - bits_f32((uint32_t)h16 << 16);
      const uint16_t m16 = f32_to_bf16_rne(r1);
      const uint16_t l16 = f32_to_bf16_rne(r1 - bits_f32((uint32_t)m16 << 16));
      const int b = bc * TB + j;
      const int64_t off = (int64_t)(br * TB + i) * D + ((b & ~12) | ((b & 4) << 1) | ((b & 8) >> 1));
      P[off] = h16;
      P[piece + off] = m16;
      P[2 * piece + off] = l16;
    }
}

hipError_t launch_pool(int d, int64_t BH, int64_t N, int block, const void* k, const void* v,
                       const Strides& kv,
                       float* kbar, float* vbar, uint16_t* kp, uint16_t* vbt, int64_t Mp,
                       hipStream_t stream) {
  const int64_t M = (N + block - 1) / block;
  const int64_t nb = (kp || vbt) ? Mp : M;
  const bool small = BH * ((nb + kPoolBlocks - 1) / kPoolBlocks) < kPoolMinGroups;
  const int per = small ? kPoolBlocksSmall : kPoolBlocks;
  dim3 grid((unsigned)((nb + per - 1) / per), (unsigned)BH);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(64 * kPoolWaves), 0, stream, (const uint16_t*)k,
                       (const uint16_t*)v, kv, N, block, M, Mp, kbar, vbar, kp, vbt);
  };
  if (d == 64)
    small ? go(pool_kv_kernel<64, kPoolBlocksSmall>) : go(pool_kv_kernel<64, kPoolBlocks>);
  else
    small ? go(pool_kv_kernel<128, kPoolBlocksSmall>) : go(pool_kv_kernel<128, kPoolBlocks>);
  return hipGetLastError();
}

hipError_t launch_kstats(int d, int64_t BH, int64_t M, const float* kbar, double* kglob,
                         double* c64, uint16_t* cp, double* f64top, int32_t* ftop,
                         hipStream_t stream) {
  if (d == 64) {
    hipLaunchKernelGGL(kstats_kernel<64>, dim3((unsigned)(BH * 4)), dim3(kThreads), 0, stream,
                       kbar, M, kglob, c64);
    hipLaunchKernelGGL(kdeflate_kernel<64>, dim3((unsigned)BH), dim3(kThreads), 0, stream, c64, cp,
                       f64top, ftop, BH);
  } else {
    hipLaunchKernelGGL(kstats_kernel<128>, dim3((unsigned)(BH * 16)), dim3(kThreads), 0, stream,
                       kbar, M, kglob, c64);
    hipLaunchKernelGGL(kdeflate_kernel<128>, dim3((unsigned)BH), dim3(kThreads), 0, stream, c64, cp,
                       f64top, ftop, BH);
  }
  return hipGetLastError();
}

}  // namespace solattn
