// dense.hip -- the dense reference attention kernel and the full proxy map (gfx950).
//
//   dense_attn_kernel  softmax(Q K^T / sqrt(d)) V over every key, no routing: the reference the
//                      Sol-Attn speedup is measured against.  The same tile mapping and operand
//                      layouts as the fused kernels, with a software-pipelined loop in 32-key steps.
//   proxy_map_kernel   every query's proxy score for every key block, written to memory: the input
//                      of the prior-art top-k / top-p routing the fused kernel replaces.
#include "tiles.hpp"

namespace solattn {

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
