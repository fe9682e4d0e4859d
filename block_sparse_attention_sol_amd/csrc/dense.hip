// dense.hip -- the dense reference attention kernel and the full proxy map (gfx950).
//
//   dense_attn_kernel  softmax(Q K^T / sqrt(d)) V over every key, no routing: the reference the
//                      Sol-Attn speedup is measured against.  The same tile mapping and operand
//                      layouts as the fused kernels, with a software-pipelined loop in 32-key steps.
//   proxy_map_kernel   every query's proxy score for every key block, written to memory: the input
//                      of the prior-art top-k / top-p routing the fused kernel replaces.
#include "tiles.hpp"

namespace solattn {

// ---------------------------------------------------------------------------------------------
// Software-pipelined exact loop, in steps of 32 keys (half a 64-key stage).  A wave keeps two
// score blocks live: while the matrix cores compute S^T of the next 32 keys (phase A), the vector
// ALU turns the current 32 keys' scores into probabilities; while the matrix cores accumulate
// O^T += V^T P^T for the current 32 keys (phase B), the vector ALU takes the next block's row
// maximum.  K and V tiles are double buffered separately, each with its own barrier, so the next
// stage's keys can be in use while this stage's values still are.  The sched_group_barrier
// pattern asks for vector work behind every MFMA; the compiler still moves phase A's probabilities
// below the partial-block branch, after the S^T chain.  Pinning them behind each MFMA measured no
// faster: with two waves per SIMD, the other wave fills what one in-order wave leaves idle.
// ---------------------------------------------------------------------------------------------
constexpr int kSgValu = 0x002 | 0x400;  // vector and transcendental instructions

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
