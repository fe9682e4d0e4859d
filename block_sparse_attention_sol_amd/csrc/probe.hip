// probe.hip -- matrix-core rate probe (measurement only): the bf16 MFMA rate this part sustains
// when every wave issues nothing but independent 32x32x16 MFMAs on register operands.  The
// attention kernels' roofline fractions are also reported against this measured rate.
#include "common.hpp"
#include "kernels.hpp"

namespace solattn {

constexpr int kProbeChains = 8;  // independent accumulators per wave

__global__ __launch_bounds__(kThreads) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.002f * (float)((lane * 3 + e) & 7));
  }
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int k = 0; k < kProbeChains; ++k) acc[k] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kProbeChains; ++k) acc[k] = mfma32(a, b, acc[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kProbeChains; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[k][v];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

hipError_t launch_mfma_probe(int workgroups, int iters, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0, stream, iters,
                     sink);
  return hipGetLastError();
}

int mfma_probe_chains() { return kProbeChains; }

}  // namespace solattn
