// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to libsolattn).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace solattn {

// Pooled K/V of every key block.  kp / vbt (and Mp) only for the attention workspace; NULL in
// the public pooling call.
hipError_t launch_pool(int d, int64_t BH, int64_t N, int block, const void* k, const void* v,
                       const Strides& kv, float* kbar, float* vbar, uint16_t* kp, uint16_t* vbt,
                       int64_t Mp, hipStream_t stream);
// Mean (fp64, kglob [BH][d]) and covariance (fp64, c64 [BH][d][d]) of the pooled keys of every
// head, then the covariance's dominant directions w_k (k < ftop[bh], fp64, f64top
// [BH][kFactorTop][d]) split off, C = sum_k w_k w_k^T + S, and the remainder S as three bf16 pieces
// cp [3][BH][d][d].
constexpr int kFactorTop = 4;          // at most this many factor rows in fp64
constexpr double kDominant = 64.0;     // |w_k|^2 over the remaining mean diagonal: dominant
hipError_t launch_kstats(int d, int64_t BH, int64_t M, const float* kbar, double* kglob,
                         double* c64, uint16_t* cp, double* f64top, int32_t* ftop,
                         hipStream_t stream);

struct RowStatsArgs {
  const uint16_t* q;
  Strides qs;
  const uint16_t* cp;     // [3][BH][d][d] covariance with the dominant directions removed
                          // (pieces hi, mid, lo)
  const double* f64top;   // [BH][kFactorTop][d] the dominant directions w_k (fp64)
  const int32_t* ftop;    // [BH] how many of them
  const double* kglob;    // [BH][d] mean pooled key
  int64_t BH, N;
  float beta;
  float* tau;             // [BH][N] (workspace): selection threshold, -inf where sigma = 0
  float* mu;              // optional outputs
  float* sigma;
  float* tau_out;
};
hipError_t launch_rowstats(int d, const RowStatsArgs& a, hipStream_t stream);

struct SparseArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  Strides in;           // q, k, v
  Strides outs;         // out
  const uint16_t* kp;   // [3][BH][Mp][d] pooled keys (hi, mid, lo)
  const uint16_t* vbt;  // [BH][d][Mp] pooled values, transposed
  const float* tau;     // [BH][N]
  uint32_t* rowmask;    // [BH][Mp/32][N] selection words, word-major (written by the routing
                        // sweep, read back per row by the exact loop)
  int64_t BH, N, M, Mp;
  int block;
  int drop;
  const uint32_t* mask_in;  // [BH][N][Mp/32] caller's selection (replaces s >= tau), or NULL
  // latent grid of the query rows (frames, rows, 16-token segments per row) for the grouping of
  // 16-row segments into workgroups; gS = 0: consecutive rows (the only grouping at d = 64)
  int64_t gT, gH, gS;
  // optional outputs
  uint32_t* mask_out;   // [BH][N][Mp/32] selection words, row-major
  float* lse;
  int32_t* tile_kept;
  float* out_f32;
};
hipError_t launch_sparse(int d, const SparseArgs& a, hipStream_t stream);
// tile_kept[bh][t] = key blocks kept by some row of contiguous 128-row tile t, from the routing
// sweep's selection words rowmask [BH][W][N] (W = Mp / 32)
hipError_t launch_tile_union(int64_t BH, int64_t N, int64_t W, const uint32_t* rowmask,
                             int32_t* tile_kept, hipStream_t stream);

hipError_t launch_dense(int d, int64_t BH, int64_t N, const void* q, const void* k, const void* v,
                        const Strides& in, void* out, const Strides& outs, float* lse,
                        hipStream_t stream);

// Full proxy map s_map[BH][N][M] = q . Kbar_j / sqrt(d) (fp32, row-major) from the pooled-key
// pieces kp [3][BH][Mp][d].
hipError_t launch_proxy_map(int d, const uint16_t* q, const Strides& qs, const uint16_t* kp,
                            int64_t BH, int64_t N, int64_t M, int64_t Mp, float* s_map,
                            hipStream_t stream);
// Top-k (mode 0, count k) or top-p (mode 1, probability p) selection per row from s_map, written as
// mask [BH][N][ceil(M/32)].
hipError_t launch_route_select(int mode, const float* s_map, int64_t BH, int64_t N, int64_t M,
                               int block, int64_t k, float p, uint32_t* mask, hipStream_t stream);
int64_t route_max_blocks();  // largest M the selection kernel holds in registers

// The allocation-free call's workspace: a file-scope device array of kNoAllocScratchBytes per GPU
// (SOL_NOALLOC_SCRATCH_BYTES in the public header); *ptr receives the current device's copy.
constexpr size_t kNoAllocScratchBytes = size_t(256) << 20;
hipError_t noalloc_scratch(void** ptr);

// Matrix-core rate probe: `workgroups` x 4 waves, each issuing iters x mfma_probe_chains()
// independent bf16 32x32x16 MFMAs.
hipError_t launch_mfma_probe(int workgroups, int iters, float* sink, hipStream_t stream);
int mfma_probe_chains();

}  // namespace solattn
