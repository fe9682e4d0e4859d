// api.cpp -- the C ABI of libsolattn (declared in include/solattn.h): argument validation,
// workspace carving and kernel launches on the caller's stream.
//
// Every argument check happens before the first HIP call, so invalid calls return an error code
// without touching the device.  No call allocates, frees or synchronises device memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kernels.hpp"
#include "solattn.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return SOL_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t n_blocks(int64_t N, int block) { return (N + block - 1) / block; }
int64_t padded_blocks(int64_t N, int block) { return (n_blocks(N, block) + 31) / 32 * 32; }

// Offsets of the workspace regions (all 256-byte aligned).
struct Workspace {
  size_t kbar, kglob, c64, f64top, ftop, cp, kp, vbt, tau, rowmask, total;
};

Workspace layout(const sol_shape& s, int block) {
  const int64_t BH = s.B * s.H;
  const int64_t M = n_blocks(s.N, block);
  const int64_t Mp = padded_blocks(s.N, block);
  Workspace w{};
  w.kbar = 0;
  w.kglob = w.kbar + align_up((size_t)(BH * M * s.d) * sizeof(float));
  w.c64 = w.kglob + align_up((size_t)(BH * s.d) * sizeof(double));
  w.f64top = w.c64 + align_up((size_t)(BH * s.d * s.d) * sizeof(double));
  w.ftop = w.f64top + align_up((size_t)(BH * solattn::kFactorTop * s.d) * sizeof(double));
  w.cp = w.ftop + align_up((size_t)BH * sizeof(int32_t));
  w.kp = w.cp + align_up((size_t)(3 * BH * s.d * s.d) * sizeof(uint16_t));
  w.vbt = w.kp + align_up((size_t)(3 * BH * Mp * s.d) * sizeof(uint16_t));
  w.tau = w.vbt + align_up((size_t)(BH * s.d * Mp) * sizeof(uint16_t));
  w.rowmask = w.tau + align_up((size_t)(BH * s.N) * sizeof(float));
  w.total = w.rowmask + align_up((size_t)(BH * s.N * (Mp / 32)) * sizeof(uint32_t));
  return w;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(const sol_shape* s) {
  if (!s) return fail(SOL_EINVAL, "shape is NULL");
  if (s->B < 1 || s->H < 1) return fail(SOL_EINVAL, "B and H must be >= 1 (got B=%lld H=%lld)",
                                        (long long)s->B, (long long)s->H);
  if (s->N < 1 || s->N > (int64_t(1) << 22))
    return fail(SOL_EINVAL, "N must be in [1, 2^22] (got %lld)", (long long)s->N);
  if (s->B * s->H > 65535) return fail(SOL_EINVAL, "B*H must be <= 65535 (got %lld)",
                                       (long long)(s->B * s->H));
  if (s->d != 64 && s->d != 128)
    return fail(SOL_EUNSUPPORTED, "d must be 64 or 128 (got %lld)", (long long)s->d);
  const int64_t tiles = (s->N + SOL_QUERY_TILE - 1) / SOL_QUERY_TILE;
  if (s->B * s->H * tiles > (int64_t)INT32_MAX)
    return fail(SOL_EINVAL, "B*H*ceil(N/%d) exceeds the launch grid", SOL_QUERY_TILE);
  return SOL_OK;
}

int check_block(int block) {
  if (block != 64 && block != 128)
    return fail(SOL_EUNSUPPORTED, "block must be 64 or 128 (got %d)", block);
  return SOL_OK;
}

int check_tensor(const void* p, const char* name) {
  if (!p) return fail(SOL_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(SOL_EINVAL, "%s is not 16-byte aligned", name);
  return SOL_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

solattn::Strides contiguous(const sol_shape& s) {
  return solattn::Strides::contiguous(s.H, s.N, s.d);
}

solattn::Strides to_strides(const sol_shape& s, const sol_strides* st) {
  if (!st) return contiguous(s);
  return solattn::Strides{s.H, st->b, st->h, st->n};
}

// Bytes from the first element of a strided [B][H][N][d] bf16 view to the end of its last row.
size_t extent_bytes(const sol_shape& s, const solattn::Strides& st) {
  return (size_t)((s.B - 1) * st.sb + (s.H - 1) * st.sh + (s.N - 1) * st.sn + s.d) * 2;
}

// Strides the kernels accept: non-negative, multiples of 8 elements (16-byte aligned rows), rows
// at least d apart and within the copies' 32-bit per-lane offsets; for an output (writable)
// also no two elements at one address: sorted by stride, every dimension of size > 1 must step
// past the whole extent of the dimensions inside it.
int check_strides(const sol_shape& s, const sol_strides* st, const char* name, bool writable) {
  if (!st) return SOL_OK;
  const int64_t v[3] = {st->b, st->h, st->n};
  for (int64_t x : v)
    if (x < 0 || (x & 7)) return fail(SOL_EINVAL, "%s strides must be non-negative multiples of 8", name);
  if (st->n < s.d) return fail(SOL_EINVAL, "%s token stride %lld is below d", name, (long long)st->n);
  if (st->n > (int64_t(1) << 23)) return fail(SOL_EUNSUPPORTED, "%s token stride too large", name);
  if (writable) {
    int64_t dims[3][2] = {{st->n, s.N}, {st->h, s.H}, {st->b, s.B}};
    for (int i = 0; i < 3; ++i)  // sort by stride
      for (int j = i + 1; j < 3; ++j)
        if (dims[j][0] < dims[i][0]) {
          int64_t t0 = dims[i][0], t1 = dims[i][1];
          dims[i][0] = dims[j][0]; dims[i][1] = dims[j][1];
          dims[j][0] = t0; dims[j][1] = t1;
        }
    int64_t inner = s.d;  // extent covered by the dimensions inside
    for (int i = 0; i < 3; ++i) {
      if (dims[i][1] == 1) continue;
      if (dims[i][0] < inner) return fail(SOL_EINVAL, "%s strides make elements overlap", name);
      inner = dims[i][0] * (dims[i][1] - 1) + inner;
    }
  }
  return SOL_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SOL_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int sol_mfma_probe(int workgroups, int iters, float* sink, void* stream) {
  if (workgroups < 1) return fail(SOL_EINVAL, "workgroups must be >= 1 (got %d)", workgroups);
  if (iters < 1) return fail(SOL_EINVAL, "iters must be >= 1 (got %d)", iters);
  if (!sink) return fail(SOL_EINVAL, "sink is NULL");
  const hipError_t e = solattn::launch_mfma_probe(workgroups, iters, sink, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SOL_EHIP, "mfma probe launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* sol_version(void) { return "libsolattn 0.1 (gfx950)"; }

const char* sol_status_str(int status) {
  switch (status) {
    case SOL_OK: return "ok";
    case SOL_EINVAL: return "invalid argument";
    case SOL_EUNSUPPORTED: return "unsupported head dimension or block size";
    case SOL_EWORKSPACE: return "workspace missing or too small";
    case SOL_EHIP: return "HIP runtime error";
    case SOL_ENOTIMPL: return "not implemented";
    default: return "unknown status";
  }
}

const char* sol_last_error(void) { return g_last_error; }

size_t sol_attn_workspace_bytes(const sol_shape* shape, int block) {
  if (check_shape(shape) != SOL_OK || check_block(block) != SOL_OK) return 0;
  return layout(*shape, block).total;
}

int sol_pool_kv(const sol_shape* shape, const void* k, const void* v, int block, float* kbar,
                float* vbar, void* stream) {
  int st;
  if ((st = check_shape(shape)) || (st = check_block(block))) return st;
  if ((st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
      (st = check_tensor(kbar, "kbar")) || (st = check_tensor(vbar, "vbar")))
    return st;
  const int64_t BH = shape->B * shape->H;
  const int64_t M = n_blocks(shape->N, block);
  const size_t pooled = (size_t)(BH * M * shape->d) * sizeof(float);
  if (overlaps(kbar, pooled, vbar, pooled)) return fail(SOL_EINVAL, "kbar and vbar overlap");
  return hip_status(solattn::launch_pool((int)shape->d, BH, shape->N, block, k, v,
                                         contiguous(*shape), kbar, vbar, nullptr, nullptr, 0,
                                         (hipStream_t)stream),
                    "pool kernel launch");
}

namespace {

// sol_attn_fwd_ex and sol_attn_fwd_masked: with mask_in the caller's selection replaces the
// threshold (no row statistics are computed) and `drop` comes from the argument.
int attn_forward(const sol_shape* shape, const sol_strides* in_st, const sol_strides* out_st,
                 const void* q, const void* k, const void* v, float beta, int block, void* out,
                 void* workspace, size_t workspace_bytes, const sol_attn_debug* dbg,
                 const uint32_t* mask_in, int drop_in, void* stream,
                 const sol_grid* grid = nullptr) {
  int st;
  if ((st = check_shape(shape)) || (st = check_block(block))) return st;
  if (grid) {
    const int64_t N = shape->N;
    if (grid->T < 1 || grid->H < 1 || grid->W < 1 || grid->T > N || grid->H > N || grid->W > N ||
        grid->T * grid->H > N || grid->T * grid->H * grid->W != N)
      return fail(SOL_EINVAL, "grid %lld x %lld x %lld does not hold N = %lld tokens",
                  (long long)grid->T, (long long)grid->H, (long long)grid->W, (long long)N);
  }
  if ((st = check_strides(*shape, in_st, "input", false)) ||
      (st = check_strides(*shape, out_st, "output", true)))
    return st;
  const solattn::Strides ins = to_strides(*shape, in_st), outs = to_strides(*shape, out_st);
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
      (st = check_tensor(out, "out")))
    return st;
  if (!mask_in && std::isnan(beta)) return fail(SOL_EINVAL, "beta is NaN");
  if (mask_in && ((uintptr_t)mask_in & 3u)) return fail(SOL_EINVAL, "mask is not 4-byte aligned");
  const Workspace w = layout(*shape, block);
  if (!workspace) return fail(SOL_EWORKSPACE, "workspace is NULL (need %zu bytes)", w.total);
  if (!aligned16(workspace)) return fail(SOL_EINVAL, "workspace is not 16-byte aligned");
  if (workspace_bytes < w.total)
    return fail(SOL_EWORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, w.total);
  const size_t ein = extent_bytes(*shape, ins), eout = extent_bytes(*shape, outs);
  if (overlaps(out, eout, q, ein) || overlaps(out, eout, k, ein) || overlaps(out, eout, v, ein) ||
      overlaps(out, eout, workspace, w.total))
    return fail(SOL_EINVAL, "out overlaps an input or the workspace");
  if (dbg) {
    const void* opt[] = {dbg->mask, dbg->mu,  dbg->sigma,    dbg->tau,
                         dbg->lse,  dbg->tile_kept, dbg->out_f32};
    for (const void* p : opt)
      if (p && ((uintptr_t)p & 3u)) return fail(SOL_EINVAL, "debug output not 4-byte aligned");
    if (dbg->out_f32 && !aligned16(dbg->out_f32))
      return fail(SOL_EINVAL, "out_f32 is not 16-byte aligned");
  }

  const int d = (int)shape->d;
  const int64_t BH = shape->B * shape->H;
  const int64_t M = n_blocks(shape->N, block);
  const int64_t Mp = padded_blocks(shape->N, block);
  unsigned char* ws = (unsigned char*)workspace;
  float* kbar = (float*)(ws + w.kbar);
  double* kglob = (double*)(ws + w.kglob);
  double* c64 = (double*)(ws + w.c64);
  double* f64top = (double*)(ws + w.f64top);
  int32_t* ftop = (int32_t*)(ws + w.ftop);
  uint16_t* cp = (uint16_t*)(ws + w.cp);
  uint16_t* kp = (uint16_t*)(ws + w.kp);
  uint16_t* vbt = (uint16_t*)(ws + w.vbt);
  float* tau = (float*)(ws + w.tau);
  uint32_t* rowmask = (uint32_t*)(ws + w.rowmask);
  hipStream_t s = (hipStream_t)stream;

  auto mark = [&](int i) -> hipError_t {
    if (dbg && dbg->events[i]) return hipEventRecord((hipEvent_t)dbg->events[i], s);
    return hipSuccess;
  };
  hipError_t e = mark(0);
  if (e != hipSuccess) return hip_status(e, "event record");
  e = solattn::launch_pool(d, BH, shape->N, block, k, v, ins, kbar, nullptr, kp, vbt, Mp, s);
  if (e != hipSuccess) return hip_status(e, "pool kernel launch");
  if ((e = mark(1)) != hipSuccess) return hip_status(e, "event record");
  if (!mask_in) {
    e = solattn::launch_kstats(d, BH, M, kbar, kglob, c64, cp, f64top, ftop, s);
    if (e != hipSuccess) return hip_status(e, "pooled-key statistics launch");
    solattn::RowStatsArgs r{};
    r.q = (const uint16_t*)q;
    r.qs = ins;
    r.cp = cp;
    r.kglob = kglob;
    r.f64top = f64top;
    r.ftop = ftop;
    r.BH = BH;
    r.N = shape->N;
    r.beta = beta;
    r.tau = tau;
    if (dbg) {
      r.mu = dbg->mu;
      r.sigma = dbg->sigma;
      r.tau_out = dbg->tau;
    }
    e = solattn::launch_rowstats(d, r, s);
    if (e != hipSuccess) return hip_status(e, "row statistics launch");
  }
  if ((e = mark(2)) != hipSuccess) return hip_status(e, "event record");

  solattn::SparseArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.out = (uint16_t*)out;
  a.in = ins;
  a.outs = outs;
  a.kp = kp;
  a.vbt = vbt;
  a.tau = tau;
  a.rowmask = rowmask;
  a.mask_in = mask_in;
  a.mask_out = dbg ? dbg->mask : nullptr;
  a.BH = BH;
  a.N = shape->N;
  a.M = M;
  a.Mp = Mp;
  a.block = block;
  a.drop = drop_in;
  // the latent grid regroups the 16-row segments of the d = 128 kernel (whole segments per row)
  const bool grouped = grid && d == 128 && grid->W % 16 == 0;
  if (grouped) {
    a.gT = grid->T;
    a.gH = grid->H;
    a.gS = grid->W / 16;
  }
  if (dbg) {
    if (!mask_in) a.drop = dbg->drop_unselected ? 1 : 0;
    a.lse = dbg->lse;
    a.tile_kept = grouped ? nullptr : dbg->tile_kept;
    a.out_f32 = dbg->out_f32;
  }
  e = solattn::launch_sparse(d, a, s);
  if (e != hipSuccess) return hip_status(e, "sparse attention kernel launch");
  if ((e = mark(3)) != hipSuccess) return hip_status(e, "event record");
  if (grouped && dbg && dbg->tile_kept) {  // contiguous-tile unions, after the timed kernels
    e = solattn::launch_tile_union(BH, shape->N, Mp / 32, rowmask, dbg->tile_kept, s);
    if (e != hipSuccess) return hip_status(e, "tile union launch");
  }
  return SOL_OK;
}

}  // namespace

int sol_attn_fwd_ex(const sol_shape* shape, const void* q, const void* k, const void* v,
                    float beta, int block, void* out, void* workspace, size_t workspace_bytes,
                    const sol_attn_debug* dbg, void* stream) {
  return attn_forward(shape, nullptr, nullptr, q, k, v, beta, block, out, workspace,
                      workspace_bytes, dbg, nullptr, 0, stream);
}

int sol_attn_fwd_grid(const sol_shape* shape, const sol_grid* grid, const void* q, const void* k,
                      const void* v, float beta, int block, void* out, void* workspace,
                      size_t workspace_bytes, const sol_attn_debug* dbg, void* stream) {
  if (!grid) return fail(SOL_EINVAL, "grid is NULL");
  return attn_forward(shape, nullptr, nullptr, q, k, v, beta, block, out, workspace,
                      workspace_bytes, dbg, nullptr, 0, stream, grid);
}

int sol_attn_fwd_strided(const sol_shape* shape, const sol_strides* in_strides,
                         const sol_strides* out_strides, const void* q, const void* k,
                         const void* v, float beta, int block, void* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return attn_forward(shape, in_strides, out_strides, q, k, v, beta, block, out, workspace,
                      workspace_bytes, nullptr, nullptr, 0, stream);
}

int sol_attn_fwd_masked(const sol_shape* shape, const void* q, const void* k, const void* v,
                        const uint32_t* mask, int block, int drop_unselected, void* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!mask) return fail(SOL_EINVAL, "mask is NULL");
  return attn_forward(shape, nullptr, nullptr, q, k, v, 0.f, block, out, workspace,
                      workspace_bytes, nullptr, mask, drop_unselected ? 1 : 0, stream);
}

int sol_proxy_map(const sol_shape* shape, const void* q, const void* k, int block, float* s_map,
                  void* workspace, size_t workspace_bytes, void* stream) {
  int st;
  if ((st = check_shape(shape)) || (st = check_block(block))) return st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) ||
      (st = check_tensor(s_map, "s_map")))
    return st;
  const Workspace w = layout(*shape, block);
  if (!workspace) return fail(SOL_EWORKSPACE, "workspace is NULL (need %zu bytes)", w.total);
  if (!aligned16(workspace)) return fail(SOL_EINVAL, "workspace is not 16-byte aligned");
  if (workspace_bytes < w.total)
    return fail(SOL_EWORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, w.total);
  const int64_t BH = shape->B * shape->H;
  const int64_t M = n_blocks(shape->N, block);
  const int64_t Mp = padded_blocks(shape->N, block);
  if (overlaps(s_map, (size_t)(BH * M * shape->N) * sizeof(float), workspace, w.total))
    return fail(SOL_EINVAL, "s_map overlaps the workspace");
  unsigned char* ws = (unsigned char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const solattn::Strides cs = contiguous(*shape);
  hipError_t e = solattn::launch_pool((int)shape->d, BH, shape->N, block, k, k, cs,
                                      (float*)(ws + w.kbar), nullptr, (uint16_t*)(ws + w.kp),
                                      (uint16_t*)(ws + w.vbt), Mp, s);
  if (e != hipSuccess) return hip_status(e, "pool kernel launch");
  return hip_status(solattn::launch_proxy_map((int)shape->d, (const uint16_t*)q, cs,
                                              (const uint16_t*)(ws + w.kp), BH, shape->N, M, Mp,
                                              s_map, s),
                    "proxy map kernel launch");
}

namespace {
int route_select(const sol_shape* shape, int block, const float* s_map, int mode, int64_t k, float p,
                 uint32_t* mask, void* stream) {
  int st;
  if ((st = check_shape(shape)) || (st = check_block(block))) return st;
  if ((st = check_tensor(s_map, "s_map"))) return st;
  if (!mask) return fail(SOL_EINVAL, "mask is NULL");
  if ((uintptr_t)mask & 3u) return fail(SOL_EINVAL, "mask is not 4-byte aligned");
  if (mode == 1 && std::isnan(p)) return fail(SOL_EINVAL, "p is NaN");
  const int64_t BH = shape->B * shape->H;
  const int64_t M = n_blocks(shape->N, block);
  const int64_t W = (M + 31) / 32;
  if (M > solattn::route_max_blocks())
    return fail(SOL_EUNSUPPORTED, "selection supports at most %lld key blocks per row (got %lld)",
                (long long)solattn::route_max_blocks(), (long long)M);
  if (BH * shape->N > (int64_t)4 * 0x7fffffff)
    return fail(SOL_EUNSUPPORTED, "selection supports at most %lld rows in all", 4LL * 0x7fffffff);
  if (overlaps(mask, (size_t)(BH * shape->N * W) * 4, s_map, (size_t)(BH * M * shape->N) * 4))
    return fail(SOL_EINVAL, "mask overlaps s_map");
  return hip_status(solattn::launch_route_select(mode, s_map, BH, shape->N, M, block, k, p, mask,
                                                 (hipStream_t)stream),
                    "selection kernel launch");
}
}  // namespace

int sol_select_topk(const sol_shape* shape, int block, const float* s_map, int64_t k,
                    uint32_t* mask, void* stream) {
  return route_select(shape, block, s_map, 0, k, 0.f, mask, stream);
}

int sol_select_topp(const sol_shape* shape, int block, const float* s_map, float p, uint32_t* mask,
                    void* stream) {
  return route_select(shape, block, s_map, 1, 0, p, mask, stream);
}

int sol_attn_fwd_noalloc(const sol_shape* shape, const void* q, const void* k, const void* v,
                         float beta, int block, void* out, void* stream) {
  static_assert(SOL_NOALLOC_SCRATCH_BYTES == solattn::kNoAllocScratchBytes,
                "the header states the scratch size");
  int st;
  if ((st = check_shape(shape)) || (st = check_block(block))) return st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
      (st = check_tensor(out, "out")))
    return st;
  if (std::isnan(beta)) return fail(SOL_EINVAL, "beta is NaN");
  const size_t ext = extent_bytes(*shape, contiguous(*shape));
  if (overlaps(out, ext, q, ext) || overlaps(out, ext, k, ext) || overlaps(out, ext, v, ext))
    return fail(SOL_EINVAL, "out overlaps an input");
  // Heads are independent: run them in the largest groups whose workspace fits the scratch.
  const int64_t BH = shape->B * shape->H;
  const size_t cap = solattn::kNoAllocScratchBytes;
  auto need = [&](int64_t g) { return layout(sol_shape{1, g, shape->N, shape->d}, block).total; };
  if (need(1) > cap)
    return fail(SOL_EWORKSPACE,
                "one head needs %zu bytes of workspace; the allocation-free call holds %zu "
                "(use sol_attn_fwd with a caller workspace)", need(1), cap);
  int64_t G = (int64_t)(cap / need(1));
  if (G > BH) G = BH;
  while (G > 1 && need(G) > cap) --G;
  void* scratch = nullptr;
  hipError_t e = solattn::noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "scratch address lookup");
  const int64_t head_elems = shape->N * shape->d;
  for (int64_t h0 = 0; h0 < BH; h0 += G) {
    const int64_t g = BH - h0 < G ? BH - h0 : G;
    const sol_shape sub{1, g, shape->N, shape->d};
    const int64_t off = h0 * head_elems;
    st = attn_forward(&sub, nullptr, nullptr, (const uint16_t*)q + off, (const uint16_t*)k + off,
                      (const uint16_t*)v + off, beta, block, (uint16_t*)out + off, scratch, cap,
                      nullptr, nullptr, 0, stream);
    if (st != SOL_OK) return st;
  }
  return ok();
}

int sol_attn_fwd(const sol_shape* shape, const void* q, const void* k, const void* v, float beta,
                 int block, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return sol_attn_fwd_ex(shape, q, k, v, beta, block, out, workspace, workspace_bytes, nullptr,
                         stream);
}

int sol_dense_fwd_strided(const sol_shape* shape, const sol_strides* in_strides,
                          const sol_strides* out_strides, const void* q, const void* k,
                          const void* v, void* out, float* lse, void* stream) {
  int st;
  if ((st = check_shape(shape))) return st;
  if ((st = check_strides(*shape, in_strides, "input", false)) ||
      (st = check_strides(*shape, out_strides, "output", true)))
    return st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
      (st = check_tensor(out, "out")))
    return st;
  if (lse && ((uintptr_t)lse & 3u)) return fail(SOL_EINVAL, "lse not 4-byte aligned");
  const solattn::Strides ins = to_strides(*shape, in_strides), outs = to_strides(*shape, out_strides);
  const size_t ein = extent_bytes(*shape, ins), eout = extent_bytes(*shape, outs);
  if (overlaps(out, eout, q, ein) || overlaps(out, eout, k, ein) || overlaps(out, eout, v, ein))
    return fail(SOL_EINVAL, "out overlaps an input");
  return hip_status(solattn::launch_dense((int)shape->d, shape->B * shape->H, shape->N, q, k, v, ins,
                                          out, outs, lse, (hipStream_t)stream),
                    "dense attention kernel launch");
}

int sol_dense_fwd(const sol_shape* shape, const void* q, const void* k, const void* v, void* out,
                  float* lse, void* stream) {
  return sol_dense_fwd_strided(shape, nullptr, nullptr, q, k, v, out, lse, stream);
}

}  // extern "C"
