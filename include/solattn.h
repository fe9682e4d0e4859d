/*
 * solattn.h -- C ABI of libsolattn: the Sol-Attn sparse attention forward pass on gfx950.
 *
 * The method is the one summarised on the page "Sol-Attn: Accelerating Video Generation
 * Inference via On-the-Fly Attention Sparsification" (agihunt.info/papers/2607.24027):
 *   - each query i scores every key block j with a pre-softmax proxy (paragraph on routing);
 *   - the proxy row of query i gives a mean mu_i and a standard deviation sigma_i, and block j is
 *     kept when its score clears tau_i = mu_i + beta * sigma_i, one beta for all queries
 *     (paragraph on the per-query threshold);
 *   - kept blocks get exact attention, unselected blocks are approximated rather than dropped,
 *     all inside one online-softmax pass (paragraphs on the fused operator).
 * The page leaves the proxy and the approximation open; this library fixes them as
 *   proxy        s_ij = q_i . Kbar_j / sqrt(d),   Kbar_j = mean of the keys of block j;
 *   approximation: each unselected block enters the softmax as one pooled token with logit
 *                s_ij + ln(n_j) and value Vbar_j = mean of the values of block j (n_j = tokens);
 *   statistics   mu_i and sigma_i over all M blocks, sigma the population standard deviation;
 *   selection    kept iff s_ij >= tau_i; beta = -inf keeps all, +inf keeps none.
 * The attention is bidirectional (no causal mask) and forward only, as the page's limitations
 * paragraph states.
 *
 * Conventions shared by every call
 *   Layout    q, k, v, out: contiguous [B][H][N][d] bf16 (raw uint16 bit patterns), device memory.
 *   Blocks    key block j covers tokens [j*block, min((j+1)*block, N)); M = ceil(N / block).
 *   Scale     1/sqrt(d), fixed.
 *   Supported d in {64, 128}; block in {64, 128}; 1 <= N <= 2^22; 1 <= B*H <= 65535.
 *   Pointers  all tensor pointers are device pointers, 16-byte aligned, owned by the caller.
 *             The library never allocates or frees device memory and keeps no device state
 *             (apart from the fixed scratch array of sol_attn_fwd_noalloc, see there).
 *             out must not overlap q, k, v or the workspace.
 *   Streams   `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call only
 *             enqueues work on that stream and returns; nothing synchronises.  A fault inside a
 *             kernel surfaces at the caller's next synchronisation of the stream.
 *   Errors    calls return SOL_OK (0) or a negative sol_status.  Argument errors are detected
 *             before any HIP call is made (so they are testable without a GPU); the thread-local
 *             message from sol_last_error() says which argument.  A failed kernel launch returns
 *             SOL_EHIP.  No C++ exception crosses this interface.
 */
#ifndef SOLATTN_H
#define SOLATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sol_status {
  SOL_OK = 0,
  SOL_EINVAL = -1,        /* NULL/misaligned pointer, bad size, NaN beta */
  SOL_EUNSUPPORTED = -2,  /* d or block outside the supported set */
  SOL_EWORKSPACE = -3,    /* workspace NULL or smaller than sol_attn_workspace_bytes() */
  SOL_EHIP = -4,          /* the HIP runtime reported an error at launch */
  SOL_ENOTIMPL = -5       /* reserved: no call of this version returns it */
} sol_status;

/* Tensor extents: batch, heads, tokens, head dimension. */
typedef struct sol_shape {
  int64_t B, H, N, d;
} sol_shape;

/* Element strides of a [B][H][N][d] view whose d elements are contiguous: element (b, h, n, c)
 * is at ptr[b * b_stride + h * h_stride + n * n_stride + c].  The contiguous layout is
 * {H*N*d, N*d, d}; a transformer's [B][N][H][d] projection output is {N*H*d, d, H*d}; q, k, v
 * views into a packed [B][N][3][H][d] projection are {N*3*H*d, d, 3*H*d}.  Accepted strides are
 * non-negative multiples of 8 with n_stride >= d (n_stride <= 2^23); an output view must not map
 * two elements to one address. */
typedef struct sol_strides {
  int64_t b, h, n;
} sol_strides;

/* Query rows handled together by one tile of the fused kernel: 128 consecutive rows (or, with
 * sol_attn_fwd_grid at d = 128, eight 16-row segments of the latent grid).  A key block is
 * computed for a tile when any row of the tile keeps it (rows that do not keep it are masked
 * inside the tile). */
#define SOL_QUERY_TILE 128

/* Bytes of device workspace sol_attn_fwd needs for this shape and block size (0 on bad input).
 * Holds the pooled keys/values and their bf16 split copies, the pooled-key mean and covariance,
 * the per-row thresholds and the per-row selection words; contents are scratch between calls. */
size_t sol_attn_workspace_bytes(const sol_shape* shape, int block);

/*
 * K/V mean pooling: kbar[b][h][j][:] = (1/n_j) * sum of k[b][h][t][:] over the tokens t of block j,
 * and likewise vbar from v.  Sums in fp32, true division by n_j.
 *   k, v        [B][H][N][d] bf16, device.
 *   kbar, vbar  [B][H][M][d] fp32, device, written.
 * The proxy of the page's routing paragraph is the dot product of a query with kbar.
 */
int sol_pool_kv(const sol_shape* shape, const void* k, const void* v, int block, float* kbar,
                float* vbar, void* stream);

/*
 * Sol-Attn forward: out = the softmax over {exact keys of kept blocks} U {one pooled token per
 * unselected block}, per query row, as defined at the top of this header.
 *   q, k, v     [B][H][N][d] bf16, device.
 *   beta        global threshold offset; finite or +-infinity; NaN -> SOL_EINVAL.
 *   block       key block size (tokens per block).
 *   out         [B][H][N][d] bf16, device, written.
 *   workspace   device scratch of at least sol_attn_workspace_bytes(shape, block) bytes.
 */
int sol_attn_fwd(const sol_shape* shape, const void* q, const void* k, const void* v, float beta,
                 int block, void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Optional outputs of sol_attn_fwd_ex (every pointer may be NULL; device memory). */
typedef struct sol_attn_debug {
  uint32_t* mask;      /* [B][H][N][ceil(M/32)]: bit j%32 of word j/32 set iff query keeps block j */
  float* mu;           /* [B][H][N] row mean of the proxy scores */
  float* sigma;        /* [B][H][N] row population standard deviation */
  float* tau;          /* [B][H][N] threshold mu + beta*sigma (+-inf for infinite beta) */
  float* lse;          /* [B][H][N] natural log of the softmax denominator (with its max) */
  int32_t* tile_kept;  /* [B][H][ceil(N/SOL_QUERY_TILE)] key blocks kept by some row of each
                          contiguous 128-row query tile (the blocks the fused kernel computes for
                          that tile, unless a latent grid regroups the rows: sol_attn_fwd_grid) */
  float* out_f32;      /* [B][H][N][d] the output before its final rounding to bf16 (out is the
                          round-to-nearest-even bf16 of these values) */
  int drop_unselected; /* 0: the method.  1: ablation -- unselected blocks are dropped instead of
                          pooled (a row with nothing kept then outputs 0 and lse = -inf). */
  void* events[4];     /* hipEvent_t handles (each may be NULL), recorded on `stream` before the
                          pooling kernel, before the pooled-key statistics, before the fused
                          attention kernel and after it (so [2]..[3] brackets the fused kernel
                          alone): per-kernel timing without changing the work done. */
} sol_attn_debug;

/* sol_attn_fwd plus the optional outputs above (dbg may be NULL, then identical to sol_attn_fwd). */
int sol_attn_fwd_ex(const sol_shape* shape, const void* q, const void* k, const void* v,
                    float beta, int block, void* out, void* workspace, size_t workspace_bytes,
                    const sol_attn_debug* dbg, void* stream);

/* Latent grid of the tokens of a video DiT (the workloads of the page's results paragraph): T
 * frames of H x W latent positions, token n at frame t, row y, column x with
 * n = (t * H + y) * W + x. */
typedef struct sol_grid {
  int64_t T, H, W;
} sol_grid;

/*
 * sol_attn_fwd_ex with the tokens' latent grid.  The grid changes only how the fused kernel
 * groups query rows into workgroups, never what is computed: at d = 128 each workgroup takes
 * eight 16-query row segments from 2 frames x 4 latent rows at one horizontal position (a
 * workgroup at the bottom of a column continues in the next one), instead of 128 consecutive
 * rows.  Such
 * rows keep similar key blocks, so the union of blocks a workgroup copies and computes is
 * smaller.  Every row's selection, pooled tokens and exact blocks are the same as
 * sol_attn_fwd_ex's; results agree up to fp32 summation order.  The debug outputs keep their
 * meaning (tile_kept still counts the blocks kept by contiguous 128-row tiles).
 * With d = 64, or W not a multiple of 16, the rows keep the contiguous grouping.
 *   grid   T, H, W >= 1 and T * H * W == shape->N, else SOL_EINVAL.
 */
int sol_attn_fwd_grid(const sol_shape* shape, const sol_grid* grid, const void* q, const void* k,
                      const void* v, float beta, int block, void* out, void* workspace,
                      size_t workspace_bytes, const sol_attn_debug* dbg, void* stream);

/*
 * sol_attn_fwd on strided views (no transposes needed in a transformer block): q, k and v share
 * in_strides, out uses out_strides (either NULL = contiguous).  The workspace is as for
 * sol_attn_fwd.  SOL_EINVAL for strides outside the accepted set (see sol_strides) or an output
 * view that overlaps an input or the workspace; otherwise as sol_attn_fwd.
 */
int sol_attn_fwd_strided(const sol_shape* shape, const sol_strides* in_strides,
                         const sol_strides* out_strides, const void* q, const void* k,
                         const void* v, float beta, int block, void* out, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Dense reference attention: out = softmax(q k^T / sqrt(d)) v over all N keys, no mask
 * (bidirectional, as the page's limitations paragraph states).  The page measures Sol-Attn against
 * dense FlashAttention (paragraph on the results: the kernel-level speedup on H100 and the LTX
 * table); this is the library's own dense kernel in that role, and the speedup of the sparse pass
 * is measured against it on the same tensors.
 *   q, k, v, out  [B][H][N][d] bf16, device.   lse  [B][H][N] fp32, device, or NULL.
 */
int sol_dense_fwd(const sol_shape* shape, const void* q, const void* k, const void* v, void* out,
                  float* lse, void* stream);

/* sol_dense_fwd on strided views (strides as for sol_attn_fwd_strided). */
int sol_dense_fwd_strided(const sol_shape* shape, const sol_strides* in_strides,
                          const sol_strides* out_strides, const void* q, const void* k,
                          const void* v, void* out, float* lse, void* stream);

/*
 * Prior-art routing, for comparison (page above, paragraph on routing: top-k keeps a fixed number
 * of key blocks per query, top-p keeps blocks until their cumulative probability reaches a
 * threshold, and both need the full proxy map in memory before the sparse pass).  These calls
 * build that pipeline from the same proxy as sol_attn_fwd: map -> selection -> attention with the
 * caller's selection.
 *
 * sol_proxy_map: s_map[b][h][i][j] = q_i . Kbar_j / sqrt(d) for every query row i and key block j
 * (fp32, row-major: [B][H][N][M], B*H*N*M*4 bytes, device, written; the same fp32-accurate
 * values the fused kernel compares with tau).  Pools K into the workspace first (the workspace
 * of sol_attn_workspace_bytes(shape, block), contents scratch).  s_map must not overlap the
 * workspace.
 */
int sol_proxy_map(const sol_shape* shape, const void* q, const void* k, int block, float* s_map,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Top-k selection from s_map: for each row, the k blocks with the largest s_ij, equal scores
 * keeping the lower block index first.  k <= 0 keeps none, k >= M keeps all.
 *   mask  [B][H][N][ceil(M/32)] uint32, device, written (bit j%32 of word j/32 = block j kept).
 * A row's scores are held in registers: M <= 2048 (else SOL_EUNSUPPORTED).
 */
int sol_select_topk(const sol_shape* shape, int block, const float* s_map, int64_t k,
                    uint32_t* mask, void* stream);

/*
 * Top-p selection from s_map: the probability of block j in row i is its share of the softmax
 * over the row's pooled logits s_ij + ln n_j; blocks are taken in decreasing order of probability
 * (equal values: lower index first) and a block is kept while the probability of the blocks before
 * it is below p.  p <= 0 keeps none, p >= 1 keeps all, NaN -> SOL_EINVAL.  Sums in fp32: a row
 * whose cumulative probability passes within rounding of p at a block may decide that block
 * either way.  mask as for sol_select_topk.
 */
int sol_select_topp(const sol_shape* shape, int block, const float* s_map, float p,
                    uint32_t* mask, void* stream);

/*
 * sol_attn_fwd with the caller's selection instead of the threshold: block j is computed exactly
 * for row i iff bit j of mask[b][h][i] is set ([B][H][N][ceil(M/32)] uint32, device, read; bits
 * at or beyond M are ignored).  Unselected blocks enter as pooled tokens, or are dropped when
 * drop_unselected is non-zero (a row with nothing kept then outputs 0).  No row statistics are
 * computed.  Other arguments and errors as for sol_attn_fwd.
 */
int sol_attn_fwd_masked(const sol_shape* shape, const void* q, const void* k, const void* v,
                        const uint32_t* mask, int block, int drop_unselected, void* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * sol_attn_fwd without a caller workspace, for callers that cannot allocate device memory (code
 * under stream capture, tight serving loops, harnesses that forbid allocation).  Arguments,
 * result and errors as for sol_attn_fwd; q, k, v, out contiguous [B][H][N][d] bf16, owned by the
 * caller.  The workspace is a library-owned device array of SOL_NOALLOC_SCRATCH_BYTES per GPU,
 * reserved when the library's kernels are loaded on that GPU and held until the process ends; the
 * call itself allocates and frees nothing.  Heads are independent, so they run in the largest
 * groups whose workspace (sol_attn_workspace_bytes for those heads) fits the array, one group
 * after another on `stream`; the output is that of sol_attn_fwd up to the order in which a row's
 * kept blocks are summed.  SOL_EWORKSPACE when a single head needs more than the array holds
 * (sol_attn_workspace_bytes of a one-head shape); nothing is launched then.
 * Every call on one GPU shares that GPU's array (each kernel writes what it later reads, so no
 * contents carry over from a previous call): calls that may overlap in time on one GPU -- on
 * different streams, or from several threads -- race and must be serialised by the caller.
 */
#define SOL_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int sol_attn_fwd_noalloc(const sol_shape* shape, const void* q, const void* k, const void* v,
                         float beta, int block, void* out, void* stream);

/*
 * Matrix-core rate probe (measurement only, not part of the attention path): `workgroups`
 * workgroups of 4 waves each issue iters x 8 independent bf16 32x32x16 MFMAs (32768 FLOPs each)
 * on register operands, so FLOPs = workgroups * 4 * iters * 8 * 32768.  sink (device,
 * [workgroups] fp32, written) receives one value per workgroup so that no work is optimised away.
 * Timed by the caller (e.g. with events on `stream`), it gives the bf16 MFMA rate this part
 * sustains, against which the attention kernels' rates are also reported.
 * Errors: SOL_EINVAL for workgroups < 1, iters < 1 or a NULL sink; SOL_EHIP if the launch fails.
 */
int sol_mfma_probe(int workgroups, int iters, float* sink, void* stream);

/* Static text for a status code. */
const char* sol_status_str(int status);
/* Message for the last error returned on the calling thread ("" if none). */
const char* sol_last_error(void);
/* Library version string. */
const char* sol_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SOLATTN_H */
