/*
 * sol_oracle.c -- plain fp64 CPU oracle for the Sol-Attn sparse attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg load it.  It shares no code, header,
 * table or helper with the GPU library, and the GPU library never calls it.
 *
 * Source of the method: the page "Sol-Attn: Accelerating Video Generation Inference via
 * On-the-Fly Attention Sparsification" (agihunt.info/papers/2607.24027), a summary of the paper.
 *   [routing]   paragraph on the weaknesses of top-k / top-p routing: a pre-softmax proxy score per
 *               (query, key block); dropping unselected blocks costs accuracy.
 *   [observe]   paragraph on the observation: each query's proxy-score row is close to normal.
 *   [threshold] paragraph on the per-query threshold tau_i = mu_i + beta*sigma_i over that row,
 *               with one global beta.
 *   [fusion]    paragraphs on the fused operator: routing, exact sparse compute and an
 *               approximate correction for the unselected blocks inside one online softmax.
 * The page fixes neither the proxy nor the correction term.  The readings used here:
 *   proxy       s_ij = q_i . mean(K over block j) / sqrt(d)
 *   correction  each unselected block j enters the softmax as ONE pooled token with
 *               logit s_ij + ln(n_j) and value mean(V over block j), n_j = tokens in block j.
 *   statistics  mu_i = mean over all M blocks, sigma_i = population standard deviation.
 *   selection   block j is kept for query i iff s_ij >= tau_i (ties keep the block).
 *   beta        -inf keeps every block, +inf keeps none (even when sigma_i = 0); NaN is an error.
 *   blocks      contiguous runs of the flattened token order; the last block may be partial.
 *
 * Parity unpinned: whether this pooled-token form is the paper's own correction term.  The page
 * does not print that term, so no value on it can pin the choice; every other function here is
 * pinned by the tests (hand examples, limits, special cases and invariants).
 *
 * Everything is fp64.  Inputs are fp32 arrays that hold bf16 values exactly.  The code follows
 * the definition step by step, one query row at a time, with no blocking, fusion or reordering.
 * OpenMP splits rows across threads; each row is computed independently in a fixed order, so the
 * results do not depend on the thread count.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

/* Number of key blocks and the token range [lo, hi) of block j: contiguous runs of `block`
 * tokens in the flattened order; the last run holds the remainder. */
static int64_t n_blocks(int64_t N, int block) { return (N + block - 1) / block; }
static int64_t block_lo(int64_t j, int block) { return j * (int64_t)block; }
static int64_t block_hi(int64_t j, int64_t N, int block) {
  int64_t hi = (j + 1) * (int64_t)block;
  return hi < N ? hi : N;
}

/* Mean of each block of rows of x ([N][d]): xbar[j][c] = (1/n_j) * sum_{k in block j} x[k][c].
 * This is the pooled key (or value) of block j used by the proxy and by the pooled token. */
int sol_oracle_pool(const float* x, int64_t N, int d, int block, double* xbar) {
  if (!x || !xbar || N < 1 || d < 1 || block < 1) return ORACLE_EINVAL;
  int64_t M = n_blocks(N, block);
  for (int64_t j = 0; j < M; ++j) {
    int64_t lo = block_lo(j, block), hi = block_hi(j, N, block);
    double n = (double)(hi - lo);
    for (int c = 0; c < d; ++c) {
      double sum = 0.0;
      for (int64_t k = lo; k < hi; ++k) sum += (double)x[k * d + c];
      xbar[j * d + c] = sum / n;
    }
  }
  return ORACLE_OK;
}

static double dot(const float* a, const double* b, int d) {
  double acc = 0.0;
  for (int c = 0; c < d; ++c) acc += (double)a[c] * b[c];
  return acc;
}

static double dotf(const float* a, const float* b, int d) {
  double acc = 0.0;
  for (int c = 0; c < d; ++c) acc += (double)a[c] * (double)b[c];
  return acc;
}

/*
 * One attention head, a chosen set of query rows.
 *
 *   q, k, v        [N][d] fp32 (bf16 values), row-major, one (batch, head) slice.
 *   beta           the global threshold offset; +-INFINITY allowed, NaN rejected.
 *   rows           nrows query indices in [0, N).
 *   mask_override  NULL, or [nrows][W] words (W = ceil(M/32), bit j%32 of word j/32 = block j kept)
 *                  that replace the threshold selection; mu/sigma/tau are still computed.
 *   drop           0: unselected blocks enter as pooled tokens (the method).
 *                  1: unselected blocks are dropped (ablation).  A row with nothing kept then has
 *                     no logits; its output and lse are set to NaN.
 * Outputs (any may be NULL except out):
 *   out   [nrows][d]  attention output;       lse  [nrows]  log of the softmax denominator + max;
 *   mu, sigma, tau [nrows];  mask [nrows][W] selection bits;  s [nrows][M] proxy scores.
 */
int sol_oracle_rows(const float* q, const float* k, const float* v, int64_t N, int d, int block,
                    double beta, const int64_t* rows, int64_t nrows,
                    const uint32_t* mask_override, int drop, double* out, double* lse, double* mu,
                    double* sigma, double* tau, uint32_t* mask, double* s_out) {
  if (!q || !k || !v || !rows || !out || N < 1 || d < 1 || block < 1 || nrows < 0) return ORACLE_EINVAL;
  if (isnan(beta)) return ORACLE_EINVAL;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return ORACLE_EINVAL;

  const int64_t M = n_blocks(N, block);
  const int64_t W = (M + 31) / 32;
  const double inv_sqrt_d = 1.0 / sqrt((double)d);

  /* Pooled keys and values of every block (the proxy's keys, the pooled tokens' values). */
  double* kbar = (double*)malloc(sizeof(double) * (size_t)(M * d));
  double* vbar = (double*)malloc(sizeof(double) * (size_t)(M * d));
  if (!kbar || !vbar) { free(kbar); free(vbar); return ORACLE_ENOMEM; }
  sol_oracle_pool(k, N, d, block, kbar);
  sol_oracle_pool(v, N, d, block, vbar);

  int status = ORACLE_OK;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)M);
    unsigned char* sel = (unsigned char*)malloc((size_t)M);
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
    if (!s || !sel || !acc) {
#pragma omp atomic write
      status = ORACLE_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows[r];
        const float* qi = q + i * d;

        /* Step 1: proxy score of every block, s_ij = q_i . Kbar_j / sqrt(d). */
        for (int64_t j = 0; j < M; ++j) s[j] = dot(qi, kbar + j * d, d) * inv_sqrt_d;

        /* Step 2: row statistics, two passes: mean, then population standard deviation. */
        double m1 = 0.0;
        for (int64_t j = 0; j < M; ++j) m1 += s[j];
        m1 /= (double)M;
        double m2 = 0.0;
        for (int64_t j = 0; j < M; ++j) m2 += (s[j] - m1) * (s[j] - m1);
        double sd = sqrt(m2 / (double)M);

        /* Step 3: the per-query threshold tau_i = mu_i + beta * sigma_i. */
        double t;
        if (isinf(beta)) t = beta;  /* -inf keeps all, +inf keeps none, whatever sigma is */
        else t = m1 + beta * sd;

        /* Step 4: selection, s_ij >= tau_i, unless an explicit mask is supplied. */
        for (int64_t j = 0; j < M; ++j) {
          if (mask_override) sel[j] = (mask_override[r * W + j / 32] >> (j % 32)) & 1u;
          else sel[j] = s[j] >= t;
        }

        /* Step 5: the logit multiset.  Exact tokens of kept blocks; one pooled token per
         * unselected block (unless dropped).  First pass: the maximum logit. */
        double mx = -INFINITY;
        for (int64_t j = 0; j < M; ++j) {
          int64_t lo = block_lo(j, block), hi = block_hi(j, N, block);
          if (sel[j]) {
            for (int64_t kk = lo; kk < hi; ++kk) {
              double l = dotf(qi, k + kk * d, d) * inv_sqrt_d;
              if (l > mx) mx = l;
            }
          } else if (!drop) {
            double l = s[j] + log((double)(hi - lo));
            if (l > mx) mx = l;
          }
        }

        /* Step 6: softmax over the multiset and the weighted sum of values. */
        double den = 0.0;
        for (int c = 0; c < d; ++c) acc[c] = 0.0;
        for (int64_t j = 0; j < M; ++j) {
          int64_t lo = block_lo(j, block), hi = block_hi(j, N, block);
          if (sel[j]) {
            for (int64_t kk = lo; kk < hi; ++kk) {
              double w = exp(dotf(qi, k + kk * d, d) * inv_sqrt_d - mx);
              den += w;
              for (int c = 0; c < d; ++c) acc[c] += w * (double)v[kk * d + c];
            }
          } else if (!drop) {
            double w = exp(s[j] + log((double)(hi - lo)) - mx);
            den += w;
            for (int c = 0; c < d; ++c) acc[c] += w * vbar[j * d + c];
          }
        }
        for (int c = 0; c < d; ++c) out[r * d + c] = den > 0.0 ? acc[c] / den : NAN;
        if (lse) lse[r] = den > 0.0 ? mx + log(den) : NAN;
        if (mu) mu[r] = m1;
        if (sigma) sigma[r] = sd;
        if (tau) tau[r] = t;
        if (mask) {
          for (int64_t w = 0; w < W; ++w) mask[r * W + w] = 0u;
          for (int64_t j = 0; j < M; ++j)
            if (sel[j]) mask[r * W + j / 32] |= 1u << (j % 32);
        }
        if (s_out)
          for (int64_t j = 0; j < M; ++j) s_out[r * M + j] = s[j];
      }
    }
    free(s);
    free(sel);
    free(acc);
  }
  free(kbar);
  free(vbar);
  return status;
}

/*
 * Selection only, for every row of one head: the proxy, the row statistics, the threshold and
 * the selection bits (steps 1-4 above), without the attention itself.  Used to check the full
 * selection mask at sizes where the attention part would take too long.
 *   mask [N][W]; mu, sigma, tau [N] (nullable); mindist [N] (nullable): min_j |s_ij - tau_i|.
 */
int sol_oracle_select(const float* q, const float* k, int64_t N, int d, int block, double beta,
                      uint32_t* mask, double* mu, double* sigma, double* tau, double* mindist) {
  if (!q || !k || !mask || N < 1 || d < 1 || block < 1 || isnan(beta)) return ORACLE_EINVAL;
  const int64_t M = n_blocks(N, block);
  const int64_t W = (M + 31) / 32;
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  double* kbar = (double*)malloc(sizeof(double) * (size_t)(M * d));
  if (!kbar) return ORACLE_ENOMEM;
  sol_oracle_pool(k, N, d, block, kbar);
  int status = ORACLE_OK;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)M);
    if (!s) {
#pragma omp atomic write
      status = ORACLE_ENOMEM;
    } else {
#pragma omp for schedule(static)
      for (int64_t i = 0; i < N; ++i) {
        const float* qi = q + i * d;
        for (int64_t j = 0; j < M; ++j) s[j] = dot(qi, kbar + j * d, d) * inv_sqrt_d;
        double m1 = 0.0;
        for (int64_t j = 0; j < M; ++j) m1 += s[j];
        m1 /= (double)M;
        double m2 = 0.0;
        for (int64_t j = 0; j < M; ++j) m2 += (s[j] - m1) * (s[j] - m1);
        double sd = sqrt(m2 / (double)M);
        double t = isinf(beta) ? beta : m1 + beta * sd;
        double md = INFINITY;
        for (int64_t w = 0; w < W; ++w) mask[i * W + w] = 0u;
        for (int64_t j = 0; j < M; ++j) {
          if (s[j] >= t) mask[i * W + j / 32] |= 1u << (j % 32);
          double dist = fabs(s[j] - t);
          if (dist < md) md = dist;
        }
        if (mu) mu[i] = m1;
        if (sigma) sigma[i] = sd;
        if (tau) tau[i] = t;
        if (mindist) mindist[i] = md;
      }
    }
    free(s);
  }
  free(kbar);
  return status;
}

/* Plain dense softmax attention for chosen rows (no routing at all): the reference for the
 * dense kernel.  out [nrows][d], lse [nrows] (nullable). */
int sol_oracle_dense_rows(const float* q, const float* k, const float* v, int64_t N, int d,
                          const int64_t* rows, int64_t nrows, double* out, double* lse) {
  if (!q || !k || !v || !rows || !out || N < 1 || d < 1 || nrows < 0) return ORACLE_EINVAL;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return ORACLE_EINVAL;
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  int status = ORACLE_OK;
#pragma omp parallel
  {
    double* l = (double*)malloc(sizeof(double) * (size_t)N);
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
    if (!l || !acc) {
#pragma omp atomic write
      status = ORACLE_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < nrows; ++r) {
        const float* qi = q + rows[r] * d;
        double mx = -INFINITY;
        for (int64_t kk = 0; kk < N; ++kk) {
          l[kk] = dotf(qi, k + kk * d, d) * inv_sqrt_d;
          if (l[kk] > mx) mx = l[kk];
        }
        double den = 0.0;
        for (int c = 0; c < d; ++c) acc[c] = 0.0;
        for (int64_t kk = 0; kk < N; ++kk) {
          double w = exp(l[kk] - mx);
          den += w;
          for (int c = 0; c < d; ++c) acc[c] += w * (double)v[kk * d + c];
        }
        for (int c = 0; c < d; ++c) out[r * d + c] = acc[c] / den;
        if (lse) lse[r] = mx + log(den);
      }
    }
    free(l);
    free(acc);
  }
  return status;
}

/*
 * Prior-art routing on the same proxy, for comparison ([routing] paragraph: top-k keeps a fixed
 * number of blocks per query, top-p keeps blocks until their cumulative probability reaches a
 * threshold; both need the whole proxy map first).  For every row of one head:
 *   top-k (mode 0, param = k): keep the k blocks with the largest s_ij; among equal scores the
 *     lower block index comes first.  k <= 0 keeps none, k >= M keeps all.
 *   top-p (mode 1, param = p): the probability of block j is its share of the softmax over the
 *     row's pooled logits, pi_j = exp(s_ij + ln n_j) / sum_l exp(s_il + ln n_l).  Blocks are taken
 *     in decreasing order of pi (equal values: lower index first) and block j is kept when the
 *     probability of the blocks before it is still below p.  p <= 0 keeps none, p >= 1 keeps all.
 * Outputs: mask [N][W]; gap [N] (nullable): the score gap between the last kept block and the
 * next one in the order (+inf if there is none), and, for top-p, massgap [N] (nullable): the
 * smallest |cumulative probability before a block - p| over the row -- both measure how close the
 * row's selection is to changing under rounding.
 */
typedef struct {
  double key;
  int64_t j;
} route_item;

static int route_cmp(const void* a, const void* b) {
  const route_item* x = (const route_item*)a;
  const route_item* y = (const route_item*)b;
  if (x->key > y->key) return -1;
  if (x->key < y->key) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

int sol_oracle_route(const float* q, const float* k, int64_t N, int d, int block, int mode,
                     double param, uint32_t* mask, double* gap, double* massgap) {
  if (!q || !k || !mask || N < 1 || d < 1 || block < 1 || (mode != 0 && mode != 1) || isnan(param))
    return ORACLE_EINVAL;
  const int64_t M = n_blocks(N, block);
  const int64_t W = (M + 31) / 32;
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  double* kbar = (double*)malloc(sizeof(double) * (size_t)(M * d));
  if (!kbar) return ORACLE_ENOMEM;
  sol_oracle_pool(k, N, d, block, kbar);
  int status = ORACLE_OK;
#pragma omp parallel
  {
    route_item* it = (route_item*)malloc(sizeof(route_item) * (size_t)M);
    double* w = (double*)malloc(sizeof(double) * (size_t)M);
    if (!it || !w) {
#pragma omp atomic write
      status = ORACLE_ENOMEM;
    } else {
#pragma omp for schedule(static)
      for (int64_t i = 0; i < N; ++i) {
        const float* qi = q + i * d;
        /* the proxy of every block; for top-p the ordering key is the pooled logit s + ln n */
        for (int64_t j = 0; j < M; ++j) {
          double sj = dot(qi, kbar + j * d, d) * inv_sqrt_d;
          if (mode == 1) sj += log((double)(block_hi(j, N, block) - block_lo(j, block)));
          it[j].key = sj;
          it[j].j = j;
        }
        qsort(it, (size_t)M, sizeof(route_item), route_cmp);
        for (int64_t x = 0; x < W; ++x) mask[i * W + x] = 0u;
        int64_t kept = 0;
        double mg = INFINITY;
        if (mode == 0) {
          kept = param <= 0.0 ? 0 : (param >= (double)M ? M : (int64_t)param);
        } else if (param >= 1.0) {
          kept = M;
        } else if (param > 0.0) {
          /* probabilities in the sorted order; the first key is the row maximum */
          double z = 0.0;
          for (int64_t r = 0; r < M; ++r) {
            w[r] = exp(it[r].key - it[0].key);
            z += w[r];
          }
          double before = 0.0;
          for (int64_t r = 0; r < M; ++r) {
            double frac = before / z;
            double dist = fabs(frac - param);
            if (dist < mg) mg = dist;
            if (frac < param) kept = r + 1;
            before += w[r];
          }
        }
        for (int64_t r = 0; r < kept; ++r) mask[i * W + it[r].j / 32] |= 1u << (it[r].j % 32);
        if (gap) gap[i] = (kept > 0 && kept < M) ? it[kept - 1].key - it[kept].key : INFINITY;
        if (massgap) massgap[i] = mg;
      }
    }
    free(it);
    free(w);
  }
  free(kbar);
  return status;
}

/* Threads the OpenMP loops above use (for reporting the CPU baseline's core count). */
int sol_oracle_threads(void) { return omp_get_max_threads(); }
