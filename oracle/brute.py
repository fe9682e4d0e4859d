"""Brute-force numpy references used to pin the C oracle.

TEST INFRASTRUCTURE ONLY (the checker, not the product).  These are whole-matrix numpy
formulas, independent of ``sol_oracle.c``: a mistake in the oracle's row loop does not reappear
here.  They cover the two limits of the method described on the page "Sol-Attn: Accelerating
Video Generation Inference via On-the-Fly Attention Sparsification"
(agihunt.info/papers/2607.24027), paragraph on the per-query threshold:
  * every block kept (beta = -inf): plain dense softmax attention;
  * no block kept (beta = +inf): attention over the pooled tokens alone, one per block, with
    logit q.mean(K_blk)/sqrt(d) + ln(n_blk) and value mean(V_blk).
"""
from __future__ import annotations

import numpy as np


def dense_attention(q, k, v):
    """softmax(q k^T / sqrt(d)) v in fp64, row-wise stable.  Returns (out [N, d], lse [N])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    logits = q @ k.T / np.sqrt(q.shape[1])
    mx = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - mx)
    den = w.sum(axis=1, keepdims=True)
    return (w @ v) / den, (mx + np.log(den))[:, 0]


def block_ranges(N: int, block: int):
    return [(lo, min(lo + block, N)) for lo in range(0, N, block)]


def pooled_attention(q, k, v, block: int):
    """Attention over pooled tokens only (every block unselected).

    Written as its closed form: O_i = sum_j n_j e^{s_ij} Vbar_j / sum_j n_j e^{s_ij}."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, d = k.shape
    rng = block_ranges(N, block)
    kbar = np.stack([k[a:b].mean(axis=0) for a, b in rng])
    vbar = np.stack([v[a:b].mean(axis=0) for a, b in rng])
    n = np.array([b - a for a, b in rng], np.float64)
    s = q @ kbar.T / np.sqrt(d)
    mx = s.max(axis=1, keepdims=True)
    w = n[None, :] * np.exp(s - mx)
    den = w.sum(axis=1, keepdims=True)
    return (w @ vbar) / den, (mx + np.log(den))[:, 0]


def proxy_scores(q, k, block: int):
    """Proxy row s_ij = mean over block j of the exact logits q_i.k/sqrt(d) (a different but
    equal-in-exact-arithmetic route from pooling K first)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    N, d = k.shape
    logits = q @ k.T / np.sqrt(d)
    return np.stack([logits[:, a:b].mean(axis=1) for a, b in block_ranges(N, block)], axis=1)


def sol_attention_masked(q, k, v, block: int, sel):
    """Sol-Attn output for a given selection sel [N, M] (bool), written as one masked softmax over
    the concatenation [exact logits of all N keys | one pooled logit per block], where exact
    logits of unselected blocks and pooled logits of selected blocks are removed with -inf."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, d = k.shape
    rng = block_ranges(N, block)
    M = len(rng)
    sel = np.asarray(sel, bool)
    exact = q @ k.T / np.sqrt(d)                                   # [Nq, N]
    kbar = np.stack([k[a:b].mean(axis=0) for a, b in rng])
    vbar = np.stack([v[a:b].mean(axis=0) for a, b in rng])
    n = np.array([b - a for a, b in rng], np.float64)
    pooled = q @ kbar.T / np.sqrt(d) + np.log(n)[None, :]          # [Nq, M]
    key_block = np.concatenate([np.full(b - a, j) for j, (a, b) in enumerate(rng)])
    exact = np.where(sel[:, key_block], exact, -np.inf)
    pooled = np.where(sel, -np.inf, pooled)
    logits = np.concatenate([exact, pooled], axis=1)
    values = np.concatenate([v, vbar], axis=0)
    mx = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - mx)
    den = w.sum(axis=1, keepdims=True)
    assert M == sel.shape[1]
    return (w @ values) / den, (mx + np.log(den))[:, 0]
