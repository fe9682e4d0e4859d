"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each pin takes the loaded oracle library and raises AssertionError on a mismatch.  They are
collected by test_oracle.py (the real oracle must pass all of them) and by
test_oracle_mutants.py (each planted mistake must fail at least one of them).

What pins what (method: the page "Sol-Attn: Accelerating Video Generation Inference via
On-the-Fly Attention Sparsification", agihunt.info/papers/2607.24027):
  * hand examples (tests/golden/hand_examples.json): closed forms worked out by hand, including
    exact ties (keep iff s >= tau), population sigma and a partial last block (ln n_j, 1/n_j);
  * beta = -inf equals dense softmax attention, beta = +inf equals attention over pooled tokens
    only -- both numpy brute force (oracle/brute.py), with ragged last blocks;
  * finite beta equals a whole-matrix masked softmax (brute) under the oracle's selection, and the
    selection equals thresholding brute-force proxy rows (mean of exact logits per block);
  * special cases: block-constant K or block size 1 make every beta dense; q = 0 gives the mean of
    V; two blocks select by the sign pattern of beta;
  * invariances: shifting all keys, shifting all values, scaling a query, permuting tokens within
    a block, whole blocks, or queries; density non-increasing in beta; Jensen's bound
    s_ij + ln n_j <= logsumexp of the block's exact logits; outputs inside the value hull.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import brute, oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")
INF = float("inf")


def _beta(b):
    return {"inf": INF, "-inf": -INF}.get(b, b) if isinstance(b, str) else float(b)


def _bf16ish(rng, shape, scale=1.0):
    """Random values with <= 8 significant bits (exactly representable in bf16 and fp32)."""
    x = rng.standard_normal(shape) * scale
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    return (np.round(x / 2.0 ** (e - 7)) * 2.0 ** (e - 7)).astype(np.float32)


def _rand(seed, N=37, d=8, scale=1.0):
    rng = np.random.default_rng(seed)
    return (_bf16ish(rng, (N, d), scale), _bf16ish(rng, (N, d), scale), _bf16ish(rng, (N, d), scale))


def pin_hand_example1(lib):
    g = json.load(open(GOLDEN))["example1"]
    q, k, v = (np.array(g[x], np.float32) for x in ("q", "k", "v"))
    for c in g["cases"]:
        r = oracle.attn_rows(q, k, v, _beta(c["beta"]), g["block"], rows=[0], lib=lib)
        keep = oracle.mask_bits(r["mask"], 2)[0].astype(int).tolist()
        assert keep == c["keep"], (c, keep)
        assert abs(r["out"][0, 0] - c["out"]) < 1e-12, (c, r["out"])
        assert abs(r["mu"][0] - g["mu"]) < 1e-15 and abs(r["sigma"][0] - g["sigma"]) < 1e-15


def pin_hand_example2(lib):
    g = json.load(open(GOLDEN))["example2"]
    k, v = np.array(g["k"], np.float32), np.array(g["v"], np.float32)
    q = np.tile(np.array(g["q_row"], np.float32), (g["N"], 1))
    for c in g["cases"]:
        r = oracle.attn_rows(q, k, v, _beta(c["beta"]), g["block"], rows=[0], want_s=True, lib=lib)
        keep = oracle.mask_bits(r["mask"], 3)[0].astype(int).tolist()
        assert keep == c["keep"], (c, keep)
        assert np.abs(r["out"][0] - np.array(c["out"])).max() < 1e-12, (c, r["out"])
        assert abs(r["lse"][0] - c["lse"]) < 1e-12, (c, r["lse"])
        assert np.abs(r["s"][0] - np.array(g["s"])).max() < 1e-15
        assert abs(r["sigma"][0] - g["sigma"]) < 1e-14


def pin_dense_limit(lib):
    for seed, (N, d, b) in enumerate([(37, 8, 5), (64, 16, 16), (50, 4, 7)]):
        q, k, v = _rand(seed, N, d)
        ref, lse = brute.dense_attention(q, k, v)
        r = oracle.attn_rows(q, k, v, -INF, b, lib=lib)
        assert np.abs(r["out"] - ref).max() < 1e-12
        assert np.abs(r["lse"] - lse).max() < 1e-12
        assert oracle.mask_bits(r["mask"], oracle.n_blocks(N, b)).all()
        dr = oracle.dense_rows(q, k, v, lib=lib)
        assert np.abs(dr["out"] - ref).max() < 1e-12 and np.abs(dr["lse"] - lse).max() < 1e-12


def pin_pooled_limit(lib):
    for seed, (N, d, b) in enumerate([(37, 8, 5), (64, 16, 16), (50, 4, 7)]):
        q, k, v = _rand(100 + seed, N, d)
        ref, lse = brute.pooled_attention(q, k, v, b)
        r = oracle.attn_rows(q, k, v, INF, b, lib=lib)
        assert np.abs(r["out"] - ref).max() < 1e-12
        assert np.abs(r["lse"] - lse).max() < 1e-12
        assert not oracle.mask_bits(r["mask"], oracle.n_blocks(N, b)).any()


def pin_finite_beta_masked_softmax(lib):
    for seed, (N, d, b, beta) in enumerate([(37, 8, 5, 0.3), (96, 16, 16, 0.8), (50, 4, 7, -0.2),
                                            (200, 8, 9, 1.2)]):
        q, k, v = _rand(200 + seed, N, d, scale=1.5)
        M = oracle.n_blocks(N, b)
        r = oracle.attn_rows(q, k, v, beta, b, want_s=True, lib=lib)
        sel = oracle.mask_bits(r["mask"], M)
        # selection against brute-force proxies and numpy statistics
        s = brute.proxy_scores(q, k, b)
        mu, sd = s.mean(axis=1), s.std(axis=1)
        assert np.abs(r["s"] - s).max() < 1e-12
        assert np.abs(r["mu"] - mu).max() < 1e-12 and np.abs(r["sigma"] - sd).max() < 1e-12
        tau = mu + beta * sd
        clear = np.abs(s - tau[:, None]) > 1e-9
        assert (sel[clear] == (s >= tau[:, None])[clear]).all()
        assert 0 < sel.sum() < sel.size, "case should be genuinely sparse"
        ref, lse = brute.sol_attention_masked(q, k, v, b, sel)
        assert np.abs(r["out"] - ref).max() < 1e-12
        assert np.abs(r["lse"] - lse).max() < 1e-12
        # an explicit mask reproduces the same numbers
        r2 = oracle.attn_rows(q, k, v, beta, b, mask_override=r["mask"], lib=lib)
        assert np.array_equal(r2["out"], r["out"])


def pin_mask_override(lib):
    q, k, v = _rand(300, 40, 8)
    b, M = 6, oracle.n_blocks(40, 6)
    rng = np.random.default_rng(1)
    sel = rng.random((40, M)) < 0.4
    r = oracle.attn_rows(q, k, v, 0.0, b, mask_override=oracle.pack_bits(sel), lib=lib)
    ref, lse = brute.sol_attention_masked(q, k, v, b, sel)
    assert np.abs(r["out"] - ref).max() < 1e-12
    assert np.array_equal(oracle.mask_bits(r["mask"], M), sel)


def pin_block_constant_keys(lib):
    rng = np.random.default_rng(400)
    N, d, b = 45, 8, 6
    kb = _bf16ish(rng, (oracle.n_blocks(N, b), d))
    k = np.repeat(kb, b, axis=0)[:N]
    q, _, v = _rand(401, N, d)
    ref, _ = brute.dense_attention(q, k, v)
    for beta in (-INF, -1.0, 0.0, 0.7, 2.0, INF):
        r = oracle.attn_rows(q, k, v, beta, b, lib=lib)
        assert np.abs(r["out"] - ref).max() < 1e-12, beta


def pin_block_size_one(lib):
    q, k, v = _rand(500, 30, 8)
    ref, _ = brute.dense_attention(q, k, v)
    for beta in (-1.0, 0.0, 0.5, 3.0, INF):
        r = oracle.attn_rows(q, k, v, beta, 1, lib=lib)
        assert np.abs(r["out"] - ref).max() < 1e-12, beta


def pin_zero_query(lib):
    q, k, v = _rand(600, 33, 8)
    q[5] = 0.0
    for beta in (-0.5, 0.0, 1.3):
        r = oracle.attn_rows(q, k, v, beta, 4, rows=[5], lib=lib)
        assert r["sigma"][0] == 0.0
        assert oracle.mask_bits(r["mask"], 9)[0].all()
        assert np.abs(r["out"][0] - v.astype(np.float64).mean(axis=0)).max() < 1e-12
    r = oracle.attn_rows(q, k, v, INF, 4, rows=[5], lib=lib)
    assert not oracle.mask_bits(r["mask"], 9)[0].any()


def pin_two_blocks(lib):
    q, k, v = _rand(700, 16, 8)
    r0 = oracle.attn_rows(q, k, v, 0.0, 8, want_s=True, lib=lib)
    s = r0["s"]
    hi = (s[:, 0] >= s[:, 1]).astype(int)
    for beta, expect in ((-1.5, "both"), (-0.5, "max"), (0.5, "max"), (1.5, "none")):
        r = oracle.attn_rows(q, k, v, beta, 8, lib=lib)
        sel = oracle.mask_bits(r["mask"], 2).astype(int)
        neq = s[:, 0] != s[:, 1]
        if expect == "both":
            assert sel[neq].all()
        elif expect == "none":
            assert not sel[neq].any()
        else:
            assert (sel[neq, 0] == hi[neq]).all() and (sel[neq, 1] == 1 - hi[neq]).all()


def pin_invariances(lib):
    N, d, b, beta = 48, 8, 6, 0.4
    q, k, v = _rand(800, N, d)
    base = oracle.attn_rows(q, k, v, beta, b, lib=lib)
    sel0 = base["mask"]
    rng = np.random.default_rng(801)
    # shifting every key by one vector shifts each row's logits by a constant
    u = np.round(rng.standard_normal(d) * 4) / 4
    r = oracle.attn_rows(q, (k + u).astype(np.float32), v, beta, b, lib=lib)
    assert np.array_equal(r["mask"], sel0) and np.abs(r["out"] - base["out"]).max() < 1e-10
    # shifting every value shifts the output
    w = np.round(rng.standard_normal(d) * 4) / 4
    r = oracle.attn_rows(q, k, (v + w).astype(np.float32), beta, b, lib=lib)
    assert np.abs(r["out"] - (base["out"] + w)).max() < 1e-10
    # scaling a query by c > 0 scales its proxy row: selection unchanged
    r = oracle.attn_rows((q * 4.0).astype(np.float32), k, v, beta, b, lib=lib)
    assert np.array_equal(r["mask"], sel0)
    # permuting tokens inside each block changes nothing
    perm = np.concatenate([lo + rng.permutation(hi - lo) for lo, hi in brute.block_ranges(N, b)])
    r = oracle.attn_rows(q, k[perm], v[perm], beta, b, lib=lib)
    assert np.array_equal(r["mask"], sel0) and np.abs(r["out"] - base["out"]).max() < 1e-12
    # permuting whole (full) blocks permutes the selection bits, output unchanged
    M = N // b
    bp = rng.permutation(M)
    tok = np.concatenate([np.arange(j * b, (j + 1) * b) for j in bp])
    r = oracle.attn_rows(q, k[tok], v[tok], beta, b, lib=lib)
    sel_a = oracle.mask_bits(sel0, M)
    sel_b = oracle.mask_bits(r["mask"], M)
    assert np.array_equal(sel_b, sel_a[:, bp]) and np.abs(r["out"] - base["out"]).max() < 1e-12
    # permuting queries permutes rows
    qp = rng.permutation(N)
    r = oracle.attn_rows(q[qp], k, v, beta, b, lib=lib)
    assert np.abs(r["out"] - base["out"][qp]).max() < 1e-15


def pin_density_monotone(lib):
    q, k, v = _rand(900, 80, 8, scale=1.3)
    M = oracle.n_blocks(80, 7)
    prev = None
    for beta in (-INF, -2.0, -1.0, -0.3, 0.0, 0.4, 1.0, 1.7, 3.0, INF):
        sel = oracle.mask_bits(oracle.attn_rows(q, k, v, beta, 7, lib=lib)["mask"], M)
        if prev is not None:
            assert not (sel & ~prev).any(), "raising beta may only remove blocks"
        prev = sel


def pin_jensen_and_hull(lib):
    N, d, b = 60, 8, 7
    q, k, v = _rand(1000, N, d, scale=1.4)
    r = oracle.attn_rows(q, k, v, 0.5, b, want_s=True, lib=lib)
    logits = q.astype(np.float64) @ k.T.astype(np.float64) / math.sqrt(d)
    for j, (lo, hi) in enumerate(brute.block_ranges(N, b)):
        blk = logits[:, lo:hi]
        mx = blk.max(axis=1)
        lse = mx + np.log(np.exp(blk - mx[:, None]).sum(axis=1))
        assert (r["s"][:, j] + math.log(hi - lo) <= lse + 1e-12).all()
    vmin, vmax = v.min(axis=0), v.max(axis=0)
    assert (r["out"] >= vmin - 1e-12).all() and (r["out"] <= vmax + 1e-12).all()


def pin_pool(lib):
    rng = np.random.default_rng(1100)
    x = _bf16ish(rng, (53, 8))
    for b in (1, 5, 8, 53, 64):
        ref = np.stack([x[lo:hi].astype(np.float64).mean(axis=0) for lo, hi in brute.block_ranges(53, b)])
        assert np.abs(oracle.pool(x, b, lib=lib) - ref).max() < 1e-15


def pin_select_matches_rows(lib):
    q, k, v = _rand(1200, 70, 8)
    a = oracle.select(q, k, 0.6, 9, lib=lib)
    b = oracle.attn_rows(q, k, v, 0.6, 9, want_s=True, lib=lib)
    assert np.array_equal(a["mask"], b["mask"])
    assert np.abs(a["tau"] - b["tau"]).max() == 0.0
    assert np.abs(a["mindist"] - np.abs(b["s"] - b["tau"][:, None]).min(axis=1)).max() == 0.0
    ref, _ = brute.dense_attention(q, k, v)
    assert np.abs(oracle.dense_rows(q, k, v, rows=[3, 7], lib=lib)["out"] - ref[[3, 7]]).max() < 1e-12


def pin_select_hand_examples(lib):
    """The whole-head selection routine on the hand examples: every case's kept blocks, including
    the exact ties (s = tau keeps the block), the population sigma and the hand-derived mu, sigma,
    tau and smallest |s - tau|; and a q = 0 row (sigma = 0) keeps every block at finite beta."""
    gd = json.load(open(GOLDEN))
    for name, M in (("example1", 2), ("example2", 3)):
        g = gd[name]
        k = np.array(g["k"], np.float32)
        q = (np.array(g["q"], np.float32) if "q" in g
             else np.tile(np.array(g["q_row"], np.float32), (g["N"], 1)))
        s = np.array(g["s"], np.float64)
        for c in g["cases"]:
            beta = _beta(c["beta"])
            r = oracle.select(q, k, beta, g["block"], lib=lib)
            keep = oracle.mask_bits(r["mask"], M).astype(int)
            assert (keep == np.array(c["keep"])).all(), (name, c, keep)
            tau = beta if math.isinf(beta) else g["mu"] + beta * g["sigma"]
            assert np.abs(r["mu"] - g["mu"]).max() < 1e-15
            assert np.abs(r["sigma"] - g["sigma"]).max() < 1e-14
            if math.isinf(beta):
                assert (r["tau"] == tau).all()
            else:
                assert np.abs(r["tau"] - tau).max() < 1e-14
                assert np.abs(r["mindist"] - np.abs(s - tau).min()).max() < 1e-14
    q, k, _ = _rand(1250, 40, 8)
    q[3] = 0.0
    for beta in (-1.0, 0.0, 2.5):
        r = oracle.select(q, k, beta, 8, lib=lib)
        assert oracle.mask_bits(r["mask"], 5)[3].all() and r["sigma"][3] == 0.0, beta


def _route_brute(q, k, block, mode, param):
    """Top-k / top-p selection written from the definition with numpy: proxies from the exact
    logits (brute.proxy_scores), a stable sort, and a cumulative sum."""
    s = brute.proxy_scores(q, k, block)
    N, M = s.shape
    n = np.array([b - a for a, b in brute.block_ranges(k.shape[0], block)], np.float64)
    key = s + np.log(n)[None, :] if mode == "topp" else s
    sel = np.zeros((N, M), bool)
    for i in range(N):
        order = sorted(range(M), key=lambda j: (-key[i, j], j))
        if mode == "topk":
            kk = 0 if param <= 0 else min(M, int(param))
            sel[i, order[:kk]] = True
        else:
            if param >= 1:
                sel[i] = True
                continue
            if param <= 0:
                continue
            w = np.exp(key[i] - key[i].max())
            pr = w / w.sum()
            before = 0.0
            for j in order:
                if before < param:
                    sel[i, j] = True
                before += pr[j]
    return sel


def pin_route_topk(lib):
    """Top-k: brute force on random inputs (distinct scores), the limits k <= 0 and k >= M, and
    ties broken toward the lower block index (q = 0 makes every score equal)."""
    q, k, _ = _rand(11, N=70, d=8)
    M = oracle.n_blocks(70, 8)
    for kk in (1, 3, 5):
        got = oracle.mask_bits(oracle.route(q, k, 8, "topk", kk, lib=lib)["mask"], M)
        assert np.array_equal(got, _route_brute(q, k, 8, "topk", kk)), kk
        assert (got.sum(axis=1) == kk).all()
    assert not oracle.mask_bits(oracle.route(q, k, 8, "topk", 0, lib=lib)["mask"], M).any()
    assert oracle.mask_bits(oracle.route(q, k, 8, "topk", M + 5, lib=lib)["mask"], M).all()
    z = np.zeros_like(q)
    got = oracle.mask_bits(oracle.route(z, k, 8, "topk", 4, lib=lib)["mask"], M)
    assert (got[:, :4]).all() and not got[:, 4:].any()


def pin_route_topp(lib):
    """Top-p: brute force, the limits p <= 0 (none) and p >= 1 (all), a tiny p keeping only the
    most probable block (pooled logit s + ln n, which favours the full blocks over the short last
    one), and monotonicity in p."""
    q, k, _ = _rand(12, N=70, d=8)
    M = oracle.n_blocks(70, 8)
    prev = None
    for p in (0.05, 0.3, 0.6, 0.9):
        got = oracle.mask_bits(oracle.route(q, k, 8, "topp", p, lib=lib)["mask"], M)
        assert np.array_equal(got, _route_brute(q, k, 8, "topp", p)), p
        if prev is not None:
            assert (got | prev == got).all()
        prev = got
    assert not oracle.mask_bits(oracle.route(q, k, 8, "topp", 0.0, lib=lib)["mask"], M).any()
    assert oracle.mask_bits(oracle.route(q, k, 8, "topp", 1.0, lib=lib)["mask"], M).all()
    got = oracle.mask_bits(oracle.route(q, k, 8, "topp", 1e-12, lib=lib)["mask"], M)
    s = brute.proxy_scores(q, k, 8) + np.log([min(8, 70 - 8 * j) for j in range(M)])[None, :]
    assert (got.sum(axis=1) == 1).all()
    assert (np.argmax(got, axis=1) == np.argmax(s, axis=1)).all()


PINS = [f for n, f in sorted(globals().items()) if n.startswith("pin_") and callable(f)]
