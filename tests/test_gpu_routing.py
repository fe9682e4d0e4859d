"""Prior-art routing pipeline (proxy map -> top-k / top-p selection -> attention with the
caller's selection) on the GPU against the fp64 oracle.  Every call goes through the C ABI.

Acceptance bar:
  * proxy map: |s_gpu - s| <= 1e-5 * max(1, max |s|) (the fused kernel's fp32-accurate proxies);
  * selections: bit-exact per row, except rows whose decision the oracle measures as within
    rounding: a score gap at the selection boundary below 1e-4 (both orders are correct), or, for
    top-p, a cumulative probability within 1e-4 of p before some block;
  * attention with a given selection: the bar of the fused kernel (bf16 output within 2e-2 plus
    half a bf16 ulp of the oracle, mean-rel 5e-3), against the oracle run with the same mask;
  * the method's own selection fed back through the masked entry reproduces sol_attn_fwd exactly.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import oracle
from tests.parity_util import assert_close_bf16_output, sample_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
GAP = 1e-4


@pytest.fixture(scope="module")
def sol():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from block_sparse_attention_sol_amd import solattn
    solattn.load_library()
    return solattn


def _np(t):
    return t.float().cpu().numpy()


def _qkv(B, H, N, d, seed, scale=1.0):
    from block_sparse_attention_sol_amd import synth
    q, k, v = synth.random_qkv(B, H, N, d, seed=seed, scale=scale)
    return q.cuda(), k.cuda(), v.cuda()


def _log(msg):
    print(msg, flush=True)


def _check_selection(gpu_words, ref, M, mode, what):
    """Row-wise comparison with the oracle's selection; returns the number of exempt rows."""
    g = oracle.mask_bits(np.ascontiguousarray(gpu_words).view(np.uint32), M)
    o = oracle.mask_bits(ref["mask"], M)
    bad = np.nonzero((g != o).any(axis=1))[0]
    exempt = ref["gap"][bad] < GAP
    if mode == "topp":
        exempt |= ref["massgap"][bad] < GAP
    assert exempt.all(), (f"{what}: {int((~exempt).sum())} rows differ outside the rounding band; "
                          f"first row {bad[~exempt][0]}")
    return int(bad.size)


CASES = [(1, 2, 1000, 128, 128), (1, 1, 333, 64, 64), (2, 1, 130, 64, 128), (1, 1, 4100, 128, 128)]


@pytest.mark.parametrize("B,H,N,d,block", CASES)
def test_proxy_map(sol, B, H, N, d, block):
    _log(f"proxy map B={B} H={H} N={N} d={d} block={block}")
    q, k, v = _qkv(B, H, N, d, seed=N + d, scale=1.2)
    smap = sol.proxy_map(q, k, block)
    torch.cuda.synchronize()
    M = oracle.n_blocks(N, block)
    assert smap.shape == (B, H, N, M)
    for b in range(B):
        for h in range(H):
            r = oracle.attn_rows(_np(q[b, h]), _np(k[b, h]), _np(v[b, h]), 0.0, block, want_s=True)
            s = r["s"]                                   # [N, M]
            g = _np(smap[b, h]).astype(np.float64)       # [N, M]
            err = float(np.abs(g - s).max())
            assert err <= 1e-5 * max(1.0, float(np.abs(s).max())), (b, h, err)


@pytest.mark.parametrize("B,H,N,d,block", CASES)
@pytest.mark.parametrize("mode,params", [("topk", (0, 1, 3, 7, 10 ** 6)), ("topp", (0.0, 0.05, 0.3, 0.7, 0.95, 1.0))])
def test_selection_matches_oracle(sol, B, H, N, d, block, mode, params):
    _log(f"{mode} B={B} H={H} N={N} d={d} block={block}")
    q, k, v = _qkv(B, H, N, d, seed=2 * N + d, scale=1.2)
    smap = sol.proxy_map(q, k, block)
    M = oracle.n_blocks(N, block)
    for prm in params:
        if mode == "topk":
            words = sol.select_topk(smap, tuple(q.shape), block, prm)
        else:
            words = sol.select_topp(smap, tuple(q.shape), block, prm)
        torch.cuda.synchronize()
        for b in range(B):
            for h in range(H):
                ref = oracle.route(_np(q[b, h]), _np(k[b, h]), block, mode, prm)
                gw = words[b, h].cpu().numpy()
                n_exempt = _check_selection(gw, ref, M, mode, f"{mode}={prm} b{b} h{h}")
                if mode == "topk":
                    kept = oracle.mask_bits(gw.view(np.uint32), M).sum(axis=1)
                    assert (kept == min(max(prm, 0), M)).all()
                _log(f"  {mode}={prm} b{b} h{h}: {n_exempt} near-tie rows exempt")


@pytest.mark.parametrize("mode,prm,drop", [("topk", 3, False), ("topk", 3, True), ("topp", 0.5, False),
                                           ("topp", 0.8, True)])
def test_masked_attention_matches_oracle(sol, mode, prm, drop):
    _log(f"masked attention {mode}={prm} drop={drop}")
    B, H, N, d, block = 1, 2, 1100, 128, 128
    q, k, v = _qkv(B, H, N, d, seed=77, scale=1.3)
    smap = sol.proxy_map(q, k, block)
    sel = sol.select_topk(smap, tuple(q.shape), block, prm) if mode == "topk" else \
        sol.select_topp(smap, tuple(q.shape), block, prm)
    out = sol.attn_fwd_masked(q, k, v, sel, block, drop_unselected=drop)
    torch.cuda.synchronize()
    for h in range(H):
        gmask = sel[0, h].cpu().numpy().view(np.uint32)
        r = oracle.attn_rows(_np(q[0, h]), _np(k[0, h]), _np(v[0, h]), 0.0, block,
                             mask_override=gmask, drop=drop)
        ok = ~np.isnan(r["out"][:, 0])
        ma, mr = assert_close_bf16_output(_np(out[0, h])[ok], r["out"][ok], f"{mode} h{h}")
        assert (_np(out[0, h])[~ok] == 0).all()
        _log(f"  h{h}: max-abs {ma:.3e} mean-rel {mr:.3e}")


def test_masked_with_own_selection_is_the_method(sol):
    """The fused kernel's own selection fed back through the masked entry gives the same bits."""
    _log("masked entry with the method's own mask")
    q, k, v = _qkv(1, 3, 2500, 128, seed=5, scale=1.4)
    ref, dbg = sol.attn_fwd(q, k, v, 0.9, 128, debug=True)
    out = sol.attn_fwd_masked(q, k, v, dbg["mask"], 128)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_wan_shape_topk_topp_sampled(sol):
    """Wan2.1-14B shape (N=75600, d=128, block 128, last block 80 tokens), first two heads of the
    seeded draw: full top-k / top-p masks against the oracle; masked attention on sampled rows."""
    from block_sparse_attention_sol_amd import synth
    _log("wan topk/topp: generating 2 heads")
    q, k, v = (t.cuda() for t in synth.generate("wan", heads=2))
    block = 128
    M = oracle.n_blocks(q.shape[2], block)
    smap = sol.proxy_map(q, k, block)
    for mode, prm in (("topk", 17), ("topp", 0.5)):
        sel = sol.select_topk(smap, tuple(q.shape), block, prm) if mode == "topk" else \
            sol.select_topp(smap, tuple(q.shape), block, prm)
        out = sol.attn_fwd_masked(q, k, v, sel, block)
        torch.cuda.synchronize()
        for h in range(2):
            qh, kh, vh = _np(q[0, h]), _np(k[0, h]), _np(v[0, h])
            ref = oracle.route(qh, kh, block, mode, prm)
            gw = sel[0, h].cpu().numpy()
            n_exempt = _check_selection(gw, ref, M, mode, f"wan {mode} h{h}")
            rows = sample_rows(q.shape[2], 300, seed=h)
            r = oracle.attn_rows(qh, kh, vh, 0.0, block, rows=rows,
                                 mask_override=gw.view(np.uint32)[rows])
            ma, mr = assert_close_bf16_output(_np(out[0, h])[rows], r["out"], f"wan {mode} h{h}")
            _log(f"  wan {mode}={prm} h{h}: {n_exempt} exempt rows, max-abs {ma:.3e} mean-rel {mr:.3e}")
