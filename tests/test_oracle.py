"""The fp64 oracle against its pins (CPU only)."""
import math

import numpy as np
import pytest

from oracle import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_pin(pin, olib):
    pin(olib)


def test_rejects_nan_beta(olib):
    q = np.zeros((4, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.attn_rows(q, q, q, float("nan"), 2, lib=olib)
    with pytest.raises(ValueError):
        oracle.attn_rows(q, q, q, 0.0, 2, rows=[4], lib=olib)


def test_drop_ablation(olib):
    """Dropping unselected blocks (the ablation) equals softmax over the kept exact tokens."""
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((40, 8)).astype(np.float32) for _ in range(3))
    r = oracle.attn_rows(q, k, v, 0.3, 8, drop=True, lib=olib)
    sel = oracle.mask_bits(r["mask"], 5)
    logits = q.astype(np.float64) @ k.T.astype(np.float64) / math.sqrt(8)
    keep_tok = np.repeat(sel, 8, axis=1)
    logits = np.where(keep_tok, logits, -np.inf)
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    ref = (w @ v.astype(np.float64)) / w.sum(axis=1, keepdims=True)
    assert np.abs(r["out"] - ref).max() < 1e-12
    r_none = oracle.attn_rows(q, k, v, float("inf"), 8, rows=[0], drop=True, lib=olib)
    assert np.isnan(r_none["out"]).all() and np.isnan(r_none["lse"]).all()


def test_ltx_rows_near_normal(olib):
    """Soft check on the LTX-style workload: the page observes near-normal proxy rows, so the
    kept fraction per row is close to 1 - Phi(beta).  Eight heads, +-4 percentage points."""
    from block_sparse_attention_sol_amd import synth
    w = synth.WORKLOADS["ltx"]
    q, k, _ = synth.generate(w, heads=8)
    for beta in w.betas:
        dens = []
        for h in range(8):
            r = oracle.select(q[0, h].float().numpy(), k[0, h].float().numpy(), beta, w.block, lib=olib)
            dens.append(oracle.mask_bits(r["mask"], w.M).mean())
        expect = 0.5 * math.erfc(beta / math.sqrt(2.0))
        assert abs(np.mean(dens) - expect) < 0.04, (beta, np.mean(dens), expect)
