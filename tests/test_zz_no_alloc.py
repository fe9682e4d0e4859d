"""The allocation-free forward call (sol_attn_fwd_noalloc) against sol_attn_fwd with a caller
workspace, through the C ABI, on two calls in a row: first the Wan2.1-14B shape (40 heads, whose
workspace exceeds the library's scratch, so the heads run in groups), then a smaller input."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from tests.parity_util import MAX_ABS, MEAN_REL, half_ulp_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def sol():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from block_sparse_attention_sol_amd import solattn
    solattn.load_library()
    return solattn


def _compare(sol, q, k, v, beta, block, what):
    ref = sol.attn_fwd(q, k, v, beta, block)
    out = torch.full_like(q, float("nan"))
    sol.attn_fwd_noalloc(q, k, v, beta, block, out)
    torch.cuda.synchronize()
    a = out.float().cpu().numpy()
    r = ref.float().cpu().numpy()
    assert np.isfinite(a).all(), f"{what}: non-finite output"
    d = np.abs(a - r)
    # both are bf16 roundings of fp32 results that differ only in summation order: within the
    # output bar plus one bf16 ulp (two half-ulp roundings)
    excess = float((d - 2.0 * half_ulp_bf16(r)).max())
    mean_rel = float(d.sum() / np.abs(r).sum())
    same = float((a == r).mean())
    print(f"{what}: max-abs {d.max():.3e}, beyond rounding {excess:.3e}, mean-rel {mean_rel:.3e}, "
          f"identical {same:.4f}", flush=True)
    assert excess <= MAX_ABS and mean_rel <= MEAN_REL, what
    return same


def test_noalloc_matches_workspace_call_twice(sol):
    from block_sparse_attention_sol_amd import synth
    print("noalloc call 1: Wan2.1-14B shape, 40 heads", flush=True)
    q, k, v = (t.cuda() for t in synth.generate("wan"))
    B, H, N, d = q.shape
    lib = sol.load_library()
    need = lib.sol_attn_workspace_bytes(ctypes.byref(sol.SolShape(B, H, N, d)), 128)
    assert need > sol.NOALLOC_SCRATCH_BYTES, "this call must exercise grouped heads"
    _compare(sol, q, k, v, 2.21875, 128, "noalloc wan")
    del q, k, v
    print("noalloc call 2: B=2 H=3 N=5000 d=128, block 64", flush=True)
    q, k, v = (t.cuda() for t in synth.random_qkv(2, 3, 5000, 128, seed=77, scale=1.4))
    _compare(sol, q, k, v, 0.8, 64, "noalloc small")
    print("noalloc call 3: B=1 H=2 N=700 d=64, block 64", flush=True)
    q, k, v = (t.cuda() for t in synth.random_qkv(1, 2, 700, 64, seed=78, scale=1.2))
    _compare(sol, q, k, v, 0.3, 64, "noalloc d64")
