"""Host-side FLOP accounting used by the benchmark (CPU only): the union counts over groups of
query rows agree with a direct numpy count."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import oracle

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("N,block", [(1000, 128), (333, 64), (4096, 128), (1, 64)])
def test_union_units_match_direct_count(N, block):
    from block_sparse_attention_sol_amd import solattn
    rng = np.random.default_rng(N + block)
    M = (N + block - 1) // block
    W = (M + 31) // 32
    B, H = 1, 2
    sel = rng.random((B, H, N, M)) < 0.07
    packed = np.stack([np.stack([oracle.pack_bits(sel[b, h]) for h in range(H)]) for b in range(B)])
    mask = torch.from_numpy(packed.view(np.int32).reshape(B, H, N, W).copy())
    got = solattn.union_units(mask, N, block, heights=(1, 32, 128))
    n = np.array([min((j + 1) * block, N) - j * block for j in range(M)], np.float64)
    for hgt in (1, 32, 128):
        want = 0.0
        for b in range(B):
            for h in range(H):
                for g0 in range(0, N, hgt):
                    rows = min(N, g0 + hgt) - g0
                    u = sel[b, h, g0:g0 + hgt].any(axis=0)
                    want += rows * n[u].sum()
        assert got[hgt] == pytest.approx(want, rel=0, abs=0), (hgt, got[hgt], want)
    # height 128 is the tile union the oracle's density helper counts
    tile_units = sum(oracle.tile_union_density(sel[0, h], N, block)[2] for h in range(H))
    assert got[128] == tile_units
