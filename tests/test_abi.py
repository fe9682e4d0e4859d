"""The C ABI without a GPU: the library loads, exports what the header declares, and rejects bad
arguments before making any HIP call (every case below has exactly one invalid argument, so no
kernel is ever launched)."""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

from block_sparse_attention_sol_amd import solattn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "solattn.h")

FAKE = 0x7F0000000000  # 16-byte aligned host-side stand-in; never dereferenced on these paths


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(solattn.LIB_PATH):
        from block_sparse_attention_sol_amd import build
        build.build()
    return solattn.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sol_[a-z0-9_]+)\s*\(", text)))


def test_header_and_exports_agree(lib):
    declared = header_functions()
    assert declared == sorted(solattn.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_exported_symbols_are_c_names():
    syms = os.popen(f"nm -D --defined-only {solattn.LIB_PATH}").read()
    for name in solattn.EXPORTS:
        assert re.search(rf"\bT {name}\b", syms), name


def test_version_and_status_strings(lib):
    assert b"gfx950" in lib.sol_version()
    for st in (0, -1, -2, -3, -4, -5):
        assert lib.sol_status_str(st)
    assert lib.sol_status_str(99) == b"unknown status"


def _shape(B=1, H=2, N=1000, d=128):
    return solattn.SolShape(B, H, N, d)


def _ptrs(n):
    return [ctypes.c_void_p(FAKE + i * (1 << 32)) for i in range(n)]


def _fwd(lib, shape, q, k, v, beta, block, out, ws, ws_bytes):
    return lib.sol_attn_fwd(ctypes.byref(shape), q, k, v, beta, block, out, ws, ws_bytes, None)


def test_workspace_bytes(lib):
    s = _shape(1, 40, 75600, 128)
    n = lib.sol_attn_workspace_bytes(ctypes.byref(s), 128)
    M = math.ceil(75600 / 128)
    Mp = math.ceil(M / 32) * 32
    lower = (40 * M * 128 * 4 + 40 * 128 * 8 + 40 * 128 * 128 * 8 + 40 * 4 * 128 * 8 + 40 * 4 + 3 * 40 * 128 * 128 * 2
             + 3 * 40 * Mp * 128 * 2 + 40 * Mp * 128 * 2 + 40 * 75600 * 4 + 40 * 75600 * (Mp // 32) * 4)
    assert lower <= n <= lower + 8 * 256
    assert lib.sol_attn_workspace_bytes(ctypes.byref(_shape(d=96)), 128) == 0
    assert lib.sol_attn_workspace_bytes(ctypes.byref(_shape()), 32) == 0
    assert lib.sol_attn_workspace_bytes(None, 128) == 0


@pytest.mark.parametrize("case", [
    "null_shape", "null_q", "null_out", "misaligned_k", "nan_beta", "bad_d", "bad_block",
    "zero_n", "zero_heads", "huge_n", "no_workspace", "small_workspace", "out_overlaps_q",
])
def test_attn_fwd_rejects(lib, case):
    s = _shape()
    q, k, v, out, ws = _ptrs(5)
    need = lib.sol_attn_workspace_bytes(ctypes.byref(s), 128)
    beta, block, nbytes = 0.5, 128, need
    expect = solattn.SOL_EINVAL
    shape_arg = ctypes.byref(s)
    if case == "null_shape":
        shape_arg = None
    elif case == "null_q":
        q = None
    elif case == "null_out":
        out = None
    elif case == "misaligned_k":
        k = ctypes.c_void_p(FAKE + 8)
    elif case == "nan_beta":
        beta = float("nan")
    elif case == "bad_d":
        s.d = 96
        expect = solattn.SOL_EUNSUPPORTED
    elif case == "bad_block":
        block = 256
        expect = solattn.SOL_EUNSUPPORTED
    elif case == "zero_n":
        s.N = 0
    elif case == "zero_heads":
        s.H = 0
    elif case == "huge_n":
        s.N = (1 << 22) + 1
    elif case == "no_workspace":
        ws = None
        expect = solattn.SOL_EWORKSPACE
    elif case == "small_workspace":
        nbytes = need - 1
        expect = solattn.SOL_EWORKSPACE
    elif case == "out_overlaps_q":
        out = ctypes.c_void_p(q.value + 4096)
    st = lib.sol_attn_fwd(shape_arg, q, k, v, beta, block, out, ws, nbytes, None)
    assert st == expect, (case, st, lib.sol_last_error())
    assert lib.sol_last_error(), case


@pytest.mark.parametrize("case", ["null_shape", "null_q", "null_out", "misaligned_v", "nan_beta",
                                  "bad_d", "bad_block", "zero_n", "out_overlaps_k",
                                  "head_exceeds_scratch"])
def test_attn_fwd_noalloc_rejects(lib, case):
    """The allocation-free call validates everything, including whether one head's workspace fits
    its scratch (SOL_NOALLOC_SCRATCH_BYTES), before its first HIP call."""
    s = _shape()
    q, k, v, out = _ptrs(4)
    beta, block = 0.5, 128
    expect = solattn.SOL_EINVAL
    shape_arg = ctypes.byref(s)
    if case == "null_shape":
        shape_arg = None
    elif case == "null_q":
        q = None
    elif case == "null_out":
        out = None
    elif case == "misaligned_v":
        v = ctypes.c_void_p(v.value + 2)
    elif case == "nan_beta":
        beta = float("nan")
    elif case == "bad_d":
        s.d = 256
        expect = solattn.SOL_EUNSUPPORTED
    elif case == "bad_block":
        block = 96
        expect = solattn.SOL_EUNSUPPORTED
    elif case == "zero_n":
        s.N = 0
    elif case == "out_overlaps_k":
        out = ctypes.c_void_p(k.value + 256)
    elif case == "head_exceeds_scratch":
        # 2^21 tokens in 64-key blocks: 1024 selection words per row, 8 GiB of them per head
        s.N, s.H, block = 1 << 21, 1, 64
        one = solattn.SolShape(1, 1, s.N, s.d)
        assert lib.sol_attn_workspace_bytes(ctypes.byref(one), block) > solattn.NOALLOC_SCRATCH_BYTES
        expect = solattn.SOL_EWORKSPACE
    st = lib.sol_attn_fwd_noalloc(shape_arg, q, k, v, beta, block, out, None)
    assert st == expect, (case, st, lib.sol_last_error())
    assert lib.sol_last_error(), case


@pytest.mark.parametrize("case", ["null_grid", "grid_too_small", "grid_too_large", "zero_t",
                                  "negative_w", "huge_factor", "grid_ok_small_workspace"])
def test_attn_fwd_grid_rejects(lib, case):
    """The latent grid must hold exactly N tokens; it is checked with the other arguments, before
    any HIP call."""
    s = _shape()
    q, k, v, out, ws = _ptrs(5)
    need = lib.sol_attn_workspace_bytes(ctypes.byref(s), 128)
    nbytes = need
    g = solattn.SolGrid(2, 4, s.N // 8)
    assert g.T * g.H * g.W == s.N
    grid_arg = ctypes.byref(g)
    expect = solattn.SOL_EINVAL
    if case == "null_grid":
        grid_arg = None
    elif case == "grid_too_small":
        g.W -= 1
    elif case == "grid_too_large":
        g.W += 1
    elif case == "zero_t":
        g.T = 0
    elif case == "negative_w":
        g.W = -g.W
    elif case == "huge_factor":
        g.T, g.H, g.W = 1 << 40, 1 << 40, 1
    elif case == "grid_ok_small_workspace":
        nbytes = need - 1
        expect = solattn.SOL_EWORKSPACE
    st = lib.sol_attn_fwd_grid(ctypes.byref(s), grid_arg, q, k, v, 0.5, 128, out, ws, nbytes, None,
                               None)
    assert st == expect, (case, st, lib.sol_last_error())
    assert lib.sol_last_error(), case


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define SOL_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == solattn.NOALLOC_SCRATCH_BYTES


def test_infinite_beta_passes_validation_only_to_workspace_check(lib):
    """+-inf beta are valid values: with an undersized workspace the call fails on the workspace,
    not on beta."""
    s = _shape()
    q, k, v, out, ws = _ptrs(5)
    for beta in (float("inf"), float("-inf")):
        st = lib.sol_attn_fwd(ctypes.byref(s), q, k, v, beta, 128, out, ws, 16, None)
        assert st == solattn.SOL_EWORKSPACE


def test_dense_and_pool_reject(lib):
    s = _shape()
    q, k, v, out, kb = _ptrs(5)
    assert lib.sol_dense_fwd(ctypes.byref(s), q, None, v, out, None, None) == solattn.SOL_EINVAL
    s2 = _shape(d=32)
    assert lib.sol_dense_fwd(ctypes.byref(s2), q, k, v, out, None, None) == solattn.SOL_EUNSUPPORTED
    assert lib.sol_dense_fwd(ctypes.byref(s), q, k, v, q, None, None) == solattn.SOL_EINVAL
    assert lib.sol_pool_kv(ctypes.byref(s), k, v, 100, kb, out, None) == solattn.SOL_EUNSUPPORTED
    assert lib.sol_pool_kv(ctypes.byref(s), k, v, 64, None, out, None) == solattn.SOL_EINVAL
    assert lib.sol_pool_kv(ctypes.byref(s), k, v, 64, kb, kb, None) == solattn.SOL_EINVAL
    dbg = solattn.SolAttnDebug()
    dbg.mu = FAKE + 2
    need = lib.sol_attn_workspace_bytes(ctypes.byref(s), 64)
    st = lib.sol_attn_fwd_ex(ctypes.byref(s), q, k, v, 0.0, 64, out, _ptrs(6)[5], need,
                             ctypes.byref(dbg), None)
    assert st == solattn.SOL_EINVAL and b"aligned" in lib.sol_last_error()


def test_binding_refuses_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        solattn.attn_fwd(q, q, q, 0.5, 64, out=torch.zeros_like(q),
                         workspace=torch.zeros(1 << 20, dtype=torch.uint8))


def test_mfma_probe_rejects(lib):
    sink = _ptrs(1)[0]
    assert lib.sol_mfma_probe(0, 10, sink, None) == solattn.SOL_EINVAL
    assert lib.sol_mfma_probe(8, 0, sink, None) == solattn.SOL_EINVAL
    assert lib.sol_mfma_probe(8, 10, None, None) == solattn.SOL_EINVAL
    assert b"sink" in lib.sol_last_error()


def test_routing_entries_reject(lib):
    s = _shape()
    q, k, v, out, ws, smap, mask = _ptrs(7)
    need = lib.sol_attn_workspace_bytes(ctypes.byref(s), 128)
    nan = float("nan")
    assert lib.sol_attn_fwd_masked(ctypes.byref(s), q, k, v, None, 128, 0, out, ws, need,
                                   None) == solattn.SOL_EINVAL
    assert b"mask" in lib.sol_last_error()
    assert lib.sol_attn_fwd_masked(ctypes.byref(s), q, k, v, FAKE + 2, 128, 0, out, ws, need,
                                   None) == solattn.SOL_EINVAL
    assert lib.sol_attn_fwd_masked(ctypes.byref(s), q, k, v, mask, 128, 0, out, ws, 16,
                                   None) == solattn.SOL_EWORKSPACE
    assert lib.sol_proxy_map(ctypes.byref(s), q, k, 100, smap, ws, need, None) == solattn.SOL_EUNSUPPORTED
    assert lib.sol_proxy_map(ctypes.byref(s), q, k, 128, smap, ws, 16, None) == solattn.SOL_EWORKSPACE
    assert lib.sol_proxy_map(ctypes.byref(s), q, None, 128, smap, ws, need, None) == solattn.SOL_EINVAL
    assert lib.sol_proxy_map(ctypes.byref(s), q, k, 128, ws, ws, need, None) == solattn.SOL_EINVAL
    assert lib.sol_select_topk(ctypes.byref(s), 128, smap, 3, None, None) == solattn.SOL_EINVAL
    assert lib.sol_select_topk(ctypes.byref(s), 96, smap, 3, mask, None) == solattn.SOL_EUNSUPPORTED
    assert lib.sol_select_topp(ctypes.byref(s), 128, smap, nan, mask, None) == solattn.SOL_EINVAL
    assert lib.sol_select_topp(ctypes.byref(s), 128, None, 0.5, mask, None) == solattn.SOL_EINVAL
    assert lib.sol_select_topp(ctypes.byref(s), 128, smap, 0.5, smap, None) == solattn.SOL_EINVAL


def test_selection_block_limit(lib):
    s = solattn.SolShape(1, 1, 2049 * 64, 64)  # M = 2049 key blocks per row
    smap, mask = _ptrs(2)
    assert lib.sol_select_topk(ctypes.byref(s), 64, smap, 3, mask, None) == solattn.SOL_EUNSUPPORTED
    assert b"2048" in lib.sol_last_error()


def test_strides_reject(lib):
    s = _shape(B=1, H=2, N=1000, d=128)
    q, k, v, out, ws = _ptrs(5)
    need = lib.sol_attn_workspace_bytes(ctypes.byref(s), 128)

    def call(ins, outs):
        return lib.sol_attn_fwd_strided(ctypes.byref(s), ctypes.byref(ins) if ins else None,
                                        ctypes.byref(outs) if outs else None, q, k, v, 0.5, 128, out,
                                        ws, need, None)
    bnhd = solattn.SolStrides(1000 * 2 * 128, 128, 2 * 128)
    assert call(solattn.SolStrides(2 * 1000 * 128, 1000 * 128, 64), None) == solattn.SOL_EINVAL  # n < d
    assert b"below d" in lib.sol_last_error()
    assert call(solattn.SolStrides(2 * 1000 * 128, 1000 * 128, 132), None) == solattn.SOL_EINVAL  # not x8
    assert call(None, solattn.SolStrides(0, 64, 256)) == solattn.SOL_EINVAL  # heads overlap rows
    assert b"overlap" in lib.sol_last_error()
    # valid layouts get past stride validation (and fail later on the workspace size check only)
    st = lib.sol_attn_fwd_strided(ctypes.byref(s), ctypes.byref(bnhd), ctypes.byref(bnhd), q, k, v,
                                  0.5, 128, out, ws, 16, None)
    assert st == solattn.SOL_EWORKSPACE
    assert lib.sol_dense_fwd_strided(ctypes.byref(s), ctypes.byref(bnhd), None, q, k, None, out, None,
                                     None) == solattn.SOL_EINVAL
