"""Python face of the fp64 CPU oracle (``sol_oracle.c``).

TEST INFRASTRUCTURE ONLY: the checker, not the product.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg import this module.  It never imports the GPU package, and
the GPU package never imports it.

The arithmetic lives in ``sol_oracle.c`` (plain fp64 C, one query row at a time); this module only
builds the shared library with gcc, marshals numpy arrays and converts results.  The method it
follows is the one on the page "Sol-Attn: Accelerating Video Generation Inference via On-the-Fly
Attention Sparsification" (agihunt.info/papers/2607.24027): per-query threshold
tau_i = mu_i + beta*sigma_i over the row of pooled proxy scores, exact attention on the kept
blocks, one pooled token per unselected block.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sol_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-adds, so every product and sum is rounded once in fp64.
CFLAGS = ["-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall"]


def build(out: str = _LIB, extra: tuple = ()) -> str:
    """Compile sol_oracle.c into a shared library (always recompiles)."""
    cmd = ["gcc", *CFLAGS, *extra, _SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib_cache: dict = {}


def load(path: str = _LIB):
    """Load the oracle library, building it first only if it does not exist."""
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        build(path)
    lib = ctypes.CDLL(path)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    ci = ctypes.c_int
    cd = ctypes.c_double
    lib.sol_oracle_pool.argtypes = [p, i64, ci, ci, p]
    lib.sol_oracle_rows.argtypes = [p, p, p, i64, ci, ci, cd, p, i64, p, ci, p, p, p, p, p, p, p]
    lib.sol_oracle_select.argtypes = [p, p, i64, ci, ci, cd, p, p, p, p, p]
    lib.sol_oracle_dense_rows.argtypes = [p, p, p, i64, ci, p, i64, p, p]
    lib.sol_oracle_route.argtypes = [p, p, i64, ci, ci, ci, cd, p, p, p]
    for f in ("sol_oracle_pool", "sol_oracle_rows", "sol_oracle_select", "sol_oracle_dense_rows",
              "sol_oracle_route"):
        getattr(lib, f).restype = ci
    lib.sol_oracle_threads.argtypes = []
    lib.sol_oracle_threads.restype = ci
    _lib_cache[path] = lib
    return lib


def _f32(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return a


def _ptr(a) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data) if a is not None else ctypes.c_void_p(0)


def n_blocks(N: int, block: int) -> int:
    return (N + block - 1) // block


def pool(x, block: int, lib=None) -> np.ndarray:
    """Block means of x [N, d] -> [M, d] fp64."""
    lib = lib or load()
    x = _f32(x)
    N, d = x.shape
    out = np.empty((n_blocks(N, block), d), np.float64)
    rc = lib.sol_oracle_pool(_ptr(x), N, d, block, _ptr(out))
    if rc != 0:
        raise ValueError(f"sol_oracle_pool failed ({rc})")
    return out


def attn_rows(q, k, v, beta: float, block: int, rows=None, mask_override=None, drop: bool = False,
              want_s: bool = False, lib=None) -> dict:
    """Sol-Attn forward for one head on the given query rows (all rows if None).

    q, k, v: [N, d] arrays holding bf16 values (any float dtype; converted to fp32 exactly).
    Returns a dict with out [R, d], lse, mu, sigma, tau [R], mask [R, W] uint32 and, if asked,
    s [R, M] (all fp64 except the mask).
    """
    lib = lib or load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    N, d = q.shape
    M = n_blocks(N, block)
    W = (M + 31) // 32
    rows = np.arange(N, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    R = rows.shape[0]
    res = {
        "out": np.empty((R, d), np.float64),
        "lse": np.empty(R, np.float64),
        "mu": np.empty(R, np.float64),
        "sigma": np.empty(R, np.float64),
        "tau": np.empty(R, np.float64),
        "mask": np.empty((R, W), np.uint32),
    }
    s = np.empty((R, M), np.float64) if want_s else None
    mo = None
    if mask_override is not None:
        mo = np.ascontiguousarray(mask_override, np.uint32)
        if mo.shape != (R, W):
            raise ValueError(f"mask_override must be [{R}, {W}], got {mo.shape}")
    rc = lib.sol_oracle_rows(_ptr(q), _ptr(k), _ptr(v), N, d, block, float(beta), _ptr(rows), R,
                             _ptr(mo), int(bool(drop)), _ptr(res["out"]), _ptr(res["lse"]),
                             _ptr(res["mu"]), _ptr(res["sigma"]), _ptr(res["tau"]),
                             _ptr(res["mask"]), _ptr(s))
    if rc != 0:
        raise ValueError(f"sol_oracle_rows failed ({rc})")
    if want_s:
        res["s"] = s
    res["rows"] = rows
    return res


def select(q, k, beta: float, block: int, lib=None) -> dict:
    """Selection mask, mu, sigma, tau and min |s - tau| for every row of one head."""
    lib = lib or load()
    q, k = _f32(q), _f32(k)
    N, d = q.shape
    M = n_blocks(N, block)
    W = (M + 31) // 32
    res = {
        "mask": np.empty((N, W), np.uint32),
        "mu": np.empty(N, np.float64),
        "sigma": np.empty(N, np.float64),
        "tau": np.empty(N, np.float64),
        "mindist": np.empty(N, np.float64),
    }
    rc = lib.sol_oracle_select(_ptr(q), _ptr(k), N, d, block, float(beta), _ptr(res["mask"]),
                               _ptr(res["mu"]), _ptr(res["sigma"]), _ptr(res["tau"]),
                               _ptr(res["mindist"]))
    if rc != 0:
        raise ValueError(f"sol_oracle_select failed ({rc})")
    return res


def dense_rows(q, k, v, rows=None, lib=None) -> dict:
    """Plain dense softmax attention (scale 1/sqrt(d), no mask) for the given rows."""
    lib = lib or load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    N, d = q.shape
    rows = np.arange(N, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    R = rows.shape[0]
    out = np.empty((R, d), np.float64)
    lse = np.empty(R, np.float64)
    rc = lib.sol_oracle_dense_rows(_ptr(q), _ptr(k), _ptr(v), N, d, _ptr(rows), R, _ptr(out),
                                   _ptr(lse))
    if rc != 0:
        raise ValueError(f"sol_oracle_dense_rows failed ({rc})")
    return {"out": out, "lse": lse, "rows": rows}


def route(q, k, block: int, mode: str, param: float, lib=None) -> dict:
    """Prior-art routing on the same proxy for every row of one head: mode "topk" (param = k)
    or "topp" (param = p); see sol_oracle_route.  Returns mask [N, W], gap [N], massgap [N]."""
    lib = lib or load()
    q, k = _f32(q), _f32(k)
    N, d = q.shape
    M = n_blocks(N, block)
    W = (M + 31) // 32
    res = {"mask": np.empty((N, W), np.uint32), "gap": np.empty(N, np.float64),
           "massgap": np.empty(N, np.float64)}
    m = {"topk": 0, "topp": 1}[mode]
    rc = lib.sol_oracle_route(_ptr(q), _ptr(k), N, d, block, m, float(param), _ptr(res["mask"]),
                              _ptr(res["gap"]), _ptr(res["massgap"]))
    if rc != 0:
        raise ValueError(f"sol_oracle_route failed ({rc})")
    return res


def mask_bits(mask: np.ndarray, M: int) -> np.ndarray:
    """Unpack [R, W] uint32 selection words into a [R, M] bool array (bit j%32 of word j/32)."""
    mask = np.ascontiguousarray(mask, np.uint32)
    bits = np.unpackbits(mask.view(np.uint8), axis=1, bitorder="little")
    return bits[:, :M].astype(bool)


def pack_bits(sel: np.ndarray) -> np.ndarray:
    """Inverse of mask_bits: [R, M] bool -> [R, ceil(M/32)] uint32."""
    sel = np.asarray(sel, bool)
    R, M = sel.shape
    W = (M + 31) // 32
    padded = np.zeros((R, W * 32), bool)
    padded[:, :M] = sel
    return np.packbits(padded, axis=1, bitorder="little").view(np.uint32).reshape(R, W)


def tile_union_density(sel: np.ndarray, N: int, block: int, tile: int = 128) -> tuple:
    """Kept-block density at query-tile granularity for one head.

    sel: [N, M] bool.  A (tile, block) pair is computed when any row of the tile keeps the block.
    Returns (kept pairs, total pairs, kept (row, key) FLOP units = sum over kept pairs of
    rows_in_tile * n_j)."""
    M = sel.shape[1]
    n = np.array([min((j + 1) * block, N) - j * block for j in range(M)], np.int64)
    kept = 0
    units = 0
    T = (N + tile - 1) // tile
    for t in range(T):
        r0, r1 = t * tile, min((t + 1) * tile, N)
        u = sel[r0:r1].any(axis=0)
        kept += int(u.sum())
        units += int((r1 - r0) * n[u].sum())
    return kept, T * M, units


def threads(lib=None) -> int:
    """OpenMP threads the oracle runs on."""
    return int((lib or load()).sol_oracle_threads())
