"""Thin Python binding of libsolattn (ctypes over torch device tensors).

Argument marshalling only: every step of the forward pass runs in the HIP kernels of
libsolattn.so.  Names follow include/solattn.h.  The library must have been built
(``python -m block_sparse_attention_sol_amd.build``); there is no fallback -- a missing library
or a missing GPU raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsolattn.so")

SOL_OK = 0
SOL_EINVAL = -1
SOL_EUNSUPPORTED = -2
SOL_EWORKSPACE = -3
SOL_EHIP = -4
SOL_ENOTIMPL = -5
QUERY_TILE = 128

# Every symbol include/solattn.h declares.
EXPORTS = (
    "sol_attn_workspace_bytes",
    "sol_pool_kv",
    "sol_attn_fwd",
    "sol_attn_fwd_ex",
    "sol_attn_fwd_grid",
    "sol_attn_fwd_noalloc",
    "sol_attn_fwd_masked",
    "sol_proxy_map",
    "sol_select_topk",
    "sol_select_topp",
    "sol_mfma_probe",
    "sol_dense_fwd",
    "sol_attn_fwd_strided",
    "sol_dense_fwd_strided",
    "sol_status_str",
    "sol_last_error",
    "sol_version",
)


class SolShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("d", ctypes.c_int64)]


class SolStrides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("n", ctypes.c_int64)]


class SolGrid(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("W", ctypes.c_int64)]


class SolAttnDebug(ctypes.Structure):
    _fields_ = [("mask", ctypes.c_void_p), ("mu", ctypes.c_void_p), ("sigma", ctypes.c_void_p),
                ("tau", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("tile_kept", ctypes.c_void_p),
                ("out_f32", ctypes.c_void_p), ("drop_unselected", ctypes.c_int),
                ("events", ctypes.c_void_p * 4)]


class SolError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libsolattn error {status}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libsolattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m block_sparse_attention_sol_amd.build`")
    # torch first: its bundled HIP runtime carries the same soname, so the library binds to the
    # runtime (and streams) torch uses instead of loading a second copy.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, sz, ci, cf = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
    shp = ctypes.POINTER(SolShape)
    lib.sol_attn_workspace_bytes.argtypes = [shp, ci]
    lib.sol_attn_workspace_bytes.restype = sz
    lib.sol_pool_kv.argtypes = [shp, vp, vp, ci, vp, vp, vp]
    lib.sol_attn_fwd.argtypes = [shp, vp, vp, vp, cf, ci, vp, vp, sz, vp]
    lib.sol_attn_fwd_ex.argtypes = [shp, vp, vp, vp, cf, ci, vp, vp, sz,
                                    ctypes.POINTER(SolAttnDebug), vp]
    lib.sol_attn_fwd_noalloc.argtypes = [shp, vp, vp, vp, cf, ci, vp, vp]
    lib.sol_attn_fwd_grid.argtypes = [shp, ctypes.POINTER(SolGrid), vp, vp, vp, cf, ci, vp, vp, sz,
                                      ctypes.POINTER(SolAttnDebug), vp]
    lib.sol_dense_fwd.argtypes = [shp, vp, vp, vp, vp, vp, vp]
    lib.sol_mfma_probe.argtypes = [ci, ci, vp, vp]
    stp = ctypes.POINTER(SolStrides)
    lib.sol_attn_fwd_strided.argtypes = [shp, stp, stp, vp, vp, vp, cf, ci, vp, vp, sz, vp]
    lib.sol_dense_fwd_strided.argtypes = [shp, stp, stp, vp, vp, vp, vp, vp, vp]
    lib.sol_attn_fwd_masked.argtypes = [shp, vp, vp, vp, vp, ci, ci, vp, vp, sz, vp]
    lib.sol_proxy_map.argtypes = [shp, vp, vp, ci, vp, vp, sz, vp]
    lib.sol_select_topk.argtypes = [shp, ci, vp, ctypes.c_int64, vp, vp]
    lib.sol_select_topp.argtypes = [shp, ci, vp, cf, vp, vp]
    for f in ("sol_pool_kv", "sol_attn_fwd", "sol_attn_fwd_ex", "sol_attn_fwd_noalloc",
              "sol_dense_fwd", "sol_mfma_probe",
              "sol_attn_fwd_masked", "sol_proxy_map", "sol_select_topk", "sol_select_topp",
              "sol_attn_fwd_strided", "sol_dense_fwd_strided"):
        getattr(lib, f).restype = ci
    lib.sol_status_str.argtypes = [ci]
    lib.sol_status_str.restype = ctypes.c_char_p
    lib.sol_last_error.argtypes = []
    lib.sol_last_error.restype = ctypes.c_char_p
    lib.sol_version.argtypes = []
    lib.sol_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != SOL_OK:
        lib = load_library()
        raise SolError(status, lib.sol_last_error().decode() or lib.sol_status_str(status).decode())


def _shape(q) -> SolShape:
    B, H, N, d = q.shape
    return SolShape(B, H, N, d)


def _dev(t, name, strided: bool = False):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if strided:
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{name} must be a [B, H, N, d] view with contiguous d")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _strides(t) -> SolStrides:
    return SolStrides(t.stride(0), t.stride(1), t.stride(2))


def _strided_call(q, k, v, out) -> bool:
    """Whether the views need the strided entries (any non-contiguous tensor)."""
    if all(t.is_contiguous() for t in (q, k, v, out)):
        return False
    if not (q.stride() == k.stride() == v.stride()):
        raise ValueError("q, k and v must share one stride layout")
    return True


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def n_blocks(N: int, block: int) -> int:
    return (N + block - 1) // block


def workspace_bytes(shape, block: int) -> int:
    """Workspace size for a [B, H, N, d] shape (tuple or tensor)."""
    lib = load_library()
    B, H, N, d = tuple(shape.shape) if hasattr(shape, "shape") else tuple(shape)
    return int(lib.sol_attn_workspace_bytes(ctypes.byref(SolShape(B, H, N, d)), block))


def new_workspace(shape, block: int, device="cuda"):
    import torch
    return torch.empty(max(workspace_bytes(shape, block), 1), dtype=torch.uint8, device=device)


def pool_kv(k, v, block: int, stream=None):
    """Block means of K and V: fp32 [B, H, M, d] each."""
    import torch
    lib = load_library()
    B, H, N, d = k.shape
    M = n_blocks(N, block)
    kbar = torch.empty((B, H, M, d), dtype=torch.float32, device=k.device)
    vbar = torch.empty_like(kbar)
    _check(lib.sol_pool_kv(ctypes.byref(_shape(k)), _dev(k, "k"), _dev(v, "v"), block,
                           _dev(kbar, "kbar"), _dev(vbar, "vbar"), _stream(stream)))
    return kbar, vbar


def attn_fwd(q, k, v, beta: float, block: int, out=None, workspace=None, debug: bool = False,
             drop_unselected: bool = False, events=None, stream=None, grid=None):
    """Sol-Attn forward.  Returns out, or (out, dict of debug outputs) when debug/drop/events is
    set.  events: 4 raw hipEvent_t handles recorded at the kernel boundaries (see HipEvents).
    grid: the tokens' latent grid (T, H, W), passed to sol_attn_fwd_grid (same results; the
    fused kernel groups query rows by it)."""
    import torch
    lib = load_library()
    B, H, N, d = q.shape
    for t, n in ((k, "k"), (v, "v")):
        if t.shape != q.shape or t.dtype != torch.bfloat16:
            raise ValueError(f"{n} must be bf16 with the shape of q")
    if q.dtype != torch.bfloat16:
        raise ValueError("q must be bf16")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = new_workspace(q.shape, block, q.device)
    shp = _shape(q)
    if _strided_call(q, k, v, out):
        if debug or drop_unselected or events is not None or grid is not None:
            raise ValueError("debug outputs, the drop ablation and events need contiguous tensors")
        _check(lib.sol_attn_fwd_strided(ctypes.byref(shp), ctypes.byref(_strides(q)),
                                        ctypes.byref(_strides(out)), _dev(q, "q", True),
                                        _dev(k, "k", True), _dev(v, "v", True), float(beta), block,
                                        _dev(out, "out", True), _dev(workspace, "workspace"),
                                        workspace.numel(), _stream(stream)))
        return out
    if not debug and not drop_unselected and events is None and grid is None:
        _check(lib.sol_attn_fwd(ctypes.byref(shp), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
                                float(beta), block, _dev(out, "out"), _dev(workspace, "workspace"),
                                workspace.numel(), _stream(stream)))
        return out
    M = n_blocks(N, block)
    W = (M + 31) // 32
    T = (N + QUERY_TILE - 1) // QUERY_TILE
    dev = q.device
    dbg = {}
    dstruct = SolAttnDebug()
    if debug:
        dbg = {
            "mask": torch.empty((B, H, N, W), dtype=torch.int32, device=dev),
            "mu": torch.empty((B, H, N), dtype=torch.float32, device=dev),
            "sigma": torch.empty((B, H, N), dtype=torch.float32, device=dev),
            "tau": torch.empty((B, H, N), dtype=torch.float32, device=dev),
            "lse": torch.empty((B, H, N), dtype=torch.float32, device=dev),
            "tile_kept": torch.empty((B, H, T), dtype=torch.int32, device=dev),
            "out_f32": torch.empty((B, H, N, d), dtype=torch.float32, device=dev),
        }
        for key, t in dbg.items():
            setattr(dstruct, key, t.data_ptr())
    dstruct.drop_unselected = int(bool(drop_unselected))
    if events is not None:
        for i, e in enumerate(events):
            dstruct.events[i] = e
    if grid is not None:
        g = SolGrid(*[int(x) for x in grid])
        _check(lib.sol_attn_fwd_grid(ctypes.byref(shp), ctypes.byref(g), _dev(q, "q"),
                                     _dev(k, "k"), _dev(v, "v"), float(beta), block,
                                     _dev(out, "out"), _dev(workspace, "workspace"),
                                     workspace.numel(), ctypes.byref(dstruct), _stream(stream)))
        if not debug and not drop_unselected and events is None:
            return out
        return out, dbg
    _check(lib.sol_attn_fwd_ex(ctypes.byref(shp), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
                               float(beta), block, _dev(out, "out"), _dev(workspace, "workspace"),
                               workspace.numel(), ctypes.byref(dstruct), _stream(stream)))
    return out, dbg


NOALLOC_SCRATCH_BYTES = 256 << 20  # SOL_NOALLOC_SCRATCH_BYTES


def attn_fwd_noalloc(q, k, v, beta: float, block: int, out, stream=None):
    """sol_attn_fwd_noalloc: the forward pass with the library's own device scratch (no workspace
    argument, nothing allocated by the call).  q, k, v, out: contiguous bf16 [B, H, N, d]."""
    import torch
    lib = load_library()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        if t.shape != q.shape or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous bf16 with the shape of q")
    _check(lib.sol_attn_fwd_noalloc(ctypes.byref(_shape(q)), _dev(q, "q"), _dev(k, "k"),
                                    _dev(v, "v"), float(beta), block, _dev(out, "out"),
                                    _stream(stream)))
    return out


def dense_fwd(q, k, v, out=None, want_lse: bool = False, stream=None):
    """Dense attention softmax(q k^T / sqrt(d)) v.  Returns out (and lse if asked)."""
    import torch
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if want_lse else None
    if _strided_call(q, k, v, out):
        _check(lib.sol_dense_fwd_strided(ctypes.byref(_shape(q)), ctypes.byref(_strides(q)),
                                         ctypes.byref(_strides(out)), _dev(q, "q", True),
                                         _dev(k, "k", True), _dev(v, "v", True),
                                         _dev(out, "out", True),
                                         _dev(lse, "lse") if lse is not None else None,
                                         _stream(stream)))
        return (out, lse) if want_lse else out
    _check(lib.sol_dense_fwd(ctypes.byref(_shape(q)), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
                             _dev(out, "out"), _dev(lse, "lse") if lse is not None else None,
                             _stream(stream)))
    return (out, lse) if want_lse else out


def proxy_map(q, k, block: int, s_map=None, workspace=None, stream=None):
    """Full proxy map s_map [B, H, N, M] fp32 (row-major) of the prior-art routing pipeline."""
    import torch
    lib = load_library()
    B, H, N, d = q.shape
    M = n_blocks(N, block)
    if s_map is None:
        s_map = torch.empty((B, H, N, M), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = new_workspace(q.shape, block, q.device)
    _check(lib.sol_proxy_map(ctypes.byref(_shape(q)), _dev(q, "q"), _dev(k, "k"), block,
                             _dev(s_map, "s_map"), _dev(workspace, "workspace"), workspace.numel(),
                             _stream(stream)))
    return s_map


def _route_mask(q_shape, block, device):
    import torch
    B, H, N, _ = q_shape
    W = (n_blocks(N, block) + 31) // 32
    return torch.empty((B, H, N, W), dtype=torch.int32, device=device)


def select_topk(s_map, q_shape, block: int, k: int, mask=None, stream=None):
    """Top-k block selection per row from s_map; returns mask [B, H, N, ceil(M/32)] int32."""
    lib = load_library()
    if mask is None:
        mask = _route_mask(q_shape, block, s_map.device)
    _check(lib.sol_select_topk(ctypes.byref(SolShape(*q_shape)), block, _dev(s_map, "s_map"),
                               int(k), _dev(mask, "mask"), _stream(stream)))
    return mask


def select_topp(s_map, q_shape, block: int, p: float, mask=None, stream=None):
    """Top-p block selection per row from s_map; returns mask [B, H, N, ceil(M/32)] int32."""
    lib = load_library()
    if mask is None:
        mask = _route_mask(q_shape, block, s_map.device)
    _check(lib.sol_select_topp(ctypes.byref(SolShape(*q_shape)), block, _dev(s_map, "s_map"),
                               float(p), _dev(mask, "mask"), _stream(stream)))
    return mask


def attn_fwd_masked(q, k, v, mask, block: int, drop_unselected: bool = False, out=None,
                    workspace=None, stream=None):
    """Sol-Attn forward with the caller's selection mask [B, H, N, ceil(M/32)] (int32 words)."""
    import torch
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = new_workspace(q.shape, block, q.device)
    _check(lib.sol_attn_fwd_masked(ctypes.byref(_shape(q)), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
                                   _dev(mask, "mask"), block, int(bool(drop_unselected)),
                                   _dev(out, "out"), _dev(workspace, "workspace"), workspace.numel(),
                                   _stream(stream)))
    return out


MFMA_PROBE_FLOPS_PER_WAVE_ITER = 8 * 32768  # 8 independent 32x32x16 bf16 MFMAs


def mfma_probe(workgroups: int, iters: int, sink=None, stream=None):
    """Launch the matrix-core rate probe; returns (sink, FLOPs issued).  Time it with events."""
    import torch
    lib = load_library()
    if sink is None:
        sink = torch.empty(workgroups, dtype=torch.float32, device="cuda")
    _check(lib.sol_mfma_probe(int(workgroups), int(iters), _dev(sink, "sink"), _stream(stream)))
    return sink, float(workgroups) * 4 * iters * MFMA_PROBE_FLOPS_PER_WAVE_ITER


def kept_block_flops(tile_kept, mask, N: int, d: int, block: int) -> float:
    """Kept-block FLOPs F = 4*d*sum_t sum_{j kept by tile t} rows_t * n_j.

    tile_kept [B, H, T] (blocks computed per query tile) and mask [B, H, N, W] are the kernel's own
    debug outputs; the mask tells which tiles computed the (possibly partial) last block."""
    import torch
    T = tile_kept.shape[-1]
    M = n_blocks(N, block)
    n_last = N - (M - 1) * block
    rows = torch.full((T,), float(QUERY_TILE), dtype=torch.float64, device=tile_kept.device)
    rows[-1] = N - (T - 1) * QUERY_TILE
    kept = tile_kept.to(torch.float64).reshape(-1, T)
    units = (kept * block * rows).sum()
    if n_last != block:
        bit = (mask[..., (M - 1) // 32].to(torch.int64) >> ((M - 1) % 32)) & 1   # [B, H, N]
        pad = T * QUERY_TILE - N
        bit = torch.nn.functional.pad(bit.reshape(-1, N), (0, pad)).reshape(-1, T, QUERY_TILE)
        last_kept = bit.amax(dim=2).to(torch.float64)                            # [BH, T]
        units -= ((block - n_last) * last_kept * rows).sum()
    return float(4.0 * d * units)


def union_units(mask, N: int, block: int, heights=(1, 32, QUERY_TILE)) -> dict:
    """Computed (query row, key) pairs when a key block is computed for a group of `height`
    consecutive query rows whenever any row of the group keeps it: for each height,
    sum over groups g of sum over blocks j kept by some row of g of rows_g * n_j.

    Height 1 is the per-row selection itself, 32 the rows of one wave (a wave skips blocks none
    of its rows keeps), 128 the query tile.  mask [B, H, N, W] is the kernel's debug output.
    Returns {height: units}; FLOPs are 4 * d * units."""
    import torch
    B, H = mask.shape[0], mask.shape[1]
    M = n_blocks(N, block)
    dev = mask.device
    n = torch.full((M,), float(block), dtype=torch.float64, device=dev)
    n[-1] = float(N - (M - 1) * block)
    shifts = torch.arange(32, device=dev, dtype=torch.int32)
    out = {hgt: 0.0 for hgt in heights}
    for b in range(B):
        for h in range(H):
            bits = ((mask[b, h].view(torch.int32).unsqueeze(-1) >> shifts) & 1).to(torch.uint8)
            bits = bits.reshape(N, -1)[:, :M]                                  # [N, M]
            for hgt in heights:
                G = (N + hgt - 1) // hgt
                padded = torch.nn.functional.pad(bits, (0, 0, 0, G * hgt - N))
                u = padded.view(G, hgt, M).amax(dim=1).to(torch.float64)       # [G, M]
                rows = torch.full((G,), float(hgt), dtype=torch.float64, device=dev)
                rows[-1] = float(N - (G - 1) * hgt)
                out[hgt] += float((rows[:, None] * u * n[None, :]).sum())
            del bits
    return out


def dense_flops(B: int, H: int, N: int, d: int) -> float:
    return 4.0 * B * H * N * N * d


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch uses (for the library's timing hook)."""

    def __init__(self, n: int):
        import torch  # noqa: F401  (binds the runtime torch loaded)
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles.append(h.value)

    def record(self, i: int, stream=None):
        if self._hip.hipEventRecord(self.handles[i], _stream(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a: int, b: int) -> float:
        self._hip.hipEventSynchronize(self.handles[b])
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.handles[a], self.handles[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        for h in getattr(self, "handles", []):
            self._hip.hipEventDestroy(h)
