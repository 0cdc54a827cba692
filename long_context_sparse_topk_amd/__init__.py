"""Python binding of libdsa.so: one DeepSeek-Sparse-Attention layer on MI355X.

Thin ctypes marshalling over the C ABI in include/dsa.h: every step of the
layer runs in the HIP kernels of the library.  PyTorch provides device memory
and the current stream only.  There is no fallback: if the library is not
built, importing works but every call raises DsaLibraryMissing.

    idx = index_topk(q_idx, k_idx, w_idx, topk=512, q_chunk=256, q_pos=None)
    out, lse = sparse_attn_fwd(q, k, v, idx, q_pos=None, scale=None)
    dq, dk, dv = sparse_attn_bwd(q, k, v, out, dout, lse, idx, q_pos=None, scale=None)
    idx, out, lse = index_attn_fwd(q_idx, k_idx, w_idx, q, k, v, topk=512)  # pipelined

Shapes: q_idx [Sq, 4, 64], k_idx [Sk, 64], w_idx [Sq, 4] (bf16); q [Sq, H, 128],
k, v [Sk, 128] (bf16); idx [Sq, topk] int32; q_pos [Sq] int32 or None.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

HEAD_DIM = 128
IDX_DIM = 64
POOL = 4

STATUS = {0: "DSA_OK", 1: "DSA_INVALID_ARG", 2: "DSA_UNSUPPORTED_SHAPE",
          3: "DSA_WORKSPACE_TOO_SMALL", 4: "DSA_HIP_ERROR"}

# (name, restype, argtypes) of every symbol include/dsa.h declares
_P, _I64, _I32, _F, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "dsa_version": (ctypes.c_int, []),
    "dsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dsa_last_error": (ctypes.c_char_p, []),
    "dsa_index_topk_ws_bytes": (_SZ, [_I64, _I64, _I32, _I32, _I32, _I32, _I32]),
    "dsa_index_topk": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _I32,
                                      _P, _P, _SZ, _P]),
    "dsa_index_topk_fp8": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _I32,
                                          _P, _P, _SZ, _P]),
    "dsa_index_topk_stats": (ctypes.c_int, [_P, _SZ, _I64, _I64, _I32, _P, _P, _P]),
    "dsa_set_index_queries_per_wave": (ctypes.c_int, [_I32]),
    "dsa_sparse_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32,
                                           _F, _P, _P, _P]),
    "dsa_index_attn_fwd_ws_bytes": (_SZ, [_I64, _I64, _I32, _I32, _I32, _I32, _I32]),
    "dsa_index_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32,
                                          _I32, _I32, _I32, _I32, _F, _P, _P, _P, _P, _SZ, _P, _P]),
    "dsa_index_attn_fwd_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32,
                                              _I32, _I32, _I32, _I32, _F, _P, _P, _P, _P, _SZ, _P, _P]),
    "dsa_sparse_attn_bwd_ws_bytes": (_SZ, [_I64, _I64, _I32, _I32, _I32]),
    "dsa_sparse_attn_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I32, _I32,
                                           _I32, _I32, _F, _P, _P, _P, _P, _SZ, _P]),
    "dsa_sparse_attn_bwd_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I32,
                                                   _I32, _I32, _I32, _F, _P, _P, _P, _P]),
}


class DsaLibraryMissing(RuntimeError):
    pass


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libdsa.so (loading needs no GPU)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise DsaLibraryMissing(
                f"{LIB_PATH} is not built; run `python -m long_context_sparse_topk_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise DsaError(fn, status, lib().dsa_last_error().decode(errors="replace"))


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _want(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int, device: torch.device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out(t, name: str, dtype: torch.dtype, shape: tuple, device: torch.device):
    """A caller-provided buffer the kernels write: dtype, device, contiguity and exact shape,
    so that no write can leave it."""
    _want(t, name, dtype, len(shape), device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _kv_shapes(q, k, v):
    """k and v must both be [Sk, D] with q's head_dim D: the kernels read K/V rows at that
    stride, so any other width would send reads (and, in the backward, dk/dv writes) past
    the end of the buffers."""
    D = q.shape[2]
    Sk = k.shape[0]
    if tuple(k.shape) != (Sk, D) or tuple(v.shape) != (Sk, D):
        raise ValueError(f"attention shapes disagree: k {tuple(k.shape)} and v {tuple(v.shape)} "
                         f"must both be [Sk, {D}] (q's head_dim)")
    return Sk


def _positions(q_pos, Sq, device):
    if q_pos is None:
        return None
    _want(q_pos, "q_pos", torch.int32, 1, device)
    if q_pos.shape[0] != Sq:
        raise ValueError("q_pos must have Sq entries")
    return q_pos


def default_scale(head_dim: int = HEAD_DIM) -> float:
    return 1.0 / math.sqrt(head_dim)


# ---------------------------------------------------------------------------

def index_topk_ws_bytes(Sq: int, Sk: int, topk: int, idx_heads: int = 4, q_chunk: int = 256) -> int:
    return int(lib().dsa_index_topk_ws_bytes(Sq, Sk, idx_heads, IDX_DIM, POOL, topk, q_chunk))


def sparse_attn_bwd_ws_bytes(Sq: int, Sk: int, heads: int, topk: int) -> int:
    return int(lib().dsa_sparse_attn_bwd_ws_bytes(Sq, Sk, heads, HEAD_DIM, topk))


def index_topk(q_idx, k_idx, w_idx, *, topk: int, q_chunk: int = 256, q_pos=None,
               out=None, ws=None, fp8: bool = False) -> torch.Tensor:
    """Top-k pool ids [Sq, topk] int32, ascending, -1 padded.

    fp8=True calls dsa_index_topk_fp8: the same selection on e4m3 operands (exact, and
    equal to the bf16 path, for integer indexer inputs in [-3, 3])."""
    L = lib()
    dev = q_idx.device
    _want(q_idx, "q_idx", torch.bfloat16, 3, dev)
    _want(k_idx, "k_idx", torch.bfloat16, 2, dev)
    _want(w_idx, "w_idx", torch.bfloat16, 2, dev)
    Sq, HI, DI = q_idx.shape
    Sk = k_idx.shape[0]
    if k_idx.shape[1] != DI or tuple(w_idx.shape) != (Sq, HI):
        raise ValueError("indexer shapes disagree")
    q_pos = _positions(q_pos, Sq, dev)
    if out is None:
        out = torch.empty((Sq, topk), dtype=torch.int32, device=dev)
    else:
        _out(out, "out", torch.int32, (Sq, topk), dev)
    need = int(L.dsa_index_topk_ws_bytes(Sq, Sk, HI, DI, POOL, topk, q_chunk))
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    else:
        _want(ws, "ws", torch.uint8, 1, dev)
    fn = L.dsa_index_topk_fp8 if fp8 else L.dsa_index_topk
    st = fn(_ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(q_pos), Sq, Sk, HI, DI, POOL, topk, q_chunk,
            _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(dev))
    _check("dsa_index_topk_fp8" if fp8 else "dsa_index_topk", st)
    return out


def index_topk_stats(ws, *, Sq: int, Sk: int, topk: int) -> tuple:
    """(retried_rows, exact_rows) of the last indexer launch on workspace `ws` (a uint8
    device tensor passed to index_topk or index_attn_fwd): rows scored again with the
    wider threshold margin, and rows scored by the exact pass.  Synchronises the
    current stream."""
    dev = ws.device
    _want(ws, "ws", torch.uint8, 1, dev)
    retried, exact = ctypes.c_uint32(0), ctypes.c_uint32(0)
    st = lib().dsa_index_topk_stats(_ptr(ws), ws.numel(), Sq, Sk, topk, ctypes.addressof(retried),
                                    ctypes.addressof(exact), _stream(dev))
    _check("dsa_index_topk_stats", st)
    return int(retried.value), int(exact.value)


def set_index_queries_per_wave(queries_per_wave: int) -> None:
    """Force the indexer's workgroup sub-tile (4, 8 or 16 queries per wave) for every later
    call in this process, or 0 to let each call choose (the default).  A tuning and test
    setting: the selected ids do not depend on it."""
    _check("dsa_set_index_queries_per_wave", lib().dsa_set_index_queries_per_wave(int(queries_per_wave)))


def sparse_attn_fwd(q, k, v, idx, *, q_pos=None, scale: float | None = None, out=None, lse=None):
    """(out [Sq, H, 128] bf16, lse [Sq, H] fp32)."""
    L = lib()
    dev = q.device
    _want(q, "q", torch.bfloat16, 3, dev)
    _want(k, "k", torch.bfloat16, 2, dev)
    _want(v, "v", torch.bfloat16, 2, dev)
    _want(idx, "idx", torch.int32, 2, dev)
    Sq, H, D = q.shape
    Sk = _kv_shapes(q, k, v)
    if idx.shape[0] != Sq:
        raise ValueError("attention shapes disagree: idx must have Sq rows")
    q_pos = _positions(q_pos, Sq, dev)
    scale = default_scale(D) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else _out(out, "out", torch.bfloat16, (Sq, H, D), dev)
    lse = (torch.empty((Sq, H), dtype=torch.float32, device=dev) if lse is None
           else _out(lse, "lse", torch.float32, (Sq, H), dev))
    st = L.dsa_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(q_pos), Sq, Sk, H, D, POOL,
                               idx.shape[1], scale, _ptr(out), _ptr(lse), _stream(dev))
    _check("dsa_sparse_attn_fwd", st)
    return out, lse


_aux_streams = {}


def _aux_stream(dev):
    """A second stream of the device (default priority) for the pipelined forward."""
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    if key not in _aux_streams:
        _aux_streams[key] = torch.cuda.Stream(device=dev)
    return _aux_streams[key]


def index_attn_fwd(q_idx, k_idx, w_idx, q, k, v, *, topk: int, q_chunk: int = 256, q_pos=None,
                   scale: float | None = None, idx=None, out=None, lse=None, ws=None,
                   aux_stream=None, fp8: bool = False):
    """index_topk then sparse_attn_fwd, pipelined over query chunks on two streams.

    Returns (idx [Sq, topk] int32, out [Sq, H, 128] bf16, lse [Sq, H] fp32), equal bit for
    bit to the two separate calls.  The current stream waits for all of the work on return.
    fp8=True uses the fp8 indexer (dsa_index_attn_fwd_fp8).
    """
    L = lib()
    dev = q_idx.device
    _want(q_idx, "q_idx", torch.bfloat16, 3, dev)
    _want(k_idx, "k_idx", torch.bfloat16, 2, dev)
    _want(w_idx, "w_idx", torch.bfloat16, 2, dev)
    _want(q, "q", torch.bfloat16, 3, dev)
    _want(k, "k", torch.bfloat16, 2, dev)
    _want(v, "v", torch.bfloat16, 2, dev)
    Sq, HI, DI = q_idx.shape
    Sk = k_idx.shape[0]
    H, D = q.shape[1], q.shape[2]
    if k_idx.shape[1] != DI or tuple(w_idx.shape) != (Sq, HI):
        raise ValueError("indexer shapes disagree")
    if q.shape[0] != Sq or _kv_shapes(q, k, v) != Sk:
        raise ValueError("attention shapes disagree: q must have Sq rows and k, v Sk rows")
    q_pos = _positions(q_pos, Sq, dev)
    scale = default_scale(D) if scale is None else float(scale)
    idx = (torch.empty((Sq, topk), dtype=torch.int32, device=dev) if idx is None
           else _out(idx, "idx", torch.int32, (Sq, topk), dev))
    out = torch.empty_like(q) if out is None else _out(out, "out", torch.bfloat16, (Sq, H, D), dev)
    lse = (torch.empty((Sq, H), dtype=torch.float32, device=dev) if lse is None
           else _out(lse, "lse", torch.float32, (Sq, H), dev))
    need = int(L.dsa_index_attn_fwd_ws_bytes(Sq, Sk, HI, DI, POOL, topk, q_chunk))
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    else:
        _want(ws, "ws", torch.uint8, 1, dev)
    aux = _aux_stream(dev) if aux_stream is None else aux_stream
    fn = L.dsa_index_attn_fwd_fp8 if fp8 else L.dsa_index_attn_fwd
    st = fn(_ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(q), _ptr(k), _ptr(v), _ptr(q_pos), Sq, Sk, HI,
            DI, H, D, POOL, topk, q_chunk, scale, _ptr(idx), _ptr(out), _ptr(lse), _ptr(ws),
            ws.numel() * ws.element_size(), _stream(dev), ctypes.c_void_p(aux.cuda_stream))
    _check("dsa_index_attn_fwd_fp8" if fp8 else "dsa_index_attn_fwd", st)
    return idx, out, lse


def sparse_attn_bwd(q, k, v, out, dout, lse, idx, *, q_pos=None, scale: float | None = None,
                    ws=None, dq=None, dk=None, dv=None):
    """(dq [Sq, H, 128], dk [Sk, 128], dv [Sk, 128]) bf16."""
    L = lib()
    dev = q.device
    for t, n, nd in ((q, "q", 3), (k, "k", 2), (v, "v", 2), (out, "out", 3), (dout, "dout", 3)):
        _want(t, n, torch.bfloat16, nd, dev)
    _want(lse, "lse", torch.float32, 2, dev)
    _want(idx, "idx", torch.int32, 2, dev)
    Sq, H, D = q.shape
    Sk = _kv_shapes(q, k, v)
    q_pos = _positions(q_pos, Sq, dev)
    scale = default_scale(D) if scale is None else float(scale)
    if tuple(out.shape) != (Sq, H, D) or tuple(dout.shape) != (Sq, H, D) or \
            tuple(lse.shape) != (Sq, H) or idx.shape[0] != Sq:
        raise ValueError("attention shapes disagree")
    dq = torch.empty_like(q) if dq is None else _out(dq, "dq", torch.bfloat16, (Sq, H, D), dev)
    dk = torch.empty_like(k) if dk is None else _out(dk, "dk", torch.bfloat16, (Sk, D), dev)
    dv = torch.empty_like(v) if dv is None else _out(dv, "dv", torch.bfloat16, (Sk, D), dev)
    need = int(L.dsa_sparse_attn_bwd_ws_bytes(Sq, Sk, H, D, idx.shape[1]))
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    else:
        _want(ws, "ws", torch.uint8, 1, dev)
    st = L.dsa_sparse_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(idx),
                               _ptr(q_pos), Sq, Sk, H, D, POOL, idx.shape[1], scale, _ptr(dq),
                               _ptr(dk), _ptr(dv), _ptr(ws), ws.numel() * ws.element_size(),
                               _stream(dev))
    _check("dsa_sparse_attn_bwd", st)
    return dq, dk, dv


def sparse_attn_bwd_noalloc(q, k, v, out, dout, lse, idx, *, q_pos=None, scale: float | None = None,
                            dq=None, dk=None, dv=None):
    """sparse_attn_bwd without a workspace: the library uses its own device-resident scratch
    (at most 96 MiB of workspace), so the call allocates nothing when dq, dk and dv are
    given.  Calls that overlap on one GPU race (they share the scratch)."""
    L = lib()
    dev = q.device
    for t, n, nd in ((q, "q", 3), (k, "k", 2), (v, "v", 2), (out, "out", 3), (dout, "dout", 3)):
        _want(t, n, torch.bfloat16, nd, dev)
    _want(lse, "lse", torch.float32, 2, dev)
    _want(idx, "idx", torch.int32, 2, dev)
    Sq, H, D = q.shape
    Sk = _kv_shapes(q, k, v)
    q_pos = _positions(q_pos, Sq, dev)
    scale = default_scale(D) if scale is None else float(scale)
    if tuple(out.shape) != (Sq, H, D) or tuple(dout.shape) != (Sq, H, D) or \
            tuple(lse.shape) != (Sq, H) or idx.shape[0] != Sq:
        raise ValueError("attention shapes disagree")
    dq = torch.empty_like(q) if dq is None else _out(dq, "dq", torch.bfloat16, (Sq, H, D), dev)
    dk = torch.empty_like(k) if dk is None else _out(dk, "dk", torch.bfloat16, (Sk, D), dev)
    dv = torch.empty_like(v) if dv is None else _out(dv, "dv", torch.bfloat16, (Sk, D), dev)
    st = L.dsa_sparse_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                       _ptr(idx), _ptr(q_pos), Sq, Sk, H, D, POOL, idx.shape[1], scale,
                                       _ptr(dq), _ptr(dk), _ptr(dv), _stream(dev))
    _check("dsa_sparse_attn_bwd_noalloc", st)
    return dq, dk, dv
