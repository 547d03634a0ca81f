"""Python binding of libhstu (HSTU attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libhstu.so``.  PyTorch supplies device memory and the current
stream.  The functions mirror the HSTU Attention page's allocating functions
("High-level functions"): ``hstu_fwd`` returns the packed output, ``hstu_bwd``
returns (dq, dk, dv); caller-owned outputs may be passed in and are
overwritten.  ``causal=True`` is the page's ``window_size=(-1, 0)`` and
``causal=False`` its ``(-1, -1)``; ``window_size=(left, right)``, when given,
sets the mask instead ("Mask support": key j visible to query i iff
i - left <= j <= i + right, -1 = unbounded); ``func=`` (a device int32 tensor of
shape ``(N, L)`` or the page's ``(1, N, L)``, N odd, L >= T_q) selects the
arbitrary mask: packed query row r sees the local keys
``[0, F0) u [F1, F2) u ...`` with ``F_n = func[..., n, r]``.  There is no
fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

__all__ = [
    "HstuError",
    "HstuArgs",
    "HstuStride",
    "library",
    "library_path",
    "select_library",
    "debug_take",
    "hstu_fwd",
    "hstu_bwd",
    "hstu_bwd_workspace_size",
    "hstu_bwd_dq",
    "hstu_bwd_dkdv",
    "hstu_bwd_dkdv_ds",
    "hstu_bwd_dq_ds",
    "hstu_bwd_fused",
    "HSTU_OK",
    "HSTU_ERR_INVALID_ARGUMENT",
    "HSTU_ERR_UNSUPPORTED",
    "HSTU_ERR_DEVICE",
    "HSTU_MASK_NONE",
    "HSTU_MASK_CAUSAL",
    "HSTU_MASK_WINDOW",
    "HSTU_MASK_FUNC",
    "HstuLmsdArgs",
    "lmsd_fwd",
    "lmsd_bwd",
    "lmsd_bwd_workspace_size",
    "lmsd_bwd_noalloc",
    "clock_sample",
]

HSTU_OK = 0
HSTU_ERR_INVALID_ARGUMENT = 1
HSTU_ERR_UNSUPPORTED = 2
HSTU_ERR_DEVICE = 3
HSTU_MASK_NONE = 0
HSTU_MASK_CAUSAL = 1
HSTU_MASK_WINDOW = 2
HSTU_MASK_FUNC = 3
ABI_VERSION = 7

_PKG = os.path.dirname(os.path.abspath(__file__))
_lock = threading.Lock()
_libs = {}
# The debug build (bounds tests on the kernels' global indices, read back with
# debug_take) is selected by HSTU_DEBUG=1 in the environment or select_library().
_debug = os.environ.get("HSTU_DEBUG", "") == "1"


def library_path(debug: Optional[bool] = None) -> str:
    d = _debug if debug is None else debug
    return os.path.join(_PKG, "libhstu_debug.so" if d else "libhstu.so")


def select_library(debug: bool) -> bool:
    """Route the calls of this module to the debug build (True) or the release
    build (False); each is loaded on first use and stays loaded.  Returns the
    previous choice."""
    global _debug
    prev, _debug = _debug, bool(debug)
    return prev


class HstuStride(ctypes.Structure):
    _fields_ = [("token", ctypes.c_int64), ("head", ctypes.c_int64)]


class HstuArgs(ctypes.Structure):
    """Mirror of ``hstu_args_t`` in include/hstu.h."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("total_k", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32),
        ("alpha", ctypes.c_float),
        ("scaling_seqlen", ctypes.c_int32),
        ("mask", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("func_n", ctypes.c_int32),
        ("func_ld", ctypes.c_int32),
        ("func", ctypes.c_void_p),
        ("q", HstuStride),
        ("k", HstuStride),
        ("v", HstuStride),
        ("o", HstuStride),
        ("dout", HstuStride),
        ("dq", HstuStride),
        ("dk", HstuStride),
        ("dv", HstuStride),
    ]


class HstuLmsdArgs(ctypes.Structure):
    """Mirror of ``hstu_lmsd_args_t`` in include/hstu.h."""

    _fields_ = [
        ("n", ctypes.c_int64),
        ("x_stride", ctypes.c_int64),
        ("u_stride", ctypes.c_int64),
        ("dy_stride", ctypes.c_int64),
        ("dx_stride", ctypes.c_int64),
        ("du_stride", ctypes.c_int64),
        ("d", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("dropout_ratio", ctypes.c_float),
        ("apply_u_silu", ctypes.c_int32),
        ("concat_u", ctypes.c_int32),
        ("concat_x", ctypes.c_int32),
        ("compute_dweight", ctypes.c_int32),
    ]


class HstuError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


def _status_name(s: int) -> str:
    return {0: "HSTU_OK", 1: "HSTU_ERR_INVALID_ARGUMENT", 2: "HSTU_ERR_UNSUPPORTED",
            3: "HSTU_ERR_DEVICE"}.get(s, f"status {s}")


def library(debug: Optional[bool] = None) -> ctypes.CDLL:
    """Load ``libhstu.so`` (or, for the debug build, ``libhstu_debug.so``; both built
    in-tree); raise if it is missing."""
    d = _debug if debug is None else bool(debug)
    with _lock:
        if d not in _libs:
            path = library_path(d)
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{os.path.basename(path)} not found at {path}; build it with "
                    "`python -m generative_recommender_attention_amd.build` (there is no fallback)")
            lib = ctypes.CDLL(path)
            vp = ctypes.c_void_p
            argp = ctypes.POINTER(HstuArgs)
            lib.hstu_fwd.restype = ctypes.c_int
            lib.hstu_fwd.argtypes = [argp, vp, vp, vp, vp, vp, vp, vp]
            lib.hstu_bwd.restype = ctypes.c_int
            lib.hstu_bwd.argtypes = [argp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
            lib.hstu_bwd_workspace_size.restype = ctypes.c_int
            lib.hstu_bwd_workspace_size.argtypes = [argp, ctypes.POINTER(ctypes.c_size_t)]
            lib.hstu_bwd_dq.restype = ctypes.c_int
            lib.hstu_bwd_dq.argtypes = [argp, vp, vp, vp, vp, vp, vp, vp, vp]
            lib.hstu_bwd_dkdv.restype = ctypes.c_int
            lib.hstu_bwd_dkdv.argtypes = [argp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
            lib.hstu_bwd_dkdv_ds.restype = ctypes.c_int
            lib.hstu_bwd_dkdv_ds.argtypes = [argp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
            lib.hstu_bwd_fused_workspace_size.restype = ctypes.c_int
            lib.hstu_bwd_fused_workspace_size.argtypes = [argp, ctypes.POINTER(ctypes.c_size_t)]
            lib.hstu_bwd_fused.restype = ctypes.c_int
            lib.hstu_bwd_fused.argtypes = [argp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
            lib.hstu_bwd_dq_ds.restype = ctypes.c_int
            lib.hstu_bwd_dq_ds.argtypes = [argp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp]
            largp = ctypes.POINTER(HstuLmsdArgs)
            lib.hstu_lmsd_fwd.restype = ctypes.c_int
            lib.hstu_lmsd_fwd.argtypes = [largp, vp, vp, vp, vp, vp, vp, vp, vp]
            lib.hstu_lmsd_bwd_workspace_size.restype = ctypes.c_int
            lib.hstu_lmsd_bwd_workspace_size.argtypes = [largp, ctypes.POINTER(ctypes.c_size_t)]
            lib.hstu_lmsd_bwd.restype = ctypes.c_int
            lib.hstu_lmsd_bwd.argtypes = [largp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
            lib.hstu_lmsd_bwd_noalloc.restype = ctypes.c_int
            lib.hstu_lmsd_bwd_noalloc.argtypes = [largp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
            lib.hstu_clock_sample.restype = ctypes.c_int
            lib.hstu_clock_sample.argtypes = [vp, ctypes.c_int32, vp]
            lib.hstu_debug_take.restype = ctypes.c_int
            lib.hstu_debug_take.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
            lib.hstu_last_error.restype = ctypes.c_char_p
            lib.hstu_last_error.argtypes = []
            lib.hstu_status_string.restype = ctypes.c_char_p
            lib.hstu_status_string.argtypes = [ctypes.c_int]
            lib.hstu_abi_version.restype = ctypes.c_int
            lib.hstu_abi_version.argtypes = []
            if lib.hstu_abi_version() != ABI_VERSION:
                raise RuntimeError(f"libhstu ABI {lib.hstu_abi_version()} != binding ABI {ABI_VERSION}")
            _libs[d] = lib
        return _libs[d]


def _check(status: int) -> None:
    if status == HSTU_OK:
        return
    msg = library().hstu_last_error().decode(errors="replace")
    if status == HSTU_ERR_UNSUPPORTED:
        raise NotImplementedError(f"{_status_name(status)}: {msg}")
    raise HstuError(status, msg)


def _thd(name: str, t: torch.Tensor, rows: Optional[int], H: int, D: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if t.dim() != 3 or t.shape[1] != H or t.shape[2] != D or (rows is not None and t.shape[0] != rows):
        want = f"({rows if rows is not None else 'T'}, {H}, {D})"
        raise ValueError(f"{name} must have shape {want}, got {tuple(t.shape)}")
    if t.shape[0] > 0 and t.stride(2) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension")


def _stride(t: torch.Tensor) -> HstuStride:
    return HstuStride(t.stride(0), t.stride(1))


def _cu(name: str, t: torch.Tensor, device: torch.device) -> int:
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.dim() != 1:
        raise TypeError(f"{name} must be a 1-D int32 tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _launch_stream(stream, device):
    """The stream the kernels go to, as a torch stream: the current one when none is
    given; a raw ``hipStream_t`` handle is wrapped.  Every tensor a function
    allocates (outputs, workspaces) is allocated while this stream is current, so
    the caching allocator hands a block freed at return to later work on the same
    stream only, which the stream orders after the kernels that used it."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    handle = int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.ExternalStream(handle, device=device)


def _stream(s) -> int:
    return int(s.cuda_stream)


def _args(q, k, cu_q, max_seqlen_q, max_seqlen_k, alpha, scaling_seqlen, causal, window_size,
          func=None) -> HstuArgs:
    a = HstuArgs()
    a.batch = int(cu_q.shape[0]) - 1
    a.total_q = int(q.shape[0])
    a.total_k = int(k.shape[0])
    a.num_heads = int(q.shape[1])
    a.head_dim = int(q.shape[2])
    a.max_seqlen_q = int(max_seqlen_q)
    a.max_seqlen_k = int(max_seqlen_k)
    a.alpha = float(alpha)
    a.scaling_seqlen = 0 if scaling_seqlen is None else int(scaling_seqlen)
    if func is not None:
        if window_size is not None:
            raise ValueError("func and window_size cannot be combined")
        if not isinstance(func, torch.Tensor) or func.dtype != torch.int32:
            raise TypeError("func must be an int32 tensor")
        f = func[0] if func.dim() == 3 else func
        if f.dim() != 2 or f.device != q.device or f.stride(1) != 1:
            raise ValueError("func must be (N, L) or (1, N, L) on the device of q, rows contiguous")
        if f.shape[0] % 2 != 1 or f.shape[1] < q.shape[0]:
            raise ValueError("func needs an odd number of endpoint rows of at least T_q columns")
        a.mask, a.func_n, a.func_ld, a.func = HSTU_MASK_FUNC, int(f.shape[0]), int(f.stride(0)), f.data_ptr()
    elif window_size is None:
        a.mask = HSTU_MASK_CAUSAL if causal else HSTU_MASK_NONE
    else:
        left, right = (int(w) for w in window_size)
        a.mask, a.window_left, a.window_right = HSTU_MASK_WINDOW, left, right
    if scaling_seqlen is not None and int(scaling_seqlen) <= 0:
        raise ValueError("scaling_seqlen must be positive")
    return a


def _inputs(q, k, v, cu_q, cu_k):
    if q.dim() != 3:
        raise ValueError("q must be (T_q, H, D)")
    H, D = int(q.shape[1]), int(q.shape[2])
    _thd("q", q, None, H, D)
    _thd("k", k, None, H, D)
    _thd("v", v, int(k.shape[0]), H, D)
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on one device")
    pq, pk = _cu("cu_seqlens_q", cu_q, q.device), _cu("cu_seqlens_k", cu_k, q.device)
    if cu_q.shape != cu_k.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have B + 1 entries")
    return H, D, pq, pk


def hstu_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
             cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
             max_seqlen_q: int, max_seqlen_k: int, alpha: float = 1.0,
             scaling_seqlen: Optional[int] = None, causal: bool = True,
             out: Optional[torch.Tensor] = None, stream=None,
             window_size: Optional[Tuple[int, int]] = None, func: Optional[torch.Tensor] = None) -> torch.Tensor:
    """O = HSTU(q, k, v) on packed (T, H, D) bf16 tensors; returns ``out``."""
    H, D, pq, pk = _inputs(q, k, v, cu_seqlens_q, cu_seqlens_k)
    s = _launch_stream(stream, q.device)
    with torch.cuda.stream(s):
        if out is None:
            out = torch.empty_like(q, memory_format=torch.contiguous_format)
        _thd("out", out, int(q.shape[0]), H, D)
        a = _args(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_k, alpha, scaling_seqlen, causal, window_size, func)
        a.q, a.k, a.v, a.o = _stride(q), _stride(k), _stride(v), _stride(out)
        _check(library().hstu_fwd(ctypes.byref(a), q.data_ptr(), k.data_ptr(), v.data_ptr(), pq, pk,
                                  out.data_ptr(), _stream(s)))
    return out


def _bwd_common(dout, q, k, v, cu_q, cu_k, max_seqlen_q, max_seqlen_k, alpha, scaling_seqlen, causal,
                window_size, func=None):
    H, D, pq, pk = _inputs(q, k, v, cu_q, cu_k)
    _thd("dout", dout, int(q.shape[0]), H, D)
    a = _args(q, k, cu_q, max_seqlen_q, max_seqlen_k, alpha, scaling_seqlen, causal, window_size, func)
    a.q, a.k, a.v, a.dout = _stride(q), _stride(k), _stride(v), _stride(dout)
    return H, D, pq, pk, a


def hstu_bwd(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
             cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
             max_seqlen_q: int, max_seqlen_k: int, alpha: float = 1.0,
             scaling_seqlen: Optional[int] = None, causal: bool = True,
             dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
             dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None,
             window_size: Optional[Tuple[int, int]] = None, func: Optional[torch.Tensor] = None,
             store_ds: bool = True) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(dq, dk, dv) of HSTU attention for upstream gradient ``dout``.

    With ``store_ds`` the dk/dv kernel stores dS in ``workspace`` (a device byte
    tensor of ``hstu_bwd_workspace_size`` bytes, allocated here when not given) and
    dq is computed from it; with ``store_ds=False`` the dq kernel recomputes the
    scores and no workspace is used."""
    H, D, pq, pk, a = _bwd_common(dout, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                                  max_seqlen_k, alpha, scaling_seqlen, causal, window_size, func)
    s = _launch_stream(stream, q.device)
    with torch.cuda.stream(s):  # a workspace allocated here is freed on s, after the kernels
        dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
        dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
        dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
        _thd("dq", dq, int(q.shape[0]), H, D)
        _thd("dk", dk, int(k.shape[0]), H, D)
        _thd("dv", dv, int(k.shape[0]), H, D)
        a.dq, a.dk, a.dv = _stride(dq), _stride(dk), _stride(dv)
        need = ctypes.c_size_t(0)
        _check(library().hstu_bwd_workspace_size(ctypes.byref(a), ctypes.byref(need)))
        if not store_ds or need.value == 0:
            workspace = None
        elif workspace is None:
            workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = _workspace(workspace)
        _check(library().hstu_bwd(ctypes.byref(a), dout.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  pq, pk, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws_ptr, ws_bytes,
                                  _stream(s)))
    return dq, dk, dv


def hstu_bwd_fused(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                   max_seqlen_q: int, max_seqlen_k: int, alpha: float = 1.0,
                   scaling_seqlen: Optional[int] = None, causal: bool = True,
                   dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                   dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None,
                   window_size: Optional[Tuple[int, int]] = None, func: Optional[torch.Tensor] = None
                   ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(dq, dk, dv) through the fused single-pass backward (dQ added with fp32 atomics
    into ``workspace``, a device byte tensor of at least T_q H D 4 bytes, allocated here
    when not given); dQ's last bits may differ between calls."""
    H, D, pq, pk, a = _bwd_common(dout, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                                  max_seqlen_k, alpha, scaling_seqlen, causal, window_size, func)
    s = _launch_stream(stream, q.device)
    with torch.cuda.stream(s):
        dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
        dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
        dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
        _thd("dq", dq, int(q.shape[0]), H, D)
        _thd("dk", dk, int(k.shape[0]), H, D)
        _thd("dv", dv, int(k.shape[0]), H, D)
        a.dq, a.dk, a.dv = _stride(dq), _stride(dk), _stride(dv)
        need = ctypes.c_size_t(0)
        _check(library().hstu_bwd_fused_workspace_size(ctypes.byref(a), ctypes.byref(need)))
        if workspace is None and need.value > 0:
            workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = _workspace(workspace)
        _check(library().hstu_bwd_fused(ctypes.byref(a), dout.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        pq, pk, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws_ptr, ws_bytes,
                                        _stream(s)))
    return dq, dk, dv


def _workspace(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    if not isinstance(ws, torch.Tensor) or ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def hstu_bwd_workspace_size(dout, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                            alpha=1.0, scaling_seqlen=None, causal=True, window_size=None, func=None) -> int:
    """Bytes of device workspace ``hstu_bwd`` needs for this problem."""
    _, _, _, _, a = _bwd_common(dout, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, alpha,
                                scaling_seqlen, causal, window_size, func)
    need = ctypes.c_size_t(0)
    _check(library().hstu_bwd_workspace_size(ctypes.byref(a), ctypes.byref(need)))
    return int(need.value)


def hstu_bwd_dq(dout, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                alpha=1.0, scaling_seqlen=None, causal=True, dq=None, stream=None,
                window_size=None, func=None) -> torch.Tensor:
    """dq only (the query-major backward kernel)."""
    H, D, pq, pk, a = _bwd_common(dout, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                                  max_seqlen_k, alpha, scaling_seqlen, causal, window_size, func)
    s = _launch_stream(stream, q.device)
    with torch.cuda.stream(s):
        dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
        _thd("dq", dq, int(q.shape[0]), H, D)
        a.dq = _stride(dq)
        _check(library().hstu_bwd_dq(ctypes.byref(a), dout.data_ptr(), q.data_ptr(), k.data_ptr(),
                                     v.data_ptr(), pq, pk, dq.data_ptr(), _stream(s)))
    return dq


def hstu_bwd_dkdv(dout, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                  alpha=1.0, scaling_seqlen=None, causal=True, dk=None, dv=None, stream=None,
                  window_size=None, func=None):
    """(dk, dv) only (the key-major backward kernel)."""
    H, D, pq, pk, a = _bwd_common(dout, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                                  max_seqlen_k, alpha, scaling_seqlen, causal, window_size, func)
    s = _launch_stream(stream, q.device)
    with torch.cuda.stream(s):
        dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
        dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
        _thd("dk", dk, int(k.shape[0]), H, D)
        _thd("dv", dv, int(k.shape[0]), H, D)
        a.dk, a.dv = _stride(dk), _stride(dv)
        _check(library().hstu_bwd_dkdv(ctypes.byref(a), dout.data_ptr(), q.data_ptr(), k.data_ptr(),
                                       v.data_ptr(), pq, pk, dk.data_ptr(), dv.data_ptr(), _stream(s)))
    return dk, dv


# ---------------------------------------------------------------------------
# HSTU LMSD (HSTU LMSD page: hstu_lmsd_forward / hstu_lmsd_backward)
# ---------------------------------------------------------------------------
def _rowmat(name: str, t: torch.Tensor, n: Optional[int], d: int) -> int:
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be a bfloat16 tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if t.dim() != 2 or t.shape[1] != d or (n is not None and t.shape[0] != n):
        raise ValueError(f"{name} must have shape ({n if n is not None else 'N'}, {d}), got {tuple(t.shape)}")
    if t.shape[0] > 0 and t.stride(1) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension")
    return int(t.stride(0)) if t.shape[0] > 1 else d


def _vec(name: str, t: torch.Tensor, d: int, dtype=torch.bfloat16) -> None:
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.dim() != 1 or t.shape[0] != d or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous ({d},) {dtype} tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")


def _lmsd_args(x, u, eps, dropout_ratio, apply_u_silu, concat_u, concat_x, compute_dweight=True) -> HstuLmsdArgs:
    if x.dim() != 2:
        raise ValueError("x must be (N, D)")
    n, d = int(x.shape[0]), int(x.shape[1])
    a = HstuLmsdArgs()
    a.n, a.d = n, d
    a.eps, a.dropout_ratio = float(eps), float(dropout_ratio)
    a.apply_u_silu, a.concat_u, a.concat_x = int(bool(apply_u_silu)), int(bool(concat_u)), int(bool(concat_x))
    a.compute_dweight = int(bool(compute_dweight))
    a.x_stride = _rowmat("x", x, n, d)
    a.u_stride = _rowmat("u", u, n, d)
    return a


def lmsd_fwd(x: torch.Tensor, u: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor, eps: float = 1e-6,
             dropout_ratio: float = 0.0, apply_u_silu: bool = True, concat_u: bool = True, concat_x: bool = True,
             y: Optional[torch.Tensor] = None, mean: Optional[torch.Tensor] = None,
             rstd: Optional[torch.Tensor] = None, stream=None):
    """(y, mean, rstd): y = [a, x, LayerNorm(x) * a] per row (segments as flagged),
    a = SiLU(u) or u; mean and rstd are the fp32 row statistics the backward needs."""
    a = _lmsd_args(x, u, eps, dropout_ratio, apply_u_silu, concat_u, concat_x)
    n, d = a.n, a.d
    _vec("weight", weight, d)
    _vec("bias", bias, d)
    segs = 1 + a.concat_u + a.concat_x
    s = _launch_stream(stream, x.device)
    with torch.cuda.stream(s):
        y = torch.empty((n, segs * d), dtype=torch.bfloat16, device=x.device) if y is None else y
        if y.shape != (n, segs * d) or y.dtype != torch.bfloat16 or not y.is_contiguous():
            raise ValueError(f"y must be a contiguous ({n}, {segs * d}) bfloat16 tensor")
        mean = torch.empty(n, dtype=torch.float32, device=x.device) if mean is None else mean
        rstd = torch.empty(n, dtype=torch.float32, device=x.device) if rstd is None else rstd
        _vec("mean", mean, n, torch.float32)
        _vec("rstd", rstd, n, torch.float32)
        _check(library().hstu_lmsd_fwd(ctypes.byref(a), x.data_ptr(), u.data_ptr(), weight.data_ptr(),
                                       bias.data_ptr(), y.data_ptr(), mean.data_ptr(), rstd.data_ptr(), _stream(s)))
    return y, mean, rstd


def lmsd_bwd_workspace_size(x, u, eps=1e-6, dropout_ratio=0.0, apply_u_silu=True, concat_u=True, concat_x=True,
                            compute_dweight=True) -> int:
    a = _lmsd_args(x, u, eps, dropout_ratio, apply_u_silu, concat_u, concat_x, compute_dweight)
    need = ctypes.c_size_t(0)
    _check(library().hstu_lmsd_bwd_workspace_size(ctypes.byref(a), ctypes.byref(need)))
    return int(need.value)


def lmsd_bwd(dy: torch.Tensor, x: torch.Tensor, u: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor,
             mean: torch.Tensor, rstd: torch.Tensor, dropout_ratio: float = 0.0, apply_u_silu: bool = True,
             concat_u: bool = True, concat_x: bool = True, compute_dweight: bool = True, eps: float = 1e-6,
             dx=None, du=None, dweight=None, dbias=None, workspace=None, stream=None):
    """(dx, du, dweight or None, dbias) from the upstream gradient dy of y and the
    forward's saved mean and rstd (the same flags as the forward)."""
    a = _lmsd_args(x, u, eps, dropout_ratio, apply_u_silu, concat_u, concat_x, compute_dweight)
    n, d = a.n, a.d
    segs = 1 + a.concat_u + a.concat_x
    a.dy_stride = _rowmat("dy", dy, n, segs * d)
    _vec("weight", weight, d)
    _vec("bias", bias, d)
    _vec("mean", mean, n, torch.float32)
    _vec("rstd", rstd, n, torch.float32)
    s = _launch_stream(stream, x.device)
    with torch.cuda.stream(s):  # a workspace allocated here is freed on s, after the kernels
        dx = torch.empty((n, d), dtype=torch.bfloat16, device=x.device) if dx is None else dx
        du = torch.empty((n, d), dtype=torch.bfloat16, device=x.device) if du is None else du
        a.dx_stride = _rowmat("dx", dx, n, d)
        a.du_stride = _rowmat("du", du, n, d)
        dbias = torch.empty(d, dtype=torch.bfloat16, device=x.device) if dbias is None else dbias
        _vec("dbias", dbias, d)
        if compute_dweight:
            dweight = torch.empty(d, dtype=torch.bfloat16, device=x.device) if dweight is None else dweight
            _vec("dweight", dweight, d)
        else:
            dweight = None
        need = ctypes.c_size_t(0)
        _check(library().hstu_lmsd_bwd_workspace_size(ctypes.byref(a), ctypes.byref(need)))
        if workspace is None and need.value > 0:
            workspace = torch.empty(need.value, dtype=torch.uint8, device=x.device)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        _check(library().hstu_lmsd_bwd(ctypes.byref(a), dy.data_ptr(), x.data_ptr(), u.data_ptr(),
                                       weight.data_ptr(), bias.data_ptr(), mean.data_ptr(), rstd.data_ptr(),
                                       dx.data_ptr(), du.data_ptr(), dweight.data_ptr() if dweight is not None else None,
                                       dbias.data_ptr(), ws_ptr, ws_bytes, _stream(s)))
    return dx, du, dweight, dbias


def lmsd_bwd_noalloc(dy: torch.Tensor, x: torch.Tensor, u: torch.Tensor, weight: torch.Tensor,
                     bias: torch.Tensor, mean: torch.Tensor, rstd: torch.Tensor, dx: torch.Tensor,
                     du: torch.Tensor, dweight: Optional[torch.Tensor], dbias: torch.Tensor,
                     dropout_ratio: float = 0.0, apply_u_silu: bool = True, concat_u: bool = True,
                     concat_x: bool = True, eps: float = 1e-6, stream=None) -> None:
    """lmsd_bwd for callers that cannot allocate: every output is caller-owned and the
    column partials live in the library's own per-GPU scratch, so nothing is
    allocated here or in the library.  ``dweight=None`` skips dweight.  Calls that
    overlap on one GPU share that scratch and race."""
    compute_dweight = dweight is not None
    a = _lmsd_args(x, u, eps, dropout_ratio, apply_u_silu, concat_u, concat_x, compute_dweight)
    n, d = a.n, a.d
    segs = 1 + a.concat_u + a.concat_x
    a.dy_stride = _rowmat("dy", dy, n, segs * d)
    _vec("weight", weight, d)
    _vec("bias", bias, d)
    _vec("mean", mean, n, torch.float32)
    _vec("rstd", rstd, n, torch.float32)
    a.dx_stride = _rowmat("dx", dx, n, d)
    a.du_stride = _rowmat("du", du, n, d)
    _vec("dbias", dbias, d)
    if compute_dweight:
        _vec("dweight", dweight, d)
    s = _launch_stream(stream, x.device)
    _check(library().hstu_lmsd_bwd_noalloc(ctypes.byref(a), dy.data_ptr(), x.data_ptr(), u.data_ptr(),
                                           weight.data_ptr(), bias.data_ptr(), mean.data_ptr(), rstd.data_ptr(),
                                           dx.data_ptr(), du.data_ptr(),
                                           dweight.data_ptr() if compute_dweight else None, dbias.data_ptr(),
                                           _stream(s)))


def hstu_bwd_dkdv_ds(dout, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, ds,
                     alpha=1.0, scaling_seqlen=None, causal=True, dk=None, dv=None, stream=None,
                     window_size=None, func=None):
    """(dk, dv), storing dS in ``ds`` (``hstu_bwd_workspace_size`` bytes) for
    ``hstu_bwd_dq_ds``, under any mask."""
    H, D, pq, pk, a = _bwd_common(dout, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                                  max_seqlen_k, alpha, scaling_seqlen, causal, window_size, func)
    s = _launch_stream(stream, q.device)
    with torch.cuda.stream(s):
        dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
        dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
        _thd("dk", dk, int(k.shape[0]), H, D)
        _thd("dv", dv, int(k.shape[0]), H, D)
        a.dk, a.dv = _stride(dk), _stride(dv)
        ws_ptr, ws_bytes = _workspace(ds)
        _check(library().hstu_bwd_dkdv_ds(ctypes.byref(a), dout.data_ptr(), q.data_ptr(), k.data_ptr(),
                                          v.data_ptr(), pq, pk, dk.data_ptr(), dv.data_ptr(), ws_ptr, ws_bytes,
                                          _stream(s)))
    return dk, dv


def hstu_bwd_dq_ds(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, ds, alpha=1.0,
                   scaling_seqlen=None, causal=True, dq=None, stream=None, window_size=None, func=None):
    """dq from the dS that ``hstu_bwd_dkdv_ds`` stored in ``ds`` for the same
    problem (``q`` gives the shape and strides of dq only; it is not read)."""
    H, D, pq, pk = _inputs(q, k, k, cu_seqlens_q, cu_seqlens_k)
    a = _args(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_k, alpha, scaling_seqlen, causal, window_size, func)
    a.q, a.k = _stride(q), _stride(k)
    s = _launch_stream(stream, q.device)
    with torch.cuda.stream(s):
        dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
        _thd("dq", dq, int(q.shape[0]), H, D)
        a.dq = _stride(dq)
        ws_ptr, ws_bytes = _workspace(ds)
        _check(library().hstu_bwd_dq_ds(ctypes.byref(a), k.data_ptr(), pq, pk, ws_ptr, ws_bytes, dq.data_ptr(),
                                        _stream(s)))
    return dq


# ---------------------------------------------------------------------------
# Measurement helper: shader-clock samples (not part of the method)
# ---------------------------------------------------------------------------
def clock_sample(count: int = 64, device=None, stream=None) -> torch.Tensor:
    """Enqueue ``count`` one-wave workgroups that each record (100 MHz real time,
    shader cycles, XCC id, HW_ID); returns the (count, 4) int64 device tensor they
    fill (read it after the stream reaches the call)."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    s = _launch_stream(stream, device)
    with torch.cuda.stream(s):
        out = torch.empty((int(count), 4), dtype=torch.int64, device=device)
        _check(library().hstu_clock_sample(out.data_ptr(), int(count), _stream(s)))
    return out


# ---------------------------------------------------------------------------
# Debug builds: failed bounds tests of the kernels' global indices
# ---------------------------------------------------------------------------
DEBUG_SITES = {0: "sequence bounds", 1: "head", 2: "load/store row", 3: "tile copy rows", 4: "endpoint row",
               5: "stored-dS block", 6: "fused dQ accumulator", 7: "LMSD row"}


def debug_take() -> int:
    """Bits of the bounds-test sites that failed in the debug build since the last
    call (DEBUG_SITES names them), which are then cleared; synchronises the device.
    Raises NotImplementedError on the release build."""
    out = ctypes.c_uint32(0)
    _check(library().hstu_debug_take(ctypes.byref(out)))
    return int(out.value)
