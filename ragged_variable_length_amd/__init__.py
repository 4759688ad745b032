"""Python binding of librva.so (the C ABI in include/rva.h).

Argument marshalling only: tensors are passed as raw device pointers and the
current torch stream as a hipStream_t.  Every step of pack -> attend ->
unpack runs in the HIP kernels of librva.so; there is no fallback, and
importing the binding when the library has not been built raises.

PyTorch supplies device memory and streams; the helpers that allocate
outputs do so with torch before calling the library.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["RVAError", "lib", "pack", "ragged_attend", "unpack", "fused", "threshold_l2_mask",
           "qkv_projection", "out_projection", "index", "LayersPlan", "fused_persistent",
           "fused_persistent_noalloc", "set_query_split",
           "PERSISTENT",
           "Plan", "empty", "dtype_code", "F32", "F16", "BF16", "STAGED", "FUSED", "EMPTY",
           "L2_FUSED", "MAX_TOKENS"]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librva.so")

F32, F16, BF16 = 0, 1, 2
STAGED, FUSED, EMPTY, L2_FUSED, PERSISTENT, FUSED_DIRECT = 0, 1, 2, 3, 4, 5
MAX_TOKENS = 1024
HEAD_DIM = 64

_DTYPES = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}


class RVAError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({_status_string(status)}): {detail}")
        self.status = status


class _PlanDesc(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("B", ctypes.c_int), ("N", ctypes.c_int),
                ("H", ctypes.c_int), ("d", ctypes.c_int), ("dtype", ctypes.c_int),
                ("max_seqlen_hint", ctypes.c_int), ("softmax_scale", ctypes.c_float),
                ("q_pad", ctypes.c_void_p), ("k_pad", ctypes.c_void_p), ("v_pad", ctypes.c_void_p),
                ("mask", ctypes.c_void_p), ("q_packed", ctypes.c_void_p),
                ("k_packed", ctypes.c_void_p), ("v_packed", ctypes.c_void_p),
                ("o_packed", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
                ("max_seqlen", ctypes.c_void_p), ("kept_index", ctypes.c_void_p),
                ("o_pad", ctypes.c_void_p), ("x", ctypes.c_void_p), ("C", ctypes.c_int),
                ("x_dtype", ctypes.c_int), ("keep_quantile", ctypes.c_double),
                ("mask_out", ctypes.c_void_p)]


class _LayersDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("N", ctypes.c_int), ("H", ctypes.c_int), ("d", ctypes.c_int),
                ("dtype", ctypes.c_int), ("layers", ctypes.c_int), ("max_seqlen_hint", ctypes.c_int),
                ("softmax_scale", ctypes.c_float), ("x_pad", ctypes.c_void_p),
                ("mask", ctypes.c_void_p), ("w_qkv", ctypes.POINTER(ctypes.c_void_p)),
                ("b_qkv", ctypes.POINTER(ctypes.c_void_p)), ("w_o", ctypes.POINTER(ctypes.c_void_p)),
                ("b_o", ctypes.POINTER(ctypes.c_void_p)), ("resid", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
                ("max_seqlen", ctypes.c_void_p), ("kept_index", ctypes.c_void_p),
                ("y_pad", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load librva.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -c "
                          "'import __graft_entry__; __graft_entry__.build()')")
    L = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.rva_pack.argtypes = [P, P, P, P, I, I, I, I, I, P, P, P, P, P, P, P]
    L.rva_ragged_attend.argtypes = [P, P, P, P, I, I, I, I, F, I, P, P]
    L.rva_unpack.argtypes = [P, P, P, I, I, I, I, I, P, P]
    L.rva_fused.argtypes = [P, P, P, P, I, I, I, I, I, F, I, P, P, P, P]
    L.rva_fused_persistent.argtypes = [P, P, P, P, I, I, I, I, I, F, I, P, P, P, P, P]
    L.rva_fused_persistent_noalloc.argtypes = [P, P, P, P, I, I, I, I, I, F, I, P, P, P, P]
    L.rva_plan_create.argtypes = [ctypes.POINTER(_PlanDesc), ctypes.POINTER(ctypes.c_void_p)]
    L.rva_plan_launch.argtypes = [P, P]
    L.rva_layers_plan_create.argtypes = [ctypes.POINTER(_LayersDesc), ctypes.POINTER(ctypes.c_void_p)]
    L.rva_plan_destroy.argtypes = [P]
    L.rva_empty.argtypes = [I, P]
    L.rva_set_query_split.argtypes = [I]
    LL = ctypes.c_longlong
    L.rva_probe_copy.argtypes = [P, P, LL, I, P]
    L.rva_probe_read.argtypes = [P, P, LL, I, P]
    L.rva_probe_mfma.argtypes = [I, P, I, P, ctypes.POINTER(LL)]
    L.rva_probe_gather.argtypes = [P, P, P, P, P, P, P, I, I, I, P]
    L.rva_threshold_l2_mask.argtypes = [P, I, I, I, I, ctypes.c_double, P, P]
    L.rva_qkv_projection.argtypes = [P, P, P, I, I, I, P, P, I, P, P, P, P]
    L.rva_out_projection.argtypes = [P, P, P, P, I, I, I, P, P, P, I, P, P]
    L.rva_status_string.argtypes = [I]
    L.rva_status_string.restype = ctypes.c_char_p
    L.rva_last_error.argtypes = []
    L.rva_last_error.restype = ctypes.c_char_p
    L.rva_version.argtypes = []
    for name in ("rva_pack", "rva_ragged_attend", "rva_unpack", "rva_fused", "rva_plan_create",
                 "rva_plan_launch", "rva_plan_destroy", "rva_empty", "rva_version",
                 "rva_threshold_l2_mask", "rva_qkv_projection", "rva_out_projection",
                 "rva_layers_plan_create", "rva_fused_persistent",
                 "rva_fused_persistent_noalloc", "rva_set_query_split", "rva_probe_copy",
                 "rva_probe_read", "rva_probe_mfma", "rva_probe_gather"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _status_string(s: int) -> str:
    try:
        return lib().rva_status_string(s).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "?"


def _check(status: int, where: str):
    if status != 0:
        raise RVAError(status, where, lib().rva_last_error().decode())


def _ptr(t):
    # a plain int: ctypes passes it as void* (None as NULL)
    return None if t is None else t.data_ptr()


# The current stream's raw handle without building a Stream object (which
# costs about 3 us a call); the library launches on the current device.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream=None):
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None and _cur_device is not None:
        return _raw_stream(_cur_device())
    return torch.cuda.current_stream().cuda_stream


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def _dev(t, name: str, *, dtype=None, shape=None, numel=None):
    """Check one tensor argument before its pointer reaches the library: a
    torch tensor on the current device, contiguous, of the given dtype and
    shape (or with at least `numel` elements).  Raises before anything is
    enqueued; returns the tensor."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor (got {type(t).__name__})")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got one on {t.device})")
    if _cur_device is not None and t.device.index != _cur_device():
        raise ValueError(f"{name} is on {t.device}, not on the current device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} must hold at least {numel} elements (got {t.numel()})")
    return t


def _opt(t, name: str, **kw):
    return None if t is None else _dev(t, name, **kw)


def _mask_u8(mask, B=None, N=None):
    """The keep-mask as uint8 [B, N] (bool is viewed as uint8), checked."""
    if not isinstance(mask, torch.Tensor):
        raise TypeError("mask must be a torch tensor")
    if mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    elif mask.dtype != torch.uint8:
        raise TypeError("mask must be uint8 or bool")
    if mask.dim() != 2:
        raise ValueError(f"mask must be [B, N] (got {tuple(mask.shape)})")
    _dev(mask, "mask", shape=(mask.shape[0] if B is None else B, mask.shape[1] if N is None else N))
    return mask


def _like(t, dev: int, dtype, shape) -> bool:
    """Fast form of the checks: `t` is a contiguous tensor on device `dev`
    with this dtype and shape (False for anything else, non-tensors
    included).  Callers re-run _dev on failure to word the error."""
    try:
        return (t.get_device() == dev and t.dtype == dtype and t.shape == shape
                and t.is_contiguous())
    except AttributeError:
        return False


def _qkv(q, k, v):
    """Padded q/k/v: [B, N, H, 64] of one supported dtype, identical shapes.
    Returns (shape, device index)."""
    _dev(q, "q")
    sh = q.shape
    if len(sh) != 4 or sh[3] != HEAD_DIM:
        raise ValueError(f"q must be [B, N, H, {HEAD_DIM}] (got {tuple(sh)})")
    dtype_code(q)
    dev = q.get_device()
    for name, t in (("k", k), ("v", v)):
        if not _like(t, dev, q.dtype, sh):
            _dev(t, name, dtype=q.dtype, shape=sh)
            raise ValueError(f"{name} must be on the device of q")
    return sh, dev


_I32 = torch.int32


def _offsets(cu_seqlens, max_seqlen, B, dev=None):
    if cu_seqlens is not None and not (dev is not None and _like(cu_seqlens, dev, _I32, (B + 1,))):
        _dev(cu_seqlens, "cu_seqlens", dtype=_I32, shape=(B + 1,))
    if max_seqlen is not None and not (dev is not None and max_seqlen.get_device() == dev and
                                       max_seqlen.dtype == _I32 and max_seqlen.numel() >= 1 and
                                       max_seqlen.is_contiguous()):
        _dev(max_seqlen, "max_seqlen", dtype=_I32, numel=1)


def pack(q, k, v, mask, *, outputs=None, kept_index=True, stream=None):
    """Kept counts, cu_seqlens, max_seqlen and packed q/k/v (capacity B*N rows).

    q/k/v: [B,N,H,64] device tensors (any may be None, the given ones of one
    shape and dtype); mask: [B,N] uint8/bool.  Returns dict with q, k, v
    (packed, [B*N,H,64] capacity), cu_seqlens, max_seqlen ([1] int32) and
    kept_index ([B*N] capacity int32 or None).  Caller-given outputs must
    have those capacities.
    """
    given = [(nm, t) for nm, t in (("q", q), ("k", k), ("v", v)) if t is not None]
    if not given:
        raise ValueError("at least one of q, k, v is needed")
    ref = _dev(given[0][1], given[0][0])
    if ref.dim() != 4 or ref.shape[3] != HEAD_DIM:
        raise ValueError(f"{given[0][0]} must be [B, N, H, {HEAD_DIM}] (got {tuple(ref.shape)})")
    dtype_code(ref)
    for nm, t in given[1:]:
        _dev(t, nm, dtype=ref.dtype, shape=ref.shape)
    B, N, H, d = ref.shape
    m = _mask_u8(mask, B, N)
    out = dict(outputs or {})
    dev = ref.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is not None:
            if out.get(name) is None:
                out[name] = torch.empty((B * N, H, d), dtype=t.dtype, device=dev)
            _dev(out[name], f"outputs[{name!r}]", dtype=t.dtype, numel=B * N * H * d)
        else:
            out[name] = None
    if out.get("cu_seqlens") is None:
        out["cu_seqlens"] = torch.empty(B + 1, dtype=torch.int32, device=dev)
    if out.get("max_seqlen") is None:
        out["max_seqlen"] = torch.empty(1, dtype=torch.int32, device=dev)
    if kept_index and out.get("kept_index") is None:
        out["kept_index"] = torch.empty(B * N, dtype=torch.int32, device=dev)
    out.setdefault("kept_index", None)
    _offsets(out["cu_seqlens"], out["max_seqlen"], B)
    _opt(out["kept_index"], "kept_index", dtype=torch.int32, numel=B * N)
    _check(lib().rva_pack(_ptr(q), _ptr(k), _ptr(v), _ptr(m), B, N, H, d, dtype_code(ref),
                          _ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]), _ptr(out["cu_seqlens"]),
                          _ptr(out["max_seqlen"]), _ptr(out["kept_index"]), _stream(stream)),
           "rva_pack")
    return out


def index(mask, *, out=None, stream=None):
    """Offsets and kept-index list only (rva_pack with no row copies):
    returns dict with cu_seqlens [B+1], max_seqlen [1], kept_index [B*N]
    (capacity; entries past T unused)."""
    m = _mask_u8(mask)
    B, N = m.shape
    out = dict(out or {})
    dev = m.device
    if out.get("cu_seqlens") is None:
        out["cu_seqlens"] = torch.empty(B + 1, dtype=torch.int32, device=dev)
    if out.get("max_seqlen") is None:
        out["max_seqlen"] = torch.empty(1, dtype=torch.int32, device=dev)
    if out.get("kept_index") is None:
        out["kept_index"] = torch.empty(B * N, dtype=torch.int32, device=dev)
    _offsets(out["cu_seqlens"], out["max_seqlen"], B)
    _dev(out["kept_index"], "kept_index", dtype=torch.int32, numel=B * N)
    _check(lib().rva_pack(None, None, None, _ptr(m), B, N, 1, HEAD_DIM, F16, None, None, None,
                          _ptr(out["cu_seqlens"]), _ptr(out["max_seqlen"]),
                          _ptr(out["kept_index"]), _stream(stream)), "rva_pack")
    return out


def _packed(t, name, ref=None):
    """Packed rows [rows, H, 64] (matching `ref` in shape and dtype)."""
    if ref is not None:
        return _dev(t, name, dtype=ref.dtype, shape=ref.shape)
    _dev(t, name)
    if t.dim() != 3 or t.shape[2] != HEAD_DIM:
        raise ValueError(f"{name} must be [rows, H, {HEAD_DIM}] (got {tuple(t.shape)})")
    dtype_code(t)
    return t


def ragged_attend(q, k, v, cu_seqlens, max_seqlen: int, *, scale: float | None = None, out=None,
                  stream=None):
    """Attention over packed [T,H,64] q/k/v with offsets cu_seqlens [B+1].

    cu_seqlens is int32 on the device; its last entry (T) must not exceed the
    rows of q/k/v/out (the values are device data and are not read here)."""
    _packed(q, "q")
    _packed(k, "k", q)
    _packed(v, "v", q)
    _dev(cu_seqlens, "cu_seqlens", dtype=torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be int32 [B+1] with B >= 1")
    H, d = q.shape[1], q.shape[2]
    B = cu_seqlens.shape[0] - 1
    if out is None:
        out = torch.empty_like(q)
    _packed(out, "out", q)
    _check(lib().rva_ragged_attend(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), B, H, d,
                                   int(max_seqlen), float(scale or 0.0), dtype_code(q), _ptr(out),
                                   _stream(stream)), "rva_ragged_attend")
    return out


def unpack(o_packed, cu_seqlens, mask, *, out=None, stream=None):
    """Packed [T,H,64] rows -> padded [B,N,H,64]; pruned rows are +0."""
    m = _mask_u8(mask)
    B, N = m.shape
    _packed(o_packed, "o_packed")
    _dev(cu_seqlens, "cu_seqlens", dtype=torch.int32, shape=(B + 1,))
    H, d = o_packed.shape[1], o_packed.shape[2]
    if out is None:
        out = torch.empty((B, N, H, d), dtype=o_packed.dtype, device=o_packed.device)
    _dev(out, "out", dtype=o_packed.dtype, shape=(B, N, H, d))
    _check(lib().rva_unpack(_ptr(o_packed), _ptr(cu_seqlens), _ptr(m), B, N, H, d,
                            dtype_code(o_packed), _ptr(out), _stream(stream)), "rva_unpack")
    return out


_U8 = torch.uint8
_MIN_DEV = 0  # device indices of GPU tensors (CPU tensors report -1)


def _fused_fast(q, k, v, mask, out, cu, mx) -> bool:
    """The checks of _fused_args as one expression (no calls, for the
    per-call path): every tensor on q's device, which is the current one,
    contiguous, of the expected dtype and shape.  False sends the caller
    through the detailed checks, which word the error."""
    try:
        sh = q.shape
        dt = q.dtype
        dev = q.get_device()
        return (dev >= _MIN_DEV and len(sh) == 4 and sh[3] == HEAD_DIM and dt in _DTYPES
                and q.is_contiguous()
                and k.get_device() == dev and k.dtype == dt and k.shape == sh and k.is_contiguous()
                and v.get_device() == dev and v.dtype == dt and v.shape == sh and v.is_contiguous()
                and mask.get_device() == dev and mask.dtype == _U8 and mask.shape == sh[:2]
                and mask.is_contiguous()
                and (out is None or (out.get_device() == dev and out.dtype == dt
                                     and out.shape == sh and out.is_contiguous()))
                and (cu is None or (cu.get_device() == dev and cu.dtype == _I32
                                    and cu.shape == (sh[0] + 1,) and cu.is_contiguous()))
                and (mx is None or (mx.get_device() == dev and mx.dtype == _I32
                                    and mx.numel() >= 1 and mx.is_contiguous()))
                and (_cur_device is None or dev == _cur_device()))
    except AttributeError:
        return False


def _fused_args(q, k, v, mask, out, cu_seqlens, max_seqlen):
    if _fused_fast(q, k, v, mask, out, cu_seqlens, max_seqlen):
        return mask, (torch.empty_like(q) if out is None else out), tuple(q.shape)
    sh, dev = _qkv(q, k, v)
    B, N, H, d = sh
    if _like(mask, dev, _U8, (B, N)):
        m = mask
    else:
        m = _mask_u8(mask, B, N)
        if m.get_device() != dev:
            raise ValueError("mask must be on the device of q")
    if out is None:
        out = torch.empty_like(q)
    elif not _like(out, dev, q.dtype, sh):
        _dev(out, "out", dtype=q.dtype, shape=sh)
        raise ValueError("out must be on the device of q")
    _offsets(cu_seqlens, max_seqlen, B, dev)
    return m, out, (B, N, H, d)


def fused(q, k, v, mask, *, max_seqlen_hint: int = 0, scale: float | None = None, out=None,
          cu_seqlens=None, max_seqlen=None, stream=None):
    """Whole path in one launch: padded [B,N,H,64] in, padded out."""
    m, out, (B, N, H, d) = _fused_args(q, k, v, mask, out, cu_seqlens, max_seqlen)
    _check(lib().rva_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(m), B, N, H, d, int(max_seqlen_hint),
                           float(scale or 0.0), dtype_code(q), _ptr(out), _ptr(cu_seqlens),
                           _ptr(max_seqlen), _stream(stream)), "rva_fused")
    return out


def fused_persistent(q, k, v, mask, work, *, max_seqlen_hint: int = 0, scale: float | None = None,
                     out=None, cu_seqlens=None, max_seqlen=None, stream=None):
    """fused() as a persistent grid.  work: int32 [2] device tensor, zero
    before the first call (every call leaves it zero again).  Only one call
    may be in flight on one work buffer: calls on different streams that may
    overlap need distinct buffers."""
    m, out, (B, N, H, d) = _fused_args(q, k, v, mask, out, cu_seqlens, max_seqlen)
    _dev(work, "work", dtype=torch.int32, numel=2)
    _check(lib().rva_fused_persistent(_ptr(q), _ptr(k), _ptr(v), _ptr(m), B, N, H, d,
                                      int(max_seqlen_hint), float(scale or 0.0), dtype_code(q),
                                      _ptr(out), _ptr(cu_seqlens), _ptr(max_seqlen), _ptr(work),
                                      _stream(stream)), "rva_fused_persistent")
    return out


def fused_persistent_noalloc(q, k, v, mask, *, max_seqlen_hint: int = 0,
                             scale: float | None = None, out=None, cu_seqlens=None,
                             max_seqlen=None, stream=None):
    """fused_persistent() with the library's own static work counter (no
    work buffer, nothing allocated by the library).  All calls on one GPU
    share that counter: calls must not overlap (order them on one stream)."""
    m, out, (B, N, H, d) = _fused_args(q, k, v, mask, out, cu_seqlens, max_seqlen)
    _check(lib().rva_fused_persistent_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(m), B, N, H, d,
                                              int(max_seqlen_hint), float(scale or 0.0),
                                              dtype_code(q), _ptr(out), _ptr(cu_seqlens),
                                              _ptr(max_seqlen), _stream(stream)),
           "rva_fused_persistent_noalloc")
    return out


def threshold_l2_mask(x, keep_quantile: float, *, out=None, stream=None):
    """Threshold-l2 keep-mask of embeddings x [B,N,C]: uint8 [B,N], CLS kept,
    patch kept when its L2 norm reaches the per-image keep_quantile of the
    patch norms."""
    _dev(x, "x")
    if x.dim() != 3:
        raise ValueError(f"x must be [B, N, C] (got {tuple(x.shape)})")
    dtype_code(x)
    B, N, C = x.shape
    if out is None:
        out = torch.empty((B, N), dtype=torch.uint8, device=x.device)
    _dev(out, "out", dtype=torch.uint8, shape=(B, N))
    _check(lib().rva_threshold_l2_mask(_ptr(x), B, N, C, dtype_code(x), float(keep_quantile),
                                       _ptr(out), _stream(stream)), "rva_threshold_l2_mask")
    return out


def _weight(w, b, rows, C, dtype, wname, bname):
    _dev(w, wname, dtype=dtype, shape=(rows, C))
    _opt(b, bname, dtype=dtype, shape=(rows,))


def qkv_projection(x, cu_seqlens, w_qkv, b_qkv=None, *, kept_index=None, B=None, N=None,
                   out=None, stream=None):
    """[q | k | v] = x_r W_qkv^T + b_qkv on the packed rows r.

    x: padded [B,N,C] with kept_index (rows gathered), or packed [>=T, C]
    without (then B and N give the capacity B*N).  Returns packed q, k, v of
    capacity B*N rows, [B*N, C] each (rows past T = cu_seqlens[B] untouched).
    """
    _dev(x, "x")
    dtype_code(x)
    C = x.shape[-1]
    if kept_index is not None:
        if x.dim() != 3:
            raise ValueError(f"x must be padded [B, N, C] with kept_index (got {tuple(x.shape)})")
        B, N = x.shape[0], x.shape[1]
        _dev(kept_index, "kept_index", dtype=torch.int32, numel=B * N)
    if B is None or N is None:
        raise ValueError("packed input needs B and N")
    if kept_index is None:
        _dev(x, "x", numel=B * N * C)
    _dev(cu_seqlens, "cu_seqlens", dtype=torch.int32, shape=(B + 1,))
    _weight(w_qkv, b_qkv, 3 * C, C, x.dtype, "w_qkv", "b_qkv")
    if out is None:
        out = tuple(torch.empty((B * N, C), dtype=x.dtype, device=x.device) for _ in range(3))
    q, k, v = out
    for nm, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, f"out {nm}", dtype=x.dtype, numel=B * N * C)
    _check(lib().rva_qkv_projection(_ptr(x), _ptr(kept_index), _ptr(cu_seqlens), B, N, C,
                                    _ptr(w_qkv), _ptr(b_qkv), dtype_code(x), _ptr(q), _ptr(k),
                                    _ptr(v), _stream(stream)), "rva_qkv_projection")
    return q, k, v


def out_projection(o, cu_seqlens, w_o, b_o=None, *, kept_index=None, mask=None, B=None, N=None,
                   residual=None, out=None, stream=None):
    """y_r = o_r W_o^T + b_o (+ residual) on the packed rows r of o [>=T, C].

    With kept_index and mask: y is padded [B,N,C], pruned rows +0, residual
    padded.  Without: y packed [B*N, C] (capacity), residual packed.
    """
    _dev(o, "o")
    dtype_code(o)
    C = o.shape[-1]
    m = None
    if kept_index is not None:
        if mask is None:
            raise ValueError("mask is needed with kept_index")
        m = _mask_u8(mask)
        B, N = m.shape
        _dev(kept_index, "kept_index", dtype=torch.int32, numel=B * N)
    if B is None or N is None:
        raise ValueError("B and N are needed")
    _dev(o, "o", numel=B * N * C)
    _dev(cu_seqlens, "cu_seqlens", dtype=torch.int32, shape=(B + 1,))
    _weight(w_o, b_o, C, C, o.dtype, "w_o", "b_o")
    shape = (B, N, C) if kept_index is not None else None
    if out is None:
        out = torch.empty(shape or (B * N, C), dtype=o.dtype, device=o.device)
    if shape:
        _dev(out, "out", dtype=o.dtype, shape=shape)
        _opt(residual, "residual", dtype=o.dtype, shape=shape)
    else:
        _dev(out, "out", dtype=o.dtype, numel=B * N * C)
        _opt(residual, "residual", dtype=o.dtype, numel=B * N * C)
    _check(lib().rva_out_projection(_ptr(o), _ptr(kept_index), _ptr(cu_seqlens), _ptr(m), B, N, C,
                                    _ptr(w_o), _ptr(b_o), _ptr(residual), dtype_code(o), _ptr(out),
                                    _stream(stream)), "rva_out_projection")
    return out


def set_query_split(split: int):
    """Query tiles per (sequence, head) on every later attention launch of
    this process (0: each launch chooses; results never depend on it)."""
    _check(lib().rva_set_query_split(int(split)), "rva_set_query_split")


def probe_copy(src, dst, grid: int, stream=None):
    """Ceiling probe: copy src into dst (same byte size, a multiple of 16)."""
    _dev(src, "src")
    _dev(dst, "dst", numel=0)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    _check(lib().rva_probe_copy(_ptr(src), _ptr(dst), nbytes, int(grid), _stream(stream)),
           "rva_probe_copy")


def probe_read(src, sink, grid: int, stream=None):
    """Ceiling probe: read every byte of src; sink: int32 [grid * 256]."""
    _dev(src, "src")
    _dev(sink, "sink", dtype=torch.int32, numel=int(grid) * 256)
    _check(lib().rva_probe_read(_ptr(src), _ptr(sink), src.numel() * src.element_size(), int(grid),
                                _stream(stream)), "rva_probe_read")


def probe_mfma(iters: int, out, grid: int, stream=None) -> int:
    """Ceiling probe: fp16 matrix-core products; out: float32 [grid * 256].
    Returns the FLOPs of the launch."""
    _dev(out, "out", dtype=torch.float32, numel=int(grid) * 256)
    fl = ctypes.c_longlong(0)
    _check(lib().rva_probe_mfma(int(iters), _ptr(out), int(grid), _stream(stream),
                                ctypes.byref(fl)), "rva_probe_mfma")
    return fl.value


def probe_gather(q, k, v, mask, cu_seqlens, kept_index, out, stream=None):
    """Ceiling probe: rva_fused's reads and writes without its arithmetic.
    q, k, v, out: padded 16-bit [B, N, H, 64]; mask uint8 [B, N];
    cu_seqlens and kept_index as pack/index return them for that mask."""
    (B, N, H, _), _ = _qkv(q, k, v)
    if q.dtype == torch.float32:
        raise ValueError("the gather probe takes 16-bit tensors")
    m = _mask_u8(mask, B, N)
    _dev(cu_seqlens, "cu_seqlens", dtype=torch.int32, shape=(B + 1,))
    _dev(kept_index, "kept_index", dtype=torch.int32, numel=B * N)
    _dev(out, "out", dtype=q.dtype, shape=tuple(q.shape))
    _check(lib().rva_probe_gather(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(m), _ptr(cu_seqlens),
                                  _ptr(kept_index), B, N, H, _stream(stream)), "rva_probe_gather")


def empty(count: int = 1, stream=None):
    """Enqueue `count` empty one-workgroup kernels (dispatch-floor probe)."""
    _check(lib().rva_empty(int(count), _stream(stream)), "rva_empty")


class Plan:
    """A captured launch sequence (HIP graph) replayed with one launch, or
    (mode FUSED_DIRECT) the fused launch validated once and enqueued directly
    by every launch().

    Tensors given here are checked as the direct calls check them and kept
    alive by the plan; their contents may change between launches, their
    addresses may not.  A PERSISTENT plan owns one work counter: one launch
    of it may be in flight at a time.
    """

    def __init__(self, mode: int, *, q=None, k=None, v=None, mask=None, out=None, scale=None,
                 max_seqlen_hint: int = 0, packed=None, cu_seqlens=None, max_seqlen=None,
                 kept_index=None, x=None, keep_quantile: float = 0.5):
        """mode L2_FUSED: the keep-mask of `x` is written into `mask` by the
        plan, then read by the fused attention."""
        self._keep = [q, k, v, mask, out, packed, cu_seqlens, max_seqlen, kept_index, x]
        desc = _PlanDesc()
        desc.mode = mode
        desc.d = HEAD_DIM
        if mode != EMPTY:
            m, out, (B, N, H, d) = _fused_args(q, k, v, mask, out, cu_seqlens, max_seqlen)
            self._keep.append(out)
            desc.B, desc.N, desc.H, desc.d = B, N, H, d
            desc.dtype = dtype_code(q)
            desc.max_seqlen_hint = int(max_seqlen_hint)
            desc.softmax_scale = float(scale or 0.0)
            desc.q_pad, desc.k_pad, desc.v_pad = q.data_ptr(), k.data_ptr(), v.data_ptr()
            desc.mask = m.data_ptr()
            desc.o_pad = out.data_ptr()
            if mode == STAGED:
                if packed is None or cu_seqlens is None:
                    raise ValueError("a staged plan needs packed buffers and cu_seqlens")
                for nm in ("q", "k", "v", "o"):
                    _dev(packed[nm], f"packed[{nm!r}]", dtype=q.dtype, numel=B * N * H * d)
            if packed is not None:
                desc.q_packed = packed["q"].data_ptr()
                desc.k_packed = packed["k"].data_ptr()
                desc.v_packed = packed["v"].data_ptr()
                desc.o_packed = packed["o"].data_ptr()
            _opt(kept_index, "kept_index", dtype=torch.int32, numel=B * N)
            desc.cu_seqlens = cu_seqlens.data_ptr() if cu_seqlens is not None else None
            desc.max_seqlen = max_seqlen.data_ptr() if max_seqlen is not None else None
            desc.kept_index = kept_index.data_ptr() if kept_index is not None else None
            if mode == L2_FUSED:
                _dev(x, "x")
                if x.dim() != 3 or tuple(x.shape[:2]) != (B, N):
                    raise ValueError(f"x must be [{B}, {N}, C] (got {tuple(x.shape)})")
                desc.x = x.data_ptr()
                desc.C = x.shape[2]
                desc.x_dtype = dtype_code(x)
                desc.keep_quantile = float(keep_quantile)
                desc.mask_out = desc.mask
                desc.mask = None
        h = ctypes.c_void_p()
        _check(lib().rva_plan_create(ctypes.byref(desc), ctypes.byref(h)), "rva_plan_create")
        self._h = h

    def launch(self, stream=None):
        _check(lib().rva_plan_launch(self._h, _stream(stream)), "rva_plan_launch")

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().rva_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class LayersPlan(Plan):
    """One pack, `len(weights)` attention sub-layers (QKV projection, ragged
    attention, output projection added to the packed residual stream) and one
    unpack, captured as a single graph.

    x: padded [B,N,C]; mask: [B,N]; weights: list of dicts with w_qkv, b_qkv,
    w_o, b_o device tensors (biases may be None).  Scratch is allocated here
    (torch); out (padded [B,N,C]) receives the final residual stream.
    """

    def __init__(self, x, mask, weights, *, out=None, scale=None, max_seqlen_hint: int = 0):
        _dev(x, "x")
        if x.dim() != 3 or x.shape[2] % HEAD_DIM:
            raise ValueError(f"x must be [B, N, C] with C a multiple of {HEAD_DIM}")
        dtype_code(x)
        B, N, C = x.shape
        H = C // HEAD_DIM
        L = len(weights)
        m = _mask_u8(mask, B, N)
        for l, wd in enumerate(weights):
            _weight(wd["w_qkv"], wd.get("b_qkv"), 3 * C, C, x.dtype, f"w_qkv[{l}]", f"b_qkv[{l}]")
            _weight(wd["w_o"], wd.get("b_o"), C, C, x.dtype, f"w_o[{l}]", f"b_o[{l}]")
        dev = x.device
        self.scratch = {nm: torch.empty((B * N, C), dtype=x.dtype, device=dev)
                        for nm in ("resid", "q", "k", "v", "o")}
        self.cu_seqlens = torch.empty(B + 1, dtype=torch.int32, device=dev)
        self.max_seqlen = torch.empty(1, dtype=torch.int32, device=dev)
        self.kept_index = torch.empty(B * N, dtype=torch.int32, device=dev)
        self.out = out if out is not None else torch.empty_like(x)
        _dev(self.out, "out", dtype=x.dtype, shape=x.shape)
        self._keep = [x, m, weights, self.scratch, self.out]
        arr = lambda key: (ctypes.c_void_p * L)(*[
            (wd[key].data_ptr() if wd.get(key) is not None else None) for wd in weights])
        self._arrays = {k: arr(k) for k in ("w_qkv", "b_qkv", "w_o", "b_o")}
        desc = _LayersDesc()
        desc.B, desc.N, desc.H, desc.d, desc.dtype, desc.layers = B, N, H, HEAD_DIM, dtype_code(x), L
        desc.max_seqlen_hint = int(max_seqlen_hint)
        desc.softmax_scale = float(scale or 0.0)
        desc.x_pad, desc.mask = x.data_ptr(), m.data_ptr()
        for k, a in self._arrays.items():
            setattr(desc, k, ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p)))
        for nm, t in self.scratch.items():
            setattr(desc, nm, t.data_ptr())
        desc.cu_seqlens = self.cu_seqlens.data_ptr()
        desc.max_seqlen = self.max_seqlen.data_ptr()
        desc.kept_index = self.kept_index.data_ptr()
        desc.y_pad = self.out.data_ptr()
        h = ctypes.c_void_p()
        _check(lib().rva_layers_plan_create(ctypes.byref(desc), ctypes.byref(h)),
               "rva_layers_plan_create")
        self._h = h
