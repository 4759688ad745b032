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
    L.rva_plan_create.argtypes = [ctypes.POINTER(_PlanDesc), ctypes.POINTER(ctypes.c_void_p)]
    L.rva_plan_launch.argtypes = [P, P]
    L.rva_layers_plan_create.argtypes = [ctypes.POINTER(_LayersDesc), ctypes.POINTER(ctypes.c_void_p)]
    L.rva_plan_destroy.argtypes = [P]
    L.rva_empty.argtypes = [I, P]
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
                 "rva_layers_plan_create", "rva_fused_persistent"):
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


def _mask_u8(mask: torch.Tensor) -> torch.Tensor:
    if mask.dtype == torch.bool:
        return mask.view(torch.uint8)
    if mask.dtype != torch.uint8:
        raise TypeError("mask must be uint8 or bool")
    return mask


def _req(t: torch.Tensor, name: str):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def pack(q, k, v, mask, *, outputs=None, kept_index=True, stream=None):
    """Kept counts, cu_seqlens, max_seqlen and packed q/k/v (capacity B*N rows).

    q/k/v: [B,N,H,64] device tensors (any may be None); mask: [B,N] uint8/bool.
    Returns dict with q, k, v (packed, [B*N,H,64] capacity), cu_seqlens,
    max_seqlen ([1] int32) and kept_index ([B*N] capacity int32 or None).
    """
    ref = next(t for t in (q, k, v) if t is not None) if any(t is not None for t in (q, k, v)) else None
    if ref is None:
        raise ValueError("at least one of q, k, v is needed")
    B, N, H, d = ref.shape
    m = _mask_u8(mask)
    out = dict(outputs or {})
    dev = ref.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is not None:
            _req(t, name)
            if name not in out:
                out[name] = torch.empty((B * N, H, d), dtype=t.dtype, device=dev)
        else:
            out[name] = None
    if "cu_seqlens" not in out:
        out["cu_seqlens"] = torch.empty(B + 1, dtype=torch.int32, device=dev)
    if "max_seqlen" not in out:
        out["max_seqlen"] = torch.empty(1, dtype=torch.int32, device=dev)
    if kept_index and "kept_index" not in out:
        out["kept_index"] = torch.empty(B * N, dtype=torch.int32, device=dev)
    out.setdefault("kept_index", None)
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
    out.setdefault("cu_seqlens", torch.empty(B + 1, dtype=torch.int32, device=dev))
    out.setdefault("max_seqlen", torch.empty(1, dtype=torch.int32, device=dev))
    out.setdefault("kept_index", torch.empty(B * N, dtype=torch.int32, device=dev))
    _check(lib().rva_pack(None, None, None, _ptr(m), B, N, 1, HEAD_DIM, F16, None, None, None,
                          _ptr(out["cu_seqlens"]), _ptr(out["max_seqlen"]),
                          _ptr(out["kept_index"]), _stream(stream)), "rva_pack")
    return out


def ragged_attend(q, k, v, cu_seqlens, max_seqlen: int, *, scale: float | None = None, out=None,
                  stream=None):
    """Attention over packed [T,H,64] q/k/v with offsets cu_seqlens [B+1]."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _req(t, name)
    H, d = q.shape[1], q.shape[2]
    B = cu_seqlens.shape[0] - 1
    if out is None:
        out = torch.empty_like(q)
    _check(lib().rva_ragged_attend(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), B, H, d,
                                   int(max_seqlen), float(scale or 0.0), dtype_code(q), _ptr(out),
                                   _stream(stream)), "rva_ragged_attend")
    return out


def unpack(o_packed, cu_seqlens, mask, *, out=None, stream=None):
    """Packed [T,H,64] rows -> padded [B,N,H,64]; pruned rows are +0."""
    m = _mask_u8(mask)
    B, N = m.shape
    H, d = o_packed.shape[1], o_packed.shape[2]
    if out is None:
        out = torch.empty((B, N, H, d), dtype=o_packed.dtype, device=o_packed.device)
    _check(lib().rva_unpack(_ptr(o_packed), _ptr(cu_seqlens), _ptr(m), B, N, H, d,
                            dtype_code(o_packed), _ptr(out), _stream(stream)), "rva_unpack")
    return out


def fused(q, k, v, mask, *, max_seqlen_hint: int = 0, scale: float | None = None, out=None,
          cu_seqlens=None, max_seqlen=None, stream=None):
    """Whole path in one launch: padded [B,N,H,64] in, padded out."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _req(t, name)
    m = _mask_u8(mask)
    B, N, H, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    _check(lib().rva_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(m), B, N, H, d, int(max_seqlen_hint),
                           float(scale or 0.0), dtype_code(q), _ptr(out), _ptr(cu_seqlens),
                           _ptr(max_seqlen), _stream(stream)), "rva_fused")
    return out


def fused_persistent(q, k, v, mask, work, *, max_seqlen_hint: int = 0, scale: float | None = None,
                     out=None, cu_seqlens=None, max_seqlen=None, stream=None):
    """fused() as a persistent grid.  work: int32 [2] device tensor, zero
    before the first call (every call leaves it zero again)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _req(t, name)
    m = _mask_u8(mask)
    B, N, H, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    _check(lib().rva_fused_persistent(_ptr(q), _ptr(k), _ptr(v), _ptr(m), B, N, H, d,
                                      int(max_seqlen_hint), float(scale or 0.0), dtype_code(q),
                                      _ptr(out), _ptr(cu_seqlens), _ptr(max_seqlen), _ptr(work),
                                      _stream(stream)), "rva_fused_persistent")
    return out


def threshold_l2_mask(x, keep_quantile: float, *, out=None, stream=None):
    """Threshold-l2 keep-mask of embeddings x [B,N,C]: uint8 [B,N], CLS kept,
    patch kept when its L2 norm reaches the per-image keep_quantile of the
    patch norms."""
    _req(x, "x")
    B, N, C = x.shape
    if out is None:
        out = torch.empty((B, N), dtype=torch.uint8, device=x.device)
    _check(lib().rva_threshold_l2_mask(_ptr(x), B, N, C, dtype_code(x), float(keep_quantile),
                                       _ptr(out), _stream(stream)), "rva_threshold_l2_mask")
    return out


def qkv_projection(x, cu_seqlens, w_qkv, b_qkv=None, *, kept_index=None, B=None, N=None,
                   out=None, stream=None):
    """[q | k | v] = x_r W_qkv^T + b_qkv on the packed rows r.

    x: padded [B,N,C] with kept_index (rows gathered), or packed [>=T, C]
    without (then B and N give the capacity B*N).  Returns packed q, k, v of
    capacity B*N rows, [B*N, C] each (rows past T = cu_seqlens[B] untouched).
    """
    _req(x, "x")
    C = x.shape[-1]
    if kept_index is not None:
        B, N = x.shape[0], x.shape[1]
    if B is None or N is None:
        raise ValueError("packed input needs B and N")
    if out is None:
        out = tuple(torch.empty((B * N, C), dtype=x.dtype, device=x.device) for _ in range(3))
    q, k, v = out
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
    _req(o, "o")
    C = o.shape[-1]
    m = None
    if kept_index is not None:
        m = _mask_u8(mask)
        B, N = m.shape
    if B is None or N is None:
        raise ValueError("B and N are needed")
    if out is None:
        shape = (B, N, C) if kept_index is not None else (B * N, C)
        out = torch.empty(shape, dtype=o.dtype, device=o.device)
    _check(lib().rva_out_projection(_ptr(o), _ptr(kept_index), _ptr(cu_seqlens), _ptr(m), B, N, C,
                                    _ptr(w_o), _ptr(b_o), _ptr(residual), dtype_code(o), _ptr(out),
                                    _stream(stream)), "rva_out_projection")
    return out


def empty(count: int = 1, stream=None):
    """Enqueue `count` empty one-workgroup kernels (dispatch-floor probe)."""
    _check(lib().rva_empty(int(count), _stream(stream)), "rva_empty")


class Plan:
    """A captured launch sequence (HIP graph) replayed with one launch, or
    (mode FUSED_DIRECT) the fused launch validated once and enqueued directly
    by every launch().

    Tensors given here are kept alive by the plan; their contents may change
    between launches, their addresses may not.
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
            B, N, H, d = q.shape
            desc.B, desc.N, desc.H, desc.d = B, N, H, d
            desc.dtype = dtype_code(q)
            desc.max_seqlen_hint = int(max_seqlen_hint)
            desc.softmax_scale = float(scale or 0.0)
            desc.q_pad, desc.k_pad, desc.v_pad = q.data_ptr(), k.data_ptr(), v.data_ptr()
            desc.mask = _mask_u8(mask).data_ptr()
            desc.o_pad = out.data_ptr()
            if packed is not None:
                desc.q_packed = packed["q"].data_ptr()
                desc.k_packed = packed["k"].data_ptr()
                desc.v_packed = packed["v"].data_ptr()
                desc.o_packed = packed["o"].data_ptr()
            desc.cu_seqlens = cu_seqlens.data_ptr() if cu_seqlens is not None else None
            desc.max_seqlen = max_seqlen.data_ptr() if max_seqlen is not None else None
            desc.kept_index = kept_index.data_ptr() if kept_index is not None else None
            if mode == L2_FUSED:
                _req(x, "x")
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
        _req(x, "x")
        B, N, C = x.shape
        H = C // HEAD_DIM
        L = len(weights)
        m = _mask_u8(mask)
        dev = x.device
        self.scratch = {nm: torch.empty((B * N, C), dtype=x.dtype, device=dev)
                        for nm in ("resid", "q", "k", "v", "o")}
        self.cu_seqlens = torch.empty(B + 1, dtype=torch.int32, device=dev)
        self.max_seqlen = torch.empty(1, dtype=torch.int32, device=dev)
        self.kept_index = torch.empty(B * N, dtype=torch.int32, device=dev)
        self.out = out if out is not None else torch.empty_like(x)
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
