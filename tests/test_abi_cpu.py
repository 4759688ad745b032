"""Host-only checks of the C ABI: the library loads, exports every function
include/rva.h declares, and rejects invalid arguments before touching the
device (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("rva.h", "rva_probe.h")]


def _declared():
    src = "\n".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(rva_[a-z0-9_]+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    import ragged_variable_length_amd as rva
    if not os.path.exists(rva.LIB_PATH):
        from ragged_variable_length_amd import _build
        _build.build()
    return rva.lib()


def test_header_lists_the_entry_points():
    names = _declared()
    for want in ("rva_pack", "rva_ragged_attend", "rva_unpack", "rva_fused", "rva_plan_create",
                 "rva_plan_launch", "rva_plan_destroy", "rva_empty", "rva_status_string",
                 "rva_last_error", "rva_version", "rva_threshold_l2_mask",
                 "rva_qkv_projection", "rva_out_projection", "rva_layers_plan_create",
                 "rva_fused_persistent", "rva_fused_persistent_noalloc"):
        assert want in names


def test_every_declared_symbol_is_exported(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings(L):
    assert L.rva_status_string(0) == b"ok"
    assert L.rva_status_string(-1) == b"invalid argument"
    assert L.rva_status_string(-2) == b"unsupported configuration"
    assert L.rva_status_string(-3) == b"HIP runtime error"
    assert L.rva_status_string(99) == b"unknown status"
    assert L.rva_version() == 104


FAKE = ctypes.c_void_p(0x7F0000000000)  # aligned, never dereferenced: validation fails first
MIS = ctypes.c_void_p(0x7F0000000008)   # 8-byte aligned only


def _pack(L, B=2, N=8, H=1, d=64, dt=1, q=FAKE, mask=FAKE, qo=FAKE, cu=FAKE):
    return L.rva_pack(q, None, None, mask, B, N, H, d, dt, qo, None, None, cu, None, None, None)


def test_pack_validation(L):
    assert _pack(L, mask=None) == -1 and b"mask" in L.rva_last_error()
    assert _pack(L, B=0) == -1
    assert _pack(L, N=0) == -1 and _pack(L, N=1025) == -1
    assert _pack(L, H=0) == -1 and _pack(L, H=65) == -1
    assert _pack(L, d=32) == -2 and b"head_dim" in L.rva_last_error()
    assert _pack(L, dt=7) == -1 and b"dtype" in L.rva_last_error()
    assert _pack(L, qo=None) == -1 and b"both" in L.rva_last_error()
    assert _pack(L, q=MIS) == -1 and b"aligned" in L.rva_last_error()
    assert _pack(L, cu=None) == -1 and b"cu_seqlens" in L.rva_last_error()
    assert _pack(L, B=1 << 22, N=1024) == -1


def test_attend_unpack_fused_validation(L):
    f = ctypes.c_float(0.0)
    assert L.rva_ragged_attend(FAKE, FAKE, FAKE, None, 2, 2, 64, 10, f, 1, FAKE, None) == -1
    assert L.rva_ragged_attend(FAKE, None, FAKE, FAKE, 2, 2, 64, 10, f, 1, FAKE, None) == -1
    assert L.rva_ragged_attend(FAKE, FAKE, FAKE, FAKE, 2, 2, 128, 10, f, 1, FAKE, None) == -2
    assert L.rva_unpack(FAKE, FAKE, None, 2, 8, 1, 64, 1, FAKE, None) == -1
    assert L.rva_unpack(FAKE, FAKE, FAKE, 2, 8, 1, 64, 1, MIS, None) == -1
    assert L.rva_fused(FAKE, FAKE, FAKE, FAKE, 2, 8, 1, 64, 0, f, 1, None, None, None, None) == -1
    assert L.rva_fused(FAKE, FAKE, FAKE, FAKE, 2, 8, 1, 64, 0, f, 3, FAKE, None, None, None) == -1
    assert L.rva_fused(FAKE, FAKE, FAKE, FAKE, 2, 8, 1, 64, 0, f, 1, FAKE,
                       ctypes.c_void_p(0x7F0000000002), None, None) == -1
    assert L.rva_empty(-1, None) == -1
    # persistent form: the work counter is required and 4-byte aligned
    assert L.rva_fused_persistent(FAKE, FAKE, FAKE, FAKE, 2, 8, 1, 64, 0, f, 1, FAKE, None, None,
                                  None, None) == -1 and b"work" in L.rva_last_error()
    assert L.rva_fused_persistent(FAKE, FAKE, FAKE, FAKE, 2, 8, 1, 64, 0, f, 1, FAKE, None, None,
                                  ctypes.c_void_p(0x7F0000000002), None) == -1
    assert L.rva_fused_persistent(FAKE, FAKE, FAKE, None, 2, 8, 1, 64, 0, f, 1, FAKE, None, None,
                                  FAKE, None) == -1 and b"mask" in L.rva_last_error()


def test_threshold_validation(L):
    def thr(x=FAKE, B=2, N=197, C=384, dt=0, q=0.5, m=FAKE):
        return L.rva_threshold_l2_mask(x, B, N, C, dt, ctypes.c_double(q), m, None)
    assert thr(x=None) == -1 and b"x is NULL" in L.rva_last_error()
    assert thr(m=None) == -1 and b"mask_out" in L.rva_last_error()
    assert thr(x=MIS) == -1 and b"aligned" in L.rva_last_error()
    assert thr(B=0) == -1 and thr(N=0) == -1 and thr(N=1025) == -1
    assert thr(C=0) == -1 and thr(C=65537) == -1
    assert thr(C=6, dt=0) == -1 and b"16 bytes" in L.rva_last_error()
    assert thr(C=12, dt=1) == -1 and thr(C=12, dt=2) == -1
    assert thr(dt=5) == -1 and b"dtype" in L.rva_last_error()
    assert thr(q=-0.1) == -1 and thr(q=1.5) == -1 and thr(q=float("nan")) == -1
    assert b"keep_quantile" in L.rva_last_error()
    assert thr(B=1 << 22, N=1024) == -1


def test_projection_validation(L):
    def qkv(x=FAKE, idx=FAKE, cu=FAKE, B=2, N=197, C=768, w=FAKE, b=None, dt=1, q=FAKE):
        return L.rva_qkv_projection(x, idx, cu, B, N, C, w, b, dt, q, FAKE, FAKE, None)
    assert qkv(x=None) == -1 and qkv(w=None) == -1 and qkv(q=None) == -1
    assert qkv(cu=None) == -1 and b"cu_seqlens" in L.rva_last_error()
    assert qkv(dt=0) == -2 and b"fp16 or bf16" in L.rva_last_error()
    assert qkv(dt=4) == -1
    assert qkv(C=100) == -1 and qkv(C=0) == -1 and qkv(C=64 * 65) == -1
    assert qkv(B=1024, N=1024, C=2048) == -1 and b"2^31" in L.rva_last_error()
    assert qkv(x=MIS) == -1 and qkv(b=MIS) == -1
    assert qkv(idx=ctypes.c_void_p(0x7F0000000002)) == -1

    def outp(o=FAKE, idx=FAKE, cu=FAKE, m=FAKE, C=768, w=FAKE, res=None, y=FAKE):
        return L.rva_out_projection(o, idx, cu, m, 2, 197, C, w, None, res, 1, y, None)
    assert outp(m=None) == -1 and b"mask" in L.rva_last_error()
    assert outp(o=None) == -1 and outp(y=None) == -1 and outp(w=None) == -1
    assert outp(res=MIS) == -1 and outp(C=32) == -1


def test_layers_plan_validation(L):
    import ragged_variable_length_amd as rva
    d = rva._LayersDesc()
    h = ctypes.c_void_p()
    assert L.rva_layers_plan_create(None, ctypes.byref(h)) == -1
    d.B, d.N, d.H, d.d, d.dtype, d.layers = 2, 197, 12, 64, 1, 0
    assert L.rva_layers_plan_create(ctypes.byref(d), ctypes.byref(h)) == -1
    assert b"layers" in L.rva_last_error()
    d.layers = 65
    assert L.rva_layers_plan_create(ctypes.byref(d), ctypes.byref(h)) == -1
    d.layers = 2
    assert L.rva_layers_plan_create(ctypes.byref(d), ctypes.byref(h)) == -1  # no weight arrays
    assert b"w_qkv" in L.rva_last_error()
    arr = (ctypes.c_void_p * 2)(0x7F0000000000, None)  # second layer's weight missing
    d.w_qkv = d.w_o = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    for f in ("x_pad", "mask", "resid", "q", "k", "v", "o", "cu_seqlens", "kept_index", "y_pad"):
        setattr(d, f, 0x7F0000000000)
    assert L.rva_layers_plan_create(ctypes.byref(d), ctypes.byref(h)) == -1
    assert b"w_qkv" in L.rva_last_error()
    d.dtype = 0
    assert L.rva_layers_plan_create(ctypes.byref(d), ctypes.byref(h)) == -2
    assert h.value is None


def test_plan_validation(L):
    import ragged_variable_length_amd as rva
    d = rva._PlanDesc()
    h = ctypes.c_void_p()
    d.mode = 9
    assert L.rva_plan_create(ctypes.byref(d), ctypes.byref(h)) == -1
    assert L.rva_plan_create(None, ctypes.byref(h)) == -1
    d.mode = rva.FUSED
    d.B, d.N, d.H, d.d, d.dtype = 2, 8, 1, 64, 1
    assert L.rva_plan_create(ctypes.byref(d), ctypes.byref(h)) == -1  # null pointers
    assert h.value is None
    d.mode = rva.L2_FUSED
    d.q_pad = d.k_pad = d.v_pad = d.o_pad = 0x7F0000000000
    d.mask = None
    d.x, d.C, d.x_dtype, d.keep_quantile, d.mask_out = 0x7F0000000000, 384, 0, 2.0, 0x7F0000000000
    assert L.rva_plan_create(ctypes.byref(d), ctypes.byref(h)) == -1  # keep_quantile range
    assert b"keep_quantile" in L.rva_last_error()
    d.keep_quantile, d.mask_out = 0.5, None
    assert L.rva_plan_create(ctypes.byref(d), ctypes.byref(h)) == -1
    assert b"mask_out" in L.rva_last_error()
    assert L.rva_plan_launch(None, None) == -1
    assert L.rva_plan_destroy(None) == 0


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import ragged_variable_length_amd as rva
    monkeypatch.setattr(rva, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(rva, "_lib", None)
    with pytest.raises(ImportError):
        rva.lib()


def test_persistent_item_limit(L):
    """B*H >= 2^30 would wrap the persistent form's 32-bit work counter: both
    persistent entry points reject it by host arithmetic, before any HIP
    call (none can succeed here without a GPU, so reaching one would show as
    a different error)."""
    f = ctypes.c_float(0.0)
    st = L.rva_fused_persistent(FAKE, FAKE, FAKE, FAKE, 1 << 24, 1, 64, 64, 0, f, 1, FAKE, None,
                                None, FAKE, None)
    assert st == -1 and b"counter" in L.rva_last_error()
    st = L.rva_fused_persistent_noalloc(FAKE, FAKE, FAKE, FAKE, 1 << 24, 1, 64, 64, 0, f, 1, FAKE,
                                        None, None, None)
    assert st == -1 and b"counter" in L.rva_last_error()
    st = L.rva_fused_persistent_noalloc(FAKE, FAKE, FAKE, None, 4, 8, 2, 64, 0, f, 1, FAKE,
                                        None, None, None)
    assert st == -1 and b"mask" in L.rva_last_error()


def test_probe_validation(L):
    """The ceiling probes reject bad sizes and overlapping buffers before any
    HIP call."""
    LL = ctypes.c_longlong
    assert L.rva_probe_copy(FAKE, MIS, LL(1024), 4, None) == -1 and b"aligned" in L.rva_last_error()
    assert L.rva_probe_copy(FAKE, ctypes.c_void_p(0x7F0000000100), LL(1024), 4, None) == -1
    assert b"overlap" in L.rva_last_error()
    assert L.rva_probe_copy(FAKE, ctypes.c_void_p(0x7F0000100000), LL(24), 4, None) == -1
    assert L.rva_probe_read(FAKE, FAKE, LL(0), 4, None) == -1
    assert L.rva_probe_read(FAKE, FAKE, LL(1024), 0, None) == -1
    assert L.rva_probe_mfma(0, FAKE, 4, None, None) == -1
    # gather probe: shapes as rva_fused (16-bit), every pointer present and aligned
    g = L.rva_probe_gather
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 197, 12, None) == -1
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 197, 0, None) == -1
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1 << 20, 12, None) == -1
    assert g(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 197, 12, None) == -1
    assert b"q" in L.rva_last_error()
    assert g(FAKE, FAKE, FAKE, MIS, FAKE, FAKE, FAKE, 4, 197, 12, None) == -1
    assert b"aligned" in L.rva_last_error()
    assert g(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 4, 197, 12, None) == -1
    assert b"mask" in L.rva_last_error()
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 197, 12, None) == -1
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 4, 197, 12, None) == -1
    assert b"kept_index" in L.rva_last_error()
