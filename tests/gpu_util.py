"""Helpers for the GPU tests: moving workloads to the device and comparing
device results with the oracle.  Imports torch lazily-safe (CPU-only hosts
can import this module)."""
import numpy as np
import torch

TOL = {"f16": 2e-3, "bf16": 1e-2, "f32": 1e-4}


def to_dev(x: np.ndarray, dtype: str, dev) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.view(torch.int16).to(dev).view(torch.bfloat16)
    else:
        t = t.to(dev)
    return t


def upload(w, dev):
    q, k, v = (to_dev(x, w.dtype, dev) for x in (w.q, w.k, w.v))
    mask = torch.from_numpy(w.mask).to(dev)
    return q, k, v, mask


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a device tensor as a numpy unsigned array."""
    t = t.detach().contiguous().cpu()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.element_size() == 4:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.numpy()


def host_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    return x.view(np.uint16) if x.itemsize == 2 else x.view(np.uint32)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_err(got: np.ndarray, ref: np.ndarray) -> float:
    if got.size == 0:
        return 0.0
    assert np.isfinite(got).all(), "non-finite value in device output"
    return float(np.abs(got - ref).max())


# Projection tolerance, derived from the arithmetic: products of two 16-bit
# values are exact in fp32, the K-term sum is accumulated in fp32 (error at
# most (K + 2) 2^-24 times the sum of |terms|, bias and residual included),
# and the result is rounded once to the output type (half an ulp: 2^-11
# relative for fp16, 2^-8 for bf16, plus fp16's subnormal spacing near zero).
U_OUT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
ABS_FLOOR = {"f16": 2.0 ** -24, "bf16": 2.0 ** -133}


def linear_bound(xs, w, b, r, dtype=None):
    """Accumulation part of the bound for y = xs w^T + b + r (fp64 decoded);
    the same for every 16-bit input type."""
    K = xs.shape[1]
    mag = np.abs(xs) @ np.abs(w).T
    if b is not None:
        mag = mag + np.abs(b)
    if r is not None:
        mag = mag + np.abs(r)
    return mag * (K + 2) * 2.0 ** -24


def check_linear(got, ref, mag_bound, dtype, what):
    """Every element within its own bound."""
    tol = U_OUT[dtype] * np.abs(ref) + mag_bound * (1 + U_OUT[dtype]) + ABS_FLOOR[dtype]
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), what
    bad = err > tol
    assert not bad.any(), (what, float(err.max()), np.argwhere(bad)[:4])


# The 1024-image mixed batch and its oracle output, computed once per test
# session and shared by every full-size check (about 10 s of CPU work).
_MIXED = {}


def mixed_full():
    """dict(w=workload, ref=oracle O at the kept positions [T, H, 64] float64
    in kept-index order, cu=cu_seqlens, mx=max_seqlen, keep=bool [B, N])."""
    if not _MIXED:
        import oracle
        import workloads as W
        w = W.mixed_peak()
        ref, cu, mx, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype)
        keep = w.mask.astype(bool)
        _MIXED.update(w=w, ref=ref[keep], cu=cu, mx=mx, keep=keep)
        del ref
    return _MIXED


def check_mixed_full(out: torch.Tensor, what: str, cu=None, mx=None) -> float:
    """Every element of a padded device output of the mixed batch against the
    oracle: pruned rows exactly +0, kept rows within the fp16 bound; offsets
    bit-exact when given.  Returns the max abs error."""
    m = mixed_full()
    b = bits(out)
    assert (b[~m["keep"]] == 0).all(), f"{what}: pruned rows not +0"
    got = b[m["keep"]].view(np.float16).astype(np.float64)
    err = max_err(got, m["ref"])
    assert err <= TOL["f16"], f"{what}: max abs err {err:.3e}"
    if cu is not None:
        assert np.array_equal(cu.cpu().numpy(), m["cu"]), f"{what}: cu_seqlens"
    if mx is not None:
        assert int(mx.item()) == int(m["mx"]), f"{what}: max_seqlen"
    return err
