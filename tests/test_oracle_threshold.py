"""Pins for the Threshold-l2 keep-mask oracle, independent of its own code.

The checks take the mask and squared-norm routines as arguments so that the
mutation tests at the bottom can plant plausible mistakes in stand-ins for
the oracle and confirm that some pin catches each one.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import threshold_l2 as TL


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _fsum_sq(x64):
    """Exactly rounded sum of squares per row (Shewchuk's algorithm via math.fsum)."""
    B, N, C = x64.shape
    out = np.empty((B, N))
    for b in range(B):
        for j in range(N):
            out[b, j] = math.fsum(float(v) * float(v) for v in x64[b, j])
    return out


# ------------------------------------------------------------------ pin checks

def check_sq_norms_vs_fsum(sq_norms):
    """Channel-order fp64 sum within its textbook error bound of the exactly
    rounded sum (|err| <= (C - 1) u sum for non-negative terms)."""
    x = _rng(11).standard_normal((3, 9, 384)).astype(np.float32)
    got = sq_norms(x, "f32")
    ref = _fsum_sq(x.astype(np.float64))
    bound = 383 * 2.0 ** -53 * ref
    assert np.all(np.abs(got - ref) <= bound + 1e-300), np.abs(got - ref).max()


def check_sq_norms_integers(sq_norms):
    """Small integers: every square and partial sum is exact, so the result is
    the exact integer sum of squares."""
    rng = _rng(12)
    x = rng.integers(-40, 41, size=(2, 5, 33)).astype(np.float32)
    ref = (x.astype(np.int64) ** 2).sum(axis=2).astype(np.float64)
    assert np.array_equal(sq_norms(x, "f32"), ref)


def check_quantile_rule(mask_fn):
    """Against numpy's linear-interpolation quantile on norms without near-ties:
    CLS kept, patch kept iff its norm >= np.quantile(patch norms, q)."""
    for seed, (B, N, C) in ((13, (5, 197, 64)), (14, (3, 50, 16)), (15, (2, 577, 32))):
        x = _rng(seed).standard_normal((B, N, C)).astype(np.float32)
        norms = np.sqrt(_fsum_sq(x.astype(np.float64)))
        for b in range(B):  # guard: no two patch norms within 1e-9 relative
            s = np.sort(norms[b, 1:])
            assert np.all(np.diff(s) > 1e-9 * s[1:])
        for q in (0.1, 0.25, 0.5, 0.7, 0.9, 0.33):
            ref = np.zeros((B, N), dtype=np.uint8)
            ref[:, 0] = 1
            for b in range(B):
                thr = np.quantile(norms[b, 1:], q)
                ref[b, 1:] = norms[b, 1:] >= thr
            got = mask_fn(x, "f32", q)
            assert np.array_equal(got, ref), (seed, q)


def check_bruteforce_ties(mask_fn):
    """Tiny integer inputs with many equal norms against a pure-Python
    sort-and-threshold loop (keep iff norm >= the r0-th smallest)."""
    rng = _rng(16)
    for N in (1, 2, 3, 7, 12):
        x = rng.integers(-2, 3, size=(3, N, 3)).astype(np.float32)
        for q in (0.0, 0.2, 0.5, 0.75, 1.0):
            got = mask_fn(x, "f32", q)
            for b in range(3):
                sq = [sum(int(v) * int(v) for v in x[b, j]) for j in range(N)]
                patches = sq[1:]
                exp = [1] + [0] * (N - 1)
                if patches:
                    order = sorted(patches)
                    r0 = math.ceil(q * (len(patches) - 1))
                    for j in range(1, N):
                        exp[j] = 1 if sq[j] >= order[r0] else 0
                assert list(got[b]) == exp, (N, q, b)


def check_closed_form_counts(mask_fn):
    """Distinct norms: exactly P - ceil(q (P - 1)) patches kept, and they are
    the largest ones; q = 0 keeps every patch, q = 1 only the largest."""
    x = _rng(17).standard_normal((4, 197, 48)).astype(np.float32)
    norms = _fsum_sq(x.astype(np.float64))
    P = 196
    for q in (0.0, 0.05, 0.5, 0.8, 0.99, 1.0):
        m = mask_fn(x, "f32", q)
        assert np.all(m[:, 0] == 1)
        k = P - math.ceil(q * (P - 1))
        assert np.all(m[:, 1:].sum(axis=1) == k), q
        for b in range(4):
            top = np.argsort(norms[b, 1:])[::-1][:k] + 1
            assert np.all(m[b, top] == 1)


def check_cls_independent(mask_fn):
    """CLS takes no part in the ranking: scaling token 0 changes nothing."""
    x = _rng(18).standard_normal((2, 40, 8)).astype(np.float32)
    y = x.copy()
    y[:, 0] *= 1000.0
    for q in (0.3, 0.5):
        assert np.array_equal(mask_fn(x, "f32", q), mask_fn(y, "f32", q))


ALL_CHECKS_SQ = [check_sq_norms_vs_fsum, check_sq_norms_integers]
ALL_CHECKS_MASK = [check_quantile_rule, check_bruteforce_ties, check_closed_form_counts,
                   check_cls_independent]


@pytest.mark.parametrize("check", ALL_CHECKS_SQ, ids=lambda f: f.__name__)
def test_sq_norms_pins(check):
    check(oracle.sq_norms)


@pytest.mark.parametrize("check", ALL_CHECKS_MASK, ids=lambda f: f.__name__)
def test_mask_pins(check):
    check(oracle.threshold_l2_mask)


def test_dtypes_decode_consistently():
    """16-bit inputs give the norms of their decoded values."""
    x = _rng(19).standard_normal((2, 10, 64)).astype(np.float32)
    h = x.astype(np.float16)
    assert np.array_equal(oracle.sq_norms(h, "f16"), oracle.sq_norms(h.astype(np.float32), "f32"))
    b = W.f32_to_bf16_bits(x)
    bf = (b.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(oracle.sq_norms(b, "bf16"), oracle.sq_norms(bf, "f32"))


def test_generator_mask_agrees():
    """The DeiT-S input recipe draws its mask with numpy's quantile on fp64
    embeddings; the oracle on the same embeddings rounded to fp32 agrees."""
    w = W.deit_s_224_threshold_l2()
    x32 = w.meta["x"]
    assert x32.dtype == np.float32 and x32.shape == (w.B, w.N, 384)
    assert np.array_equal(oracle.threshold_l2_mask(x32, "f32", 0.5), w.mask)


def test_keep_rank_and_validation():
    assert oracle.keep_rank(197, 0.5) == 98
    assert oracle.keep_rank(197, 0.0) == 0
    assert oracle.keep_rank(197, 1.0) == 195
    assert oracle.keep_rank(1, 0.5) == 0
    assert oracle.keep_rank(2, 0.7) == 0
    with pytest.raises(ValueError):
        oracle.threshold_l2_mask(np.zeros((1, 3, 4), np.float32), "f32", 1.5)


# ------------------------------------------------------------------ mutations
# Plausible mistakes planted in stand-ins for the oracle; some pin must fail.

def _mask_from(sq_fn, rank_fn=TL.keep_rank, strict=False, include_cls=False):
    def mask_fn(x, dtype, q):
        s = sq_fn(x, dtype)
        B, N = s.shape
        r0 = rank_fn(N, q)
        m = np.zeros((B, N), dtype=np.uint8)
        m[:, 0] = 1
        for b in range(B):
            pool = s[b, :] if include_cls else s[b, 1:]
            p = s[b, 1:]
            if strict:
                cnt = (pool[None, :] < p[:, None]).sum(axis=1)
                m[b, 1:] = cnt >= r0
            else:
                cnt = (pool[None, :] <= p[:, None]).sum(axis=1)
                m[b, 1:] = cnt >= r0 + 1
        return m
    return mask_fn


def _sq_drop_last(x, dtype):
    xf = oracle.decode(x, dtype)[..., :-1]
    return (xf * xf).sum(axis=-1)


def _sq_abs(x, dtype):
    return np.abs(oracle.decode(x, dtype)).sum(axis=-1)


def _sq_shifted(x, dtype):
    xf = oracle.decode(x, dtype)
    return (xf * np.roll(xf, 1, axis=-1)).sum(axis=-1)


MUTANTS = {
    "strict_less_ties": _mask_from(oracle.sq_norms, strict=True),
    "cls_in_ranking": _mask_from(oracle.sq_norms, include_cls=True),
    "floor_rank": _mask_from(oracle.sq_norms,
                             rank_fn=lambda N, q: int(math.floor(q * max(N - 2, 0)))),
    "rank_over_P": _mask_from(oracle.sq_norms,
                              rank_fn=lambda N, q: int(math.ceil(q * max(N - 1, 0)))),
    "dropped_channel": _mask_from(_sq_drop_last),
    "l1_not_l2": _mask_from(_sq_abs),
    "shifted_index": _mask_from(_sq_shifted),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_caught(name):
    fn = MUTANTS[name]
    caught = 0
    for check in ALL_CHECKS_MASK:
        try:
            check(fn)
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin catches mutant {name}"


@pytest.mark.parametrize("fn", [_sq_drop_last, _sq_abs, _sq_shifted], ids=lambda f: f.__name__)
def test_sq_mutant_caught(fn):
    caught = 0
    for check in ALL_CHECKS_SQ:
        try:
            check(fn)
        except AssertionError:
            caught += 1
    assert caught >= 1
