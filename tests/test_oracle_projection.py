"""Pins for the projection oracle, independent of its own code.  Checks take
the oracle's routines as arguments so that the mutation tests can plant
mistakes in stand-ins and confirm a pin catches each."""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle import projection as PJ


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ------------------------------------------------------------------ pin checks

def check_bruteforce(linear):
    """Scalar triple loop in pure Python on tiny inputs."""
    rng = _rng(31)
    M, K, Nout = 5, 7, 6
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((Nout, K))
    b = rng.standard_normal(Nout)
    r = rng.standard_normal((M, Nout))
    got = linear(x, w, b, r)
    for m in range(M):
        for n in range(Nout):
            acc = 0.0
            for k in range(K):
                acc += float(x[m, k]) * float(w[n, k])
            assert abs(got[m, n] - (acc + b[n] + r[m, n])) < 1e-12


def check_closed_forms(linear):
    """Identity weight returns x + b; zero weight returns b; a one-hot weight
    row picks one input column."""
    rng = _rng(32)
    x = rng.standard_normal((9, 8))
    b = rng.standard_normal(8)
    assert np.allclose(linear(x, np.eye(8), b), x + b, rtol=0, atol=1e-15)
    assert np.array_equal(linear(x, np.zeros((8, 8)), b), np.broadcast_to(b, (9, 8)))
    w = np.zeros((3, 8))
    w[0, 5] = w[1, 0] = w[2, 7] = 1.0
    assert np.array_equal(linear(x, w), x[:, [5, 0, 7]])


def check_linearity(linear):
    rng = _rng(33)
    x1, x2 = rng.standard_normal((2, 6, 10))
    w = rng.standard_normal((4, 10))
    y = linear(2.0 * x1 - 3.0 * x2, w)
    assert np.allclose(y, 2.0 * linear(x1, w) - 3.0 * linear(x2, w), rtol=0, atol=1e-12)


def check_qkv_split(qkv_projection):
    """The three outputs are the column groups of one product on the packed
    rows: q uses weight rows 0..C-1, k rows C..2C-1, v rows 2C..3C-1."""
    rng = _rng(34)
    B, N, C = 3, 11, 16
    x = rng.standard_normal((B, N, C)).astype(np.float32).astype(np.float16)
    mask = (rng.random((B, N)) < 0.6).astype(np.uint8)
    w = (rng.standard_normal((3 * C, C)) * 0.25).astype(np.float32).astype(np.float16)
    b = rng.standard_normal(3 * C).astype(np.float32).astype(np.float16)
    q, k, v = qkv_projection(x, mask, w, b, "f16")
    xf = x.astype(np.float64)
    rows = [xf[i, j] for i in range(B) for j in range(N) if mask[i, j]]
    xp = np.array(rows).reshape(-1, C)
    wf, bf = w.astype(np.float64), b.astype(np.float64)
    for t, part in enumerate((q, k, v)):
        ref = xp @ wf[t * C:(t + 1) * C].T + bf[t * C:(t + 1) * C]
        assert part.shape == (int(mask.sum()), C)
        assert np.allclose(part, ref, rtol=0, atol=1e-12), t


def check_out_scatter(out_projection):
    """Padded output: kept rows are the packed product rows in kept order
    (plus the padded residual), pruned rows exactly +0."""
    rng = _rng(35)
    B, N, C = 2, 9, 8
    mask = (rng.random((B, N)) < 0.5).astype(np.uint8)
    mask[:, 0] = 1
    T = int(mask.sum())
    o = rng.standard_normal((T, C)).astype(np.float32)
    w = rng.standard_normal((C, C)).astype(np.float32)
    b = rng.standard_normal(C).astype(np.float32)
    res = rng.standard_normal((B, N, C)).astype(np.float32)
    y = out_projection(o, mask, w, b, "f32", residual=res)
    r = 0
    for i in range(B):
        for j in range(N):
            if mask[i, j]:
                ref = o[r].astype(np.float64) @ w.astype(np.float64).T + b + res[i, j]
                assert np.allclose(y[i, j], ref, rtol=0, atol=1e-12)
                r += 1
            else:
                assert np.all(y[i, j] == 0) and not np.any(np.signbit(y[i, j]))
    # packed form equals the kept rows of the padded form
    yp = out_projection(o, None, w, b, "f32", residual=oracle.pack_rows(res, mask))
    assert np.allclose(yp, oracle.pack_rows(y, mask), rtol=0, atol=1e-12)


CHECKS_LINEAR = [check_bruteforce, check_closed_forms, check_linearity]


@pytest.mark.parametrize("check", CHECKS_LINEAR, ids=lambda f: f.__name__)
def test_linear_pins(check):
    check(PJ.linear)


def test_qkv_pin():
    check_qkv_split(PJ.qkv_projection)


def test_out_pin():
    check_out_scatter(PJ.out_projection)


def test_weights_generator():
    wts = W.projection_weights(C=64, dtype="f16")
    assert wts["w_qkv"].shape == (192, 64) and wts["b_qkv"].shape == (192,)
    assert wts["w_o"].shape == (64, 64) and wts["b_o"].shape == (64,)
    wq = wts["w_qkv"].astype(np.float64)
    assert 0.5 / 64 < wq.var() < 2.0 / 64  # variance 1/C


# ------------------------------------------------------------------ mutations

def _lin_transposed(x, w, b=None, residual=None):
    # weight used as [K, Nout] instead of [Nout, K]
    y = np.asarray(x, np.float64) @ np.asarray(w, np.float64)
    return y + (b if b is not None else 0) + (residual if residual is not None else 0)


def _lin_no_bias(x, w, b=None, residual=None):
    return PJ.linear(x, w, None, residual)


def _lin_no_residual(x, w, b=None, residual=None):
    return PJ.linear(x, w, b, None)


def _lin_bias_twice(x, w, b=None, residual=None):
    y = PJ.linear(x, w, b, residual)
    return y + (b if b is not None else 0)


@pytest.mark.parametrize("fn", [_lin_transposed, _lin_no_bias, _lin_no_residual, _lin_bias_twice],
                         ids=lambda f: f.__name__)
def test_linear_mutant_caught(fn):
    caught = 0
    for check in CHECKS_LINEAR:
        try:
            check(fn)
        except (AssertionError, ValueError):
            caught += 1
    assert caught >= 1


def _qkv_swapped(x_pad, mask, w, b, dtype):
    q, k, v = PJ.qkv_projection(x_pad, mask, w, b, dtype)
    return k, q, v


def _qkv_unpacked_rows(x_pad, mask, w, b, dtype):
    x = oracle.decode(x_pad, dtype).reshape(-1, x_pad.shape[-1])[: int(mask.sum())]
    y = PJ.linear(x, oracle.decode(w, dtype), oracle.decode(b, dtype))
    C = w.shape[1]
    return y[:, :C], y[:, C:2 * C], y[:, 2 * C:]


@pytest.mark.parametrize("fn", [_qkv_swapped, _qkv_unpacked_rows], ids=lambda f: f.__name__)
def test_qkv_mutant_caught(fn):
    with pytest.raises(AssertionError):
        check_qkv_split(fn)


def _out_residual_everywhere(o, mask, w, b, dtype, residual=None):
    y = PJ.out_projection(o, mask, w, b, dtype)
    if residual is not None:  # residual added to pruned rows too
        y = y + oracle.decode(residual, dtype)
    return y


def _out_reversed_rows(o, mask, w, b, dtype, residual=None):
    return PJ.out_projection(o[::-1].copy(), mask, w, b, dtype, residual)


@pytest.mark.parametrize("fn", [_out_residual_everywhere, _out_reversed_rows], ids=lambda f: f.__name__)
def test_out_mutant_caught(fn):
    with pytest.raises(AssertionError):
        check_out_scatter(fn)
