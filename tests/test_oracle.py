"""Pins for the fp64 oracle, independent of the oracle's own code.

Each check is written as a function of the attention (or pack) routine it
tests, so that the mutation tests at the bottom can plant a plausible mistake
in a copy of the oracle and confirm that at least one pin catches it.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import ragged as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "attention_closed_form.json")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _ragged(seed, counts, H, d, scale=1.0):
    rng = _rng(seed)
    counts = np.asarray(counts)
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(cu[-1])
    q = rng.standard_normal((T, H, d)) * scale
    k = rng.standard_normal((T, H, d)) * scale
    v = rng.standard_normal((T, H, d))
    return q, k, v, cu


# ------------------------------------------------------------------ pin checks
# Each returns None on success and raises AssertionError otherwise.

def check_golden(attend):
    fx_all = json.load(open(GOLDEN))["fixtures"]
    for fx in fx_all:
        m = np.array(fx["mask"], dtype=np.uint8)
        q, k, v = (np.array(fx[n], dtype=np.float64) for n in ("q", "k", "v"))
        cu = np.array(fx["expected_cu_seqlens"], dtype=np.int32)
        idx = np.array(fx["expected_kept_index"], dtype=np.int64)
        B, N = m.shape
        flat = lambda x: x.reshape((B * N,) + x.shape[2:])[idx]
        o = attend(flat(q), flat(k), flat(v), cu, fx["scale"])
        out = np.zeros((B * N,) + o.shape[1:])
        out[idx] = o
        e = np.array(fx["expected_o_fraction"], dtype=np.float64)
        e = (e[..., 0] / e[..., 1]).reshape(out.shape)
        assert np.abs(out - e).max() < 1e-12, np.abs(out - e).max()


def _brute(q, k, v, cu, scale):
    """Scalar pure-Python attention: one query, one key, one exp at a time."""
    T, H, d = q.shape
    out = [[[0.0] * d for _ in range(H)] for _ in range(T)]
    for b in range(len(cu) - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        for h in range(H):
            for i in range(lo, hi):
                logits = []
                for j in range(lo, hi):
                    s = 0.0
                    for c in range(d):
                        s += float(q[i, h, c]) * float(k[j, h, c])
                    logits.append(s * scale)
                top = max(logits)
                w = [math.exp(x - top) for x in logits]
                z = sum(w)
                for c in range(d):
                    acc = 0.0
                    for jj, j in enumerate(range(lo, hi)):
                        acc += w[jj] * float(v[j, h, c])
                    out[i][h][c] = acc / z
    return np.array(out, dtype=np.float64).reshape(T, H, d)


def check_brute_force(attend):
    for seed, counts, H, d in [(1, [3, 1, 5], 2, 4), (2, [0, 7, 2], 1, 3), (3, [8], 2, 2),
                               (4, [2, 0, 0, 4], 3, 4)]:
        q, k, v, cu = _ragged(seed, counts, H, d)
        scale = 1.0 / math.sqrt(d)
        got = attend(q, k, v, cu, None)
        ref = _brute(q, k, v, cu, scale)
        assert np.abs(got - ref).max() < 1e-12


def check_sdpa_masked_dense(attend):
    """Masked-dense equivalence through torch's SDPA in fp64 on CPU: padded
    [B, H, N, d] inputs with a key mask give the same rows at kept queries."""
    import torch
    import torch.nn.functional as Fn
    rng = _rng(11)
    B, N, H, d = 3, 13, 2, 8
    mask = (rng.random((B, N)) < 0.6).astype(np.uint8)
    mask[:, 0] = 1
    q = rng.standard_normal((B, N, H, d))
    k = rng.standard_normal((B, N, H, d))
    v = rng.standard_normal((B, N, H, d))
    cu, _ = R.seqlens(mask)
    o = attend(R.pack_rows(q, mask), R.pack_rows(k, mask), R.pack_rows(v, mask), cu, None)
    o_pad = R.unpack(o, mask)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
    am = torch.from_numpy(mask.astype(bool))[:, None, None, :].expand(B, H, N, N)
    ref = Fn.scaled_dot_product_attention(tq, tk, tv, attn_mask=am).permute(0, 2, 1, 3).numpy()
    keep = mask.astype(bool)
    assert np.abs(o_pad[keep] - ref[keep]).max() < 1e-12


def check_zero_pruning_is_padded_dense(attend):
    """0% pruning: the ragged path equals plain padded dense attention."""
    import torch
    import torch.nn.functional as Fn
    rng = _rng(12)
    B, N, H, d = 2, 9, 3, 8
    mask = np.ones((B, N), dtype=np.uint8)
    q, k, v = (rng.standard_normal((B, N, H, d)) for _ in range(3))
    cu, _ = R.seqlens(mask)
    o = attend(q.reshape(B * N, H, d), k.reshape(B * N, H, d), v.reshape(B * N, H, d), cu, None)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
    ref = Fn.scaled_dot_product_attention(tq, tk, tv).permute(0, 2, 1, 3).reshape(B * N, H, d)
    assert np.abs(o - ref.numpy()).max() < 1e-12


def check_q_zero_mean(attend):
    q, k, v, cu = _ragged(21, [5, 1, 9], 2, 6)
    q[:] = 0.0
    o = attend(q, k, v, cu, None)
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        mean = v[lo:hi].mean(axis=0)
        assert np.abs(o[lo:hi] - mean[None]).max() < 1e-12


def check_single_token(attend):
    q, k, v, cu = _ragged(22, [1, 1, 1], 2, 5, scale=30.0)
    o = attend(q, k, v, cu, None)
    assert np.array_equal(o, v)


def check_equal_keys_mean(attend):
    q, k, v, cu = _ragged(23, [4, 7], 2, 6)
    for b in range(len(cu) - 1):
        k[cu[b]:cu[b + 1]] = k[cu[b]][None]
    o = attend(q, k, v, cu, None)
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        assert np.abs(o[lo:hi] - v[lo:hi].mean(axis=0)[None]).max() < 1e-12


def check_permutation(attend):
    q, k, v, cu = _ragged(24, [6, 5], 2, 4)
    o = attend(q, k, v, cu, None)
    perm = np.concatenate([np.array([4, 0, 5, 2, 1, 3]), 6 + np.array([3, 4, 0, 2, 1])])
    o2 = attend(q[perm], k[perm], v[perm], cu, None)
    assert np.abs(o2 - o[perm]).max() < 1e-12
    # permuting keys and values together (queries fixed) leaves O unchanged
    o3 = attend(q, k[perm], v[perm], cu, None)
    assert np.abs(o3 - o).max() < 1e-12


def check_independence(attend):
    q, k, v, cu = _ragged(25, [4, 6, 3], 2, 4)
    o = attend(q, k, v, cu, None)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[4:10] += 5.0
    k2[4:10] *= -3.0
    v2[4:10] += 100.0
    o2 = attend(q2, k2, v2, cu, None)
    assert np.array_equal(o2[:4], o[:4]) and np.array_equal(o2[10:], o[10:])
    assert not np.array_equal(o2[4:10], o[4:10])


def check_key_shift(attend):
    q, k, v, cu = _ragged(26, [5, 8], 2, 4)
    o = attend(q, k, v, cu, None)
    k2 = k + np.array([0.7, -1.3, 2.0, 0.1])[None, None, :]
    assert np.abs(attend(q, k2, v, cu, None) - o).max() < 1e-11


def check_linear_in_v(attend):
    q, k, v, cu = _ragged(27, [5, 3], 2, 4)
    _, _, w, _ = _ragged(28, [5, 3], 2, 4)
    a = attend(q, k, 2.0 * v - 3.0 * w, cu, None)
    b = 2.0 * attend(q, k, v, cu, None) - 3.0 * attend(q, k, w, cu, None)
    assert np.abs(a - b).max() < 1e-11


def check_convex_bounds_and_hardmax(attend):
    q, k, v, cu = _ragged(29, [6, 9], 2, 4)
    o = attend(q, k, v, cu, None)
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        assert (o[lo:hi] <= v[lo:hi].max(axis=0)[None] + 1e-12).all()
        assert (o[lo:hi] >= v[lo:hi].min(axis=0)[None] - 1e-12).all()
    # large logits: stays finite and tends to the row of the best key
    big = attend(q * 1e4, k, v, cu, None)
    assert np.isfinite(big).all()
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        for h in range(q.shape[1]):
            s = q[lo:hi, h] @ k[lo:hi, h].T
            arg = s.argmax(axis=1)
            assert np.abs(big[lo:hi, h] - v[lo:hi, h][arg]).max() < 1e-6


ATTEND_PINS = [check_golden, check_brute_force, check_sdpa_masked_dense,
               check_zero_pruning_is_padded_dense, check_q_zero_mean, check_single_token,
               check_equal_keys_mean, check_permutation, check_independence, check_key_shift,
               check_linear_in_v, check_convex_bounds_and_hardmax]


@pytest.mark.parametrize("pin", ATTEND_PINS, ids=lambda f: f.__name__)
def test_attend_pin(pin):
    pin(R.attend)


# ------------------------------------------------------------------ pack / unpack pins

def _brute_pack(mask):
    B, N = len(mask), len(mask[0])
    cu, idx, mx = [0], [], 0
    for b in range(B):
        n = 0
        for j in range(N):
            if mask[b][j]:
                idx.append(b * N + j)
                n += 1
        cu.append(cu[-1] + n)
        mx = max(mx, n)
    return cu, idx, mx


def check_pack(seqlens, kept_index):
    rng = _rng(31)
    cases = [np.zeros((3, 5), np.uint8), np.ones((2, 7), np.uint8),
             (rng.random((6, 11)) < 0.4).astype(np.uint8), (rng.random((1, 1)) < 2).astype(np.uint8)]
    fx = json.load(open(GOLDEN))["fixtures"]
    for f in fx:
        m = np.array(f["mask"], np.uint8)
        cu, mx = seqlens(m)
        assert cu.tolist() == f["expected_cu_seqlens"] and mx == f["expected_max_seqlen"]
        assert kept_index(m).tolist() == f["expected_kept_index"]
    for m in cases:
        cu_b, idx_b, mx_b = _brute_pack(m.tolist())
        cu, mx = seqlens(m)
        idx = kept_index(m)
        assert cu.dtype == np.int32 and idx.dtype == np.int32
        assert cu.tolist() == cu_b and idx.tolist() == idx_b and mx == mx_b
        assert cu[-1] == m.sum() and (np.diff(cu) >= 0).all()


def test_pack_pins():
    check_pack(R.seqlens, R.kept_index)


def test_pack_rows_and_unpack_roundtrip():
    rng = _rng(32)
    B, N, H, d = 4, 10, 2, 3
    mask = (rng.random((B, N)) < 0.5).astype(np.uint8)
    x = rng.standard_normal((B, N, H, d)).astype(np.float16)
    p = R.pack_rows(x, mask)
    # brute force gather
    rows = [x[b, j] for b in range(B) for j in range(N) if mask[b, j]]
    assert np.array_equal(p.view(np.uint16), np.array(rows).view(np.uint16))
    u = R.unpack(p, mask)
    ref = np.where(mask[:, :, None, None].astype(bool), x, np.float16(0))
    assert np.array_equal(u.view(np.uint16), ref.view(np.uint16))
    # pruned rows are +0 (sign bit clear)
    assert (u.view(np.uint16)[mask == 0] == 0).all()
    # kept index strictly increasing inside each image
    idx = R.kept_index(mask)
    cu, _ = R.seqlens(mask)
    for b in range(B):
        seg = idx[cu[b]:cu[b + 1]]
        assert (np.diff(seg) > 0).all() and ((seg // N) == b).all()


def test_full_path_matches_components():
    rng = _rng(33)
    B, N, H, d = 3, 12, 2, 4
    mask = (rng.random((B, N)) < 0.5).astype(np.uint8)
    q, k, v = (rng.standard_normal((B, N, H, d)).astype(np.float32) for _ in range(3))
    o, cu, mx, idx = R.pack_attend_unpack(q, k, v, mask, "f32")
    for b in range(B):
        for h in range(H):
            keep, rows = R.attend_image_head(q, k, v, mask, "f32", b, h)
            assert np.abs(o[b, keep, h] - rows).max() < 1e-14
    assert (o[mask == 0] == 0).all()


# ------------------------------------------------------------------ decoding pins

def test_decode_bf16_known_bits():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x3EAB], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133,
            (1 + 0x2B / 128) * 2.0 ** -2]
    got = R.decode(bits, "bf16")
    assert got.tolist() == want
    assert math.copysign(1, got[3]) == -1


def test_decode_f16_known_bits():
    bits = np.array([0x3C00, 0xC000, 0x0001, 0x7BFF, 0x3555], dtype=np.uint16)
    want = [1.0, -2.0, 2.0 ** -24, 65504.0, (1 + 0x155 / 1024) * 2.0 ** -2]
    assert R.decode(bits.view(np.float16), "f16").tolist() == want


def test_decode_f32_exact():
    x = np.array([1.5, -3.25e-30, 7.0e30], dtype=np.float32)
    assert R.decode(x, "f32").tolist() == [float(t) for t in x]


# ------------------------------------------------------------------ mutation tests
# Plant a plausible mistake in a copy of the oracle and check a pin fails.

def _attend_variant(kind):
    def f(qp, kp, vp, cu, scale=None):
        T, H, d = qp.shape
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        if kind == "no_scale":
            scale = 1.0
        if kind == "scale_1_over_d":
            scale = 1.0 / d
        out = np.zeros_like(vp, dtype=np.float64)
        for b in range(len(cu) - 1):
            lo, hi = int(cu[b]), int(cu[b + 1])
            if kind == "bleed" and hi < T:
                hi_k = hi + 1
            else:
                hi_k = hi
            if hi <= lo:
                continue
            for h in range(H):
                q, k, v = qp[lo:hi, h], kp[lo:hi_k, h], vp[lo:hi_k, h]
                if kind == "v_is_k":
                    v = kp[lo:hi_k, h]
                s = q @ k.T * scale
                if kind == "neg":
                    s = -s
                if kind != "no_max":
                    s = s - s.max(axis=1, keepdims=True)
                p = np.exp(s)
                if kind == "wrong_axis":
                    p = p / p.sum(axis=0, keepdims=True)
                elif kind == "no_norm":
                    pass
                else:
                    p = p / p.sum(axis=1, keepdims=True)
                if kind == "transposed" and p.shape[0] == p.shape[1]:
                    p = p.T  # weights applied with query and key roles swapped
                out[lo:hi, h] = p @ v
        return out
    return f


MUTANTS = ["no_scale", "scale_1_over_d", "bleed", "v_is_k", "transposed", "neg", "no_max",
           "wrong_axis", "no_norm"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistake(kind):
    import warnings
    bad = _attend_variant(kind)
    caught = 0
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for pin in ATTEND_PINS:
            try:
                pin(bad)
            except (AssertionError, ValueError, FloatingPointError, IndexError):
                caught += 1
    assert caught >= 1, f"no pin caught mutant {kind}"


def test_unmutated_variant_passes_every_pin():
    good = _attend_variant("none")
    for pin in ATTEND_PINS:
        pin(good)


def test_pack_pins_catch_planted_mistakes():
    def desc_index(mask):
        B, N = mask.shape
        return np.concatenate([b * N + np.flatnonzero(mask[b])[::-1] for b in range(B)]).astype(np.int32)

    def local_index(mask):
        return np.concatenate([np.flatnonzero(mask[b]) for b in range(mask.shape[0])]).astype(np.int32)

    def inclusive_cu(mask):
        n = mask.sum(axis=1)
        return np.cumsum(np.concatenate([n, [0]])).astype(np.int32), int(n.max())

    for seqlens_fn, index_fn in [(R.seqlens, desc_index), (R.seqlens, local_index),
                                 (inclusive_cu, R.kept_index)]:
        with pytest.raises(AssertionError):
            check_pack(seqlens_fn, index_fn)
