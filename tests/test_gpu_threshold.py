"""Threshold-l2 keep-mask on the device against the oracle: the mask is
integer output decided by fp64 squared norms summed in channel order on both
sides, so it must match bit for bit."""
import sys

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import TOL, f64, max_err, to_dev, upload  # noqa: E402


def _rva():
    import ragged_variable_length_amd as rva
    rva.lib()
    return rva


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _x(seed, B, N, C, dtype, kind="normal"):
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "ties":  # small integers: many equal norms
        x = rng.integers(-2, 3, size=(B, N, C)).astype(np.float32)
    elif kind == "scaled":  # rows with very different magnitudes
        x = rng.standard_normal((B, N, C)).astype(np.float32)
        x *= np.float32(2.0) ** rng.integers(-20, 20, size=(B, N, 1)).astype(np.float32)
    else:
        x = rng.standard_normal((B, N, C)).astype(np.float32)
    return W._cast(x, dtype)


CASES = [
    # (seed, B, N, C, dtype, kind)
    (1, 4, 197, 384, "f32", "normal"),     # DeiT-S width, fp32
    (2, 3, 197, 768, "f16", "normal"),     # DeiT-B width
    (3, 3, 197, 192, "bf16", "normal"),    # DeiT-T width
    (4, 2, 577, 768, "f16", "normal"),     # 384x384 token count
    (5, 5, 65, 40, "f32", "normal"),       # partial last chunk (160-byte rows), 2 waves
    (6, 3, 64, 8, "f16", "normal"),        # one 16-byte piece per row
    (7, 4, 30, 16, "f32", "ties"),         # equal norms
    (8, 2, 1024, 64, "bf16", "normal"),    # largest N: 16 waves
    (9, 3, 100, 96, "f32", "scaled"),      # wide magnitude range
    (10, 2, 1, 64, "f16", "normal"),       # CLS only
    (11, 2, 2, 64, "f32", "normal"),       # one patch
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}_B{c[1]}_N{c[2]}_C{c[3]}_{c[4]}_{c[5]}")
def test_mask_matches_oracle(device, case):
    rva = _rva()
    seed, B, N, C, dtype, kind = case
    _say(f"[threshold] {case}")
    x = _x(seed, B, N, C, dtype, kind)
    xd = to_dev(x, dtype, device)
    for q in (0.0, 0.25, 0.5, 0.9, 1.0):
        got = rva.threshold_l2_mask(xd, q).cpu().numpy()
        ref = oracle.threshold_l2_mask(x, dtype, q)
        assert np.array_equal(got, ref), (q, np.argwhere(got != ref)[:5])


def test_mask_deit_s_input(device):
    """The DeiT-S recipe's embeddings (fp32) at keep-quantile 0.5: the device
    mask equals the oracle's and the recipe's own mask."""
    rva = _rva()
    w = W.deit_s_224_threshold_l2()
    x = w.meta["x"]
    got = rva.threshold_l2_mask(to_dev(x, "f32", device), 0.5).cpu().numpy()
    assert np.array_equal(got, oracle.threshold_l2_mask(x, "f32", 0.5))
    assert np.array_equal(got, w.mask)


def test_mask_full_size(device):
    """DeiT-B-width embeddings for 1024 images (the bench's keep-mask input):
    every image's mask against the oracle bit for bit, plus the closed-form
    kept count on all of them."""
    rva = _rva()
    x = W.embeddings()
    B, N, C = x.shape
    _say(f"[threshold] full size {x.shape}")
    got = rva.threshold_l2_mask(to_dev(x, "f16", device), 0.5).cpu().numpy()
    ref = oracle.threshold_l2_mask(x, "f16", 0.5)
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]
    # with distinct norms exactly P - r0 patches are kept in every image
    k = (N - 1) - oracle.keep_rank(N, 0.5)
    assert np.all(got[:, 0] == 1) and np.all(got[:, 1:].sum(axis=1) == k)


def test_mask_repeat_and_stream(device):
    """Identical results on repeated calls and on a side stream."""
    rva = _rva()
    x = to_dev(_x(21, 6, 197, 384, "f32"), "f32", device)
    a = rva.threshold_l2_mask(x, 0.4)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = rva.threshold_l2_mask(x, 0.4, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_l2_fused_plan(device):
    """Mask then fused attention, captured as one plan; replays follow new
    embeddings, with eager work between replays."""
    rva = _rva()
    w = W.deit_s_224_threshold_l2()
    q, k, v, _ = upload(w, device)
    B, N, H, d = q.shape
    mask = torch.empty((B, N), dtype=torch.uint8, device=device)
    out = torch.empty_like(q)
    cu = torch.empty(B + 1, dtype=torch.int32, device=device)
    x = to_dev(w.meta["x"], "f32", device)
    plan = rva.Plan(rva.L2_FUSED, q=q, k=k, v=v, mask=mask, out=out, cu_seqlens=cu, x=x,
                    keep_quantile=0.5)
    for rep in range(3):
        xs = w.meta["x"] if rep == 0 else _x(40 + rep, B, N, 384, "f32")
        x.copy_(torch.from_numpy(xs))
        plan.launch()
        torch.cuda.synchronize()
        rva.threshold_l2_mask(x, 0.3)  # eager work between replays
        torch.cuda.synchronize()
        m_ref = oracle.threshold_l2_mask(xs, "f32", 0.5)
        assert np.array_equal(mask.cpu().numpy(), m_ref), rep
        ref, cu_ref, _, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, m_ref, w.dtype)
        assert np.array_equal(cu.cpu().numpy(), cu_ref)
        o = f64(out)
        assert max_err(o, ref) <= TOL[w.dtype], rep
        assert np.all(o[m_ref == 0] == 0)
    plan.close()
