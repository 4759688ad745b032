"""Captured launch plans (HIP graphs) and the full-size mixed batch in the
launch configuration the bench times."""
import sys

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import TOL, bits, f64, max_err, upload  # noqa: E402


def _rva():
    import ragged_variable_length_amd as rva
    rva.lib()
    return rva


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _fresh_mask(seed, B, N):
    rng = np.random.Generator(np.random.PCG64(seed))
    m = (rng.random((B, N)) < rng.uniform(0.1, 0.9, size=(B, 1))).astype(np.uint8)
    m[:, 0] = 1
    return m


@pytest.mark.parametrize("mode", ["fused", "staged", "fused_direct"])
def test_plan_replays_follow_mask_changes(device, mode):
    rva = _rva()
    w = W.deit_b_224(0.5)
    _say(f"[plan] {mode}")
    q, k, v, mask = upload(w, device)
    B, N, H, d = q.shape
    out = torch.empty_like(q)
    cu = torch.empty(B + 1, dtype=torch.int32, device=device)
    mx = torch.empty(1, dtype=torch.int32, device=device)
    kw = dict(q=q, k=k, v=v, mask=mask, out=out, cu_seqlens=cu, max_seqlen=mx)
    if mode == "staged":
        packed = {nm: torch.empty((B * N, H, d), dtype=q.dtype, device=device)
                  for nm in ("q", "k", "v", "o")}
        plan = rva.Plan(rva.STAGED, packed=packed, **kw)
    elif mode == "fused_direct":
        plan = rva.Plan(rva.FUSED_DIRECT, **kw)
    else:
        plan = rva.Plan(rva.FUSED, **kw)
    for rep in range(4):
        m = w.mask if rep == 0 else _fresh_mask(100 + rep, B, N)
        mask.copy_(torch.from_numpy(m))
        plan.launch()
        torch.cuda.synchronize()
        # eager work between replays
        eager = rva.fused(q, k, v, mask)
        torch.cuda.synchronize()
        ref, cu_ref, mx_ref, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, m, w.dtype)
        assert cu.cpu().numpy().tolist() == cu_ref.tolist()
        assert int(mx.item()) == mx_ref
        assert max_err(f64(out), ref) <= TOL[w.dtype]
        assert np.array_equal(bits(out), bits(eager))
        assert (bits(out)[m == 0] == 0).all()
    plan.close()


def test_empty_plan_and_empty_launches(device):
    rva = _rva()
    p = rva.Plan(rva.EMPTY)
    for _ in range(3):
        p.launch()
    rva.empty(5)
    torch.cuda.synchronize()
    p.close()


def test_mixed_full_size_sampled(device):
    """The 1024-image mixed batch through the captured fused launch (the bench's
    configuration): offsets exactly, attention on sampled (image, head) pairs,
    pruned rows zero everywhere."""
    rva = _rva()
    w = W.mixed_peak()
    _say(f"[mixed] B={w.B} T={w.total_kept}")
    q, k, v, mask = upload(w, device)
    B, N, H, d = q.shape
    out = torch.empty_like(q)
    cu = torch.empty(B + 1, dtype=torch.int32, device=device)
    mx = torch.empty(1, dtype=torch.int32, device=device)
    plan = rva.Plan(rva.FUSED, q=q, k=k, v=v, mask=mask, out=out, cu_seqlens=cu, max_seqlen=mx)
    plan.launch()
    plan.launch()
    torch.cuda.synchronize()
    cu_ref, mx_ref = oracle.seqlens(w.mask)
    assert cu.cpu().numpy().tolist() == cu_ref.tolist()
    assert int(mx.item()) == mx_ref
    ob = out.cpu()
    assert (bits(ob)[w.mask == 0] == 0).all()
    rng = np.random.Generator(np.random.PCG64(5))
    counts = w.counts
    picks = [(int(np.argmax(counts)), 0), (int(np.argmin(counts)), H - 1)]
    picks += [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 30), rng.integers(0, H, 30))]
    worst = 0.0
    for b, h in picks:
        keep, rows = oracle.attend_image_head(w.q, w.k, w.v, w.mask, w.dtype, b, h)
        got = ob[b, keep, h].float().numpy().astype(np.float64)
        worst = max(worst, max_err(got, rows))
    _say(f"   sampled max abs err {worst:.3e}")
    assert worst <= TOL[w.dtype]
    plan.close()


def test_direct_plan_on_callers_stream(device):
    """A direct-launch plan enqueues on the stream it is given (the current
    stream by default): work queued before it on a side stream is seen."""
    rva = _rva()
    w = W.deit_b_224(0.8)
    q, k, v, mask = upload(w, device)
    ref = rva.fused(q, k, v, mask)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    q2 = torch.empty_like(q)
    plan = rva.Plan(rva.FUSED_DIRECT, q=q2, k=k, v=v, mask=mask, out=out)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        q2.copy_(q)
        plan.launch()
    side.synchronize()
    assert np.array_equal(bits(out), bits(ref))
    plan.close()
