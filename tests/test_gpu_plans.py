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


def _mixed_dev(device):
    from gpu_util import mixed_full
    w = mixed_full()["w"]
    q, k, v, mask = upload(w, device)
    B = w.B
    return w, q, k, v, mask, (torch.empty_like(q), torch.empty(B + 1, dtype=torch.int32, device=device),
                              torch.empty(1, dtype=torch.int32, device=device))


@pytest.mark.parametrize("form", ["fused_graph", "fused_direct_plan", "fused_call"])
def test_mixed_full_size_fused(device, form):
    """The 1024-image mixed batch (12,288 image-head pairs) through the fused
    single launch, as the bench times it (direct call, direct-launch plan)
    and as a captured graph: offsets exactly, every kept element against the
    oracle, pruned rows +0."""
    from gpu_util import check_mixed_full
    rva = _rva()
    w, q, k, v, mask, (out, cu, mx) = _mixed_dev(device)
    _say(f"[mixed] {form} B={w.B} T={w.total_kept}")
    hint = int(w.counts.max())
    if form == "fused_call":
        for _ in range(2):
            rva.fused(q, k, v, mask, out=out, cu_seqlens=cu, max_seqlen=mx, max_seqlen_hint=hint)
    else:
        mode = rva.FUSED if form == "fused_graph" else rva.FUSED_DIRECT
        plan = rva.Plan(mode, q=q, k=k, v=v, mask=mask, out=out, cu_seqlens=cu, max_seqlen=mx,
                        max_seqlen_hint=hint)
        plan.launch()
        plan.launch()
        plan.close()
    torch.cuda.synchronize()
    err = check_mixed_full(out, form, cu, mx)
    _say(f"   max abs err over every element {err:.3e}")


@pytest.mark.parametrize("form", ["calls", "staged_graph"])
def test_mixed_full_size_staged(device, form):
    """The mixed batch through the separate pack -> ragged attention ->
    unpack launches (direct calls, and the staged graph): packed offsets and
    kept index exactly, every element of the padded output against the
    oracle."""
    from gpu_util import check_mixed_full
    rva = _rva()
    w, q, k, v, mask, (out, cu, mx) = _mixed_dev(device)
    B, N, H, d = q.shape
    _say(f"[mixed] staged {form}")
    if form == "calls":
        pk = rva.pack(q, k, v, mask)
        o = torch.empty_like(pk["q"])
        rva.ragged_attend(pk["q"], pk["k"], pk["v"], pk["cu_seqlens"], int(w.counts.max()), out=o)
        rva.unpack(o, pk["cu_seqlens"], mask, out=out)
        torch.cuda.synchronize()
        T = w.total_kept
        assert np.array_equal(pk["kept_index"][:T].cpu().numpy(), oracle.kept_index(w.mask))
        check_mixed_full(out, form, pk["cu_seqlens"], pk["max_seqlen"])
    else:
        packed = {nm: torch.empty((B * N, H, d), dtype=q.dtype, device=device) for nm in "qkvo"}
        plan = rva.Plan(rva.STAGED, q=q, k=k, v=v, mask=mask, out=out, packed=packed,
                        cu_seqlens=cu, max_seqlen=mx, max_seqlen_hint=N)
        plan.launch()
        torch.cuda.synchronize()
        check_mixed_full(out, form, cu, mx)
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
