"""The persistent form of the fused path: a resident grid that pulls the
one-launch kernel's items (head pairs, or single heads of tail images) from
a device counter and runs the same per-item code.  Checked: identical bits
to the one-launch fused kernel on every workload, the oracle on the
standard workloads and on every element of the full mixed batch, the work
counter back at zero after every call, and the persistent plan's replays."""
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


def _assert_same_bits(a, b):
    assert np.array_equal(bits(a), bits(b)), "differs from the one-launch fused kernel"


def _outs(q, device):
    B = q.shape[0]
    return (torch.empty_like(q), torch.empty(B + 1, dtype=torch.int32, device=device),
            torch.empty(1, dtype=torch.int32, device=device))


WORKLOADS = [("deit_s", lambda: W.deit_s_224_threshold_l2()),
             ("deit_b_p50", lambda: W.deit_b_224(0.5)),
             ("deit_b_p0", lambda: W.deit_b_224(0.0)),
             ("deit_b_384", lambda: W.deit_b_384()),
             ("tiny_counts", lambda: W.random_workload(seed=5, B=3, N=40, H=2, dtype="bf16",
                                                        counts=[40, 0, 1])),
             # fp32 inputs: the persistent entry point runs the one-launch kernel
             ("tiny_f32", lambda: W.tiny())]


@pytest.mark.parametrize("name,make", WORKLOADS, ids=[n for n, _ in WORKLOADS])
def test_persistent_equals_fused_and_oracle(device, name, make):
    rva = _rva()
    w = make()
    _say(f"[persistent] {name}")
    q, k, v, mask = upload(w, device)
    hint = int(w.counts.max()) if w.counts.max() > 0 else 1
    work = torch.zeros(2, dtype=torch.int32, device=device)
    o1, cu1, mx1 = _outs(q, device)
    o2, cu2, mx2 = _outs(q, device)
    # the one-launch reference with one workgroup per (image, head): small
    # launches would otherwise take the key-split form (another order of
    # summation), which the persistent form does not have
    rva.set_query_split(1)
    try:
        rva.fused(q, k, v, mask, out=o1, cu_seqlens=cu1, max_seqlen=mx1, max_seqlen_hint=hint)
    finally:
        rva.set_query_split(0)
    for _ in range(2):  # the second call checks the counter came back to zero
        o2.fill_(7.0)
        rva.fused_persistent(q, k, v, mask, work, out=o2, cu_seqlens=cu2, max_seqlen=mx2,
                             max_seqlen_hint=hint)
        torch.cuda.synchronize()
        _assert_same_bits(o2, o1)
        assert np.array_equal(cu2.cpu().numpy(), cu1.cpu().numpy())
        assert int(mx2.item()) == int(mx1.item())
        assert work.cpu().tolist() == [0, 0]
    ref, cu_ref, mx_ref, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype)
    assert np.array_equal(cu2.cpu().numpy(), cu_ref)
    assert max_err(f64(o2), ref) <= TOL[w.dtype]


def test_persistent_fewer_items_than_workgroups(device):
    """Two images of one head: most resident workgroups find no item."""
    rva = _rva()
    w = W.random_workload(seed=9, B=2, N=197, H=1, dtype="f16", counts=[197, 60])
    q, k, v, mask = upload(w, device)
    work = torch.zeros(2, dtype=torch.int32, device=device)
    o = rva.fused_persistent(q, k, v, mask, work, max_seqlen_hint=197)
    torch.cuda.synchronize()
    ref, _, _, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype)
    assert max_err(f64(o), ref) <= TOL[w.dtype]
    assert work.cpu().tolist() == [0, 0]


def test_persistent_plan_replays(device):
    rva = _rva()
    w = W.deit_b_224(0.5)
    q, k, v, mask = upload(w, device)
    B, N, H, d = q.shape
    out, cu, mx = _outs(q, device)
    plan = rva.Plan(rva.PERSISTENT, q=q, k=k, v=v, mask=mask, out=out, cu_seqlens=cu,
                    max_seqlen=mx, max_seqlen_hint=N)
    rng = np.random.Generator(np.random.PCG64(44))
    for rep in range(4):
        m = w.mask if rep == 0 else (rng.random((B, N)) < rng.uniform(0.1, 0.9)).astype(np.uint8)
        mask.copy_(torch.from_numpy(m))
        plan.launch()
        torch.cuda.synchronize()
        ref_o = rva.fused(q, k, v, mask, max_seqlen_hint=N)  # eager work between replays
        torch.cuda.synchronize()
        _assert_same_bits(out, ref_o)
        ref, cu_ref, _, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, m, w.dtype)
        assert np.array_equal(cu.cpu().numpy(), cu_ref)
        assert max_err(f64(out), ref) <= TOL[w.dtype]
    plan.close()


def test_persistent_full_size(device):
    """The mixed 1024-image batch: bits equal to the one-launch fused kernel
    on repeated calls, and every element against the oracle."""
    from gpu_util import check_mixed_full, mixed_full
    rva = _rva()
    w = mixed_full()["w"]
    q, k, v, mask = upload(w, device)
    work = torch.zeros(2, dtype=torch.int32, device=device)
    o1, cu1, mx1 = _outs(q, device)
    o2, cu2, mx2 = _outs(q, device)
    rva.fused(q, k, v, mask, out=o1, cu_seqlens=cu1, max_seqlen=mx1, max_seqlen_hint=197)
    for _ in range(3):
        rva.fused_persistent(q, k, v, mask, work, out=o2, cu_seqlens=cu2, max_seqlen=mx2,
                             max_seqlen_hint=197)
    torch.cuda.synchronize()
    _assert_same_bits(o2, o1)
    assert work.cpu().tolist() == [0, 0]
    err = check_mixed_full(o2, "persistent", cu2, mx2)
    _say(f"[persistent] full size, max abs err over every element {err:.3e}")


def test_persistent_every_length(device):
    """Every kept count from 0 to 224, four images each (900 images, 3 heads:
    head pairs, single-head tail items, images with no kept token, and the
    chunked form past 208 rows, where the next item's index is handed over
    from inside the chunk loop).  Bits equal to the one-launch kernel, the
    oracle on every row, and the counter back at zero."""
    rva = _rva()
    N, H = 224, 3
    counts = [n for n in range(N + 1) for _ in range(4)]
    w = W.random_workload(35, B=len(counts), N=N, H=H, dtype="bf16", counts=counts,
                          name="persistent_every_length")
    _say(f"[persistent] every length B={w.B} N={N} H={H}")
    q, k, v, mask = upload(w, device)
    work = torch.zeros(2, dtype=torch.int32, device=device)
    o1, cu1, mx1 = _outs(q, device)
    o2, cu2, mx2 = _outs(q, device)
    rva.fused(q, k, v, mask, out=o1, cu_seqlens=cu1, max_seqlen=mx1, max_seqlen_hint=N)
    for _ in range(2):
        o2.fill_(7.0)
        rva.fused_persistent(q, k, v, mask, work, out=o2, cu_seqlens=cu2, max_seqlen=mx2,
                             max_seqlen_hint=N)
        torch.cuda.synchronize()
        _assert_same_bits(o2, o1)
        assert np.array_equal(cu2.cpu().numpy(), cu1.cpu().numpy())
        assert work.cpu().tolist() == [0, 0]
    ref, cu_ref, mx_ref, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype)
    assert np.array_equal(cu2.cpu().numpy(), cu_ref)
    assert int(mx2.item()) == int(mx_ref)
    assert max_err(f64(o2), ref) <= TOL[w.dtype]
