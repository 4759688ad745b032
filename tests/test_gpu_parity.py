"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bit-exact: cu_seqlens, max_seqlen, kept_index, packed q/k/v bits, unpacked
bits (pruned rows are +0).  Attention: max abs error within 2e-3 (fp16),
1e-2 (bf16), 1e-4 (fp32) over kept positions.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import TOL, bits, f64, host_bits, max_err, upload  # noqa: E402


def _rva():
    import ragged_variable_length_amd as rva
    rva.lib()
    return rva


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


SMALL_CONFIGS = ["tiny", "deit_s_224", "deit_b_224_p0", "deit_b_224_p20", "deit_b_224_p50",
                 "deit_b_224_p80", "deit_b_384"]

_CACHE = {}


def _workload(name):
    if name not in _CACHE:
        _CACHE[name] = W.CONFIG_BUILDERS[name]()
    return _CACHE[name]


def _edge_workloads():
    out = []
    # images keeping nothing, one token, everything; ragged tails around tile edges
    out.append(W.random_workload(11, B=5, N=197, H=3, dtype="f16", counts=[0, 1, 197, 33, 64],
                                 name="edge_f16"))
    out.append(W.random_workload(12, B=4, N=70, H=2, dtype="bf16", counts=[16, 17, 31, 0],
                                 name="edge_bf16"))
    out.append(W.random_workload(13, B=3, N=40, H=1, dtype="f32", counts=[1, 40, 15],
                                 name="edge_f32"))
    out.append(W.random_workload(14, B=2, N=1, H=4, dtype="f16", counts=[1, 0], name="n1"))
    # long sequences: several query passes and (with the default bound) two staged chunks
    out.append(W.random_workload(15, B=2, N=600, H=2, dtype="f16", counts=[577, 300],
                                 name="long_f16"))
    out.append(W.random_workload(16, B=2, N=300, H=2, dtype="f32", counts=[300, 129],
                                 name="long_f32"))
    out.append(W.random_workload(17, B=1, N=1024, H=1, dtype="bf16", counts=[1024],
                                 name="max_tokens_bf16"))
    out.append(W.random_workload(18, B=3, N=64, H=2, dtype="f16", keep_prob=0.0, name="all_pruned"))
    return out


EDGE = None


def _edges():
    global EDGE
    if EDGE is None:
        EDGE = {w.name: w for w in _edge_workloads()}
    return EDGE


ALL_NAMES = SMALL_CONFIGS + ["edge_f16", "edge_bf16", "edge_f32", "n1", "long_f16", "long_f32",
                             "max_tokens_bf16", "all_pruned"]


def _get(name):
    return _workload(name) if name in W.CONFIG_BUILDERS else _edges()[name]


@pytest.mark.parametrize("name", ALL_NAMES)
def test_pack_bit_exact(device, name):
    rva = _rva()
    w = _get(name)
    _say(f"[pack] {name} B={w.B} N={w.N} H={w.H} {w.dtype}")
    q, k, v, mask = upload(w, device)
    out = rva.pack(q, k, v, mask)
    torch.cuda.synchronize()
    cu_ref, mx_ref = oracle.seqlens(w.mask)
    idx_ref = oracle.kept_index(w.mask)
    T = int(cu_ref[-1])
    assert out["cu_seqlens"].cpu().numpy().tolist() == cu_ref.tolist()
    assert int(out["max_seqlen"].item()) == mx_ref
    assert out["kept_index"][:T].cpu().numpy().tolist() == idx_ref.tolist()
    for nm, x in (("q", w.q), ("k", w.k), ("v", w.v)):
        ref = host_bits(oracle.pack_rows(x, w.mask))
        assert np.array_equal(bits(out[nm][:T]), ref), nm


@pytest.mark.parametrize("name", ALL_NAMES)
def test_unpack_bit_exact(device, name):
    rva = _rva()
    w = _get(name)
    _say(f"[unpack] {name}")
    cu_ref, _ = oracle.seqlens(w.mask)
    T = int(cu_ref[-1])
    # packed rows: reuse the generator's v values (any bits will do)
    packed = oracle.pack_rows(w.v, w.mask)
    from gpu_util import to_dev
    o_pk = to_dev(packed if T else np.zeros((1, w.H, w.d), dtype=w.v.dtype), w.dtype, device)
    cu = torch.from_numpy(cu_ref).to(device)
    mask = torch.from_numpy(w.mask).to(device)
    o_pad = torch.full((w.B, w.N, w.H, w.d), float("nan"), device=device).to(o_pk.dtype)
    rva.unpack(o_pk, cu, mask, out=o_pad)
    torch.cuda.synchronize()
    ref = oracle.unpack(packed, w.mask) if T else np.zeros((w.B, w.N, w.H, w.d), dtype=w.v.dtype)
    assert np.array_equal(bits(o_pad), host_bits(ref))


@pytest.mark.parametrize("name", ALL_NAMES)
def test_ragged_attend_parity(device, name):
    rva = _rva()
    w = _get(name)
    _say(f"[attend] {name}")
    q, k, v, mask = upload(w, device)
    pk = rva.pack(q, k, v, mask)
    cu_ref, mx = oracle.seqlens(w.mask)
    T = int(cu_ref[-1])
    o = torch.zeros_like(pk["q"])
    rva.ragged_attend(pk["q"], pk["k"], pk["v"], pk["cu_seqlens"], max(mx, 1), out=o)
    torch.cuda.synchronize()
    qp, kp, vp = (oracle.decode(oracle.pack_rows(x, w.mask), w.dtype) for x in (w.q, w.k, w.v))
    ref = oracle.attend(qp, kp, vp, cu_ref)
    err = max_err(f64(o[:T]), ref)
    _say(f"   max abs err {err:.3e}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("name", ALL_NAMES)
def test_fused_parity(device, name):
    rva = _rva()
    w = _get(name)
    _say(f"[fused] {name}")
    q, k, v, mask = upload(w, device)
    cu = torch.full((w.B + 1,), -7, dtype=torch.int32, device=device)
    mx = torch.full((1,), -7, dtype=torch.int32, device=device)
    o = torch.full_like(q, float("nan"))
    rva.fused(q, k, v, mask, out=o, cu_seqlens=cu, max_seqlen=mx)
    torch.cuda.synchronize()
    ref, cu_ref, mx_ref, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype)
    assert cu.cpu().numpy().tolist() == cu_ref.tolist()
    assert int(mx.item()) == mx_ref
    got = f64(o)
    err = max_err(got, ref)
    _say(f"   max abs err {err:.3e}")
    assert err <= TOL[w.dtype]
    # pruned rows are exactly +0
    pr = bits(o)[w.mask == 0]
    assert (pr == 0).all()


@pytest.mark.parametrize("name", ["deit_b_224_p50", "long_f16", "long_f32", "edge_bf16"])
@pytest.mark.parametrize("hint", [1, 40, 100])
def test_chunked_staging(device, name, hint):
    """A small max_seqlen bound forces several staged key chunks; results must
    not depend on it."""
    rva = _rva()
    w = _get(name)
    _say(f"[chunked] {name} hint={hint}")
    q, k, v, mask = upload(w, device)
    o = rva.fused(q, k, v, mask, max_seqlen_hint=hint)
    pk = rva.pack(q, k, v, mask)
    o2 = rva.ragged_attend(pk["q"], pk["k"], pk["v"], pk["cu_seqlens"], hint)
    torch.cuda.synchronize()
    ref, cu_ref, _, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype)
    assert max_err(f64(o), ref) <= TOL[w.dtype]
    T = int(cu_ref[-1])
    ref_pk = ref.reshape(-1, w.H, w.d)[oracle.kept_index(w.mask)]
    assert max_err(f64(o2[:T]), ref_pk) <= TOL[w.dtype]


RESIDENT_EDGES = [1, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64, 65, 95, 96, 97, 103, 104, 105, 112,
                  127, 128, 129, 160, 176, 191, 192, 193, 200, 207, 208, 209, 223, 224, 0]


SPLITS = [0, 1, 2, 3, 16]  # 0: the launch chooses; k: k query tiles per (sequence, head)


class _split:
    """Force rva_set_query_split(k) inside the block, back to 0 after."""

    def __init__(self, k):
        self.k = k

    def __enter__(self):
        _rva().set_query_split(self.k)

    def __exit__(self, *exc):
        _rva().set_query_split(0)


@pytest.mark.parametrize("split", SPLITS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_resident_boundaries(device, dtype, split):
    """Kept counts on every 16- and 32-row boundary up to the padded length,
    in a batch large enough that the fused form pairs heads (5 heads, so the
    last group has one): sequences staged whole one or two heads at a time,
    with a fourth query block per wave, and past the whole-sequence capacity
    in chunks.  Fused and packed forms against the oracle, every row."""
    rva = _rva()
    B, N, H = 512, 224, 5
    counts = [RESIDENT_EDGES[b % len(RESIDENT_EDGES)] for b in range(B)]
    w = W.random_workload(31 if dtype == "f16" else 32, B=B, N=N, H=H, dtype=dtype,
                          counts=counts, name=f"resident_{dtype}")
    _say(f"[resident] {dtype} B={B} N={N} H={H} split={split}")
    q, k, v, mask = upload(w, device)
    o = torch.full_like(q, float("nan"))
    pk = rva.pack(q, k, v, mask)
    o2 = torch.full_like(pk["q"], float("nan"))
    with _split(split):
        rva.fused(q, k, v, mask, out=o)
        rva.ragged_attend(pk["q"], pk["k"], pk["v"], pk["cu_seqlens"], N, out=o2)
    torch.cuda.synchronize()
    ref, cu_ref, _, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype)
    err = max_err(f64(o), ref)
    _say(f"   fused max abs err {err:.3e}")
    assert err <= TOL[w.dtype]
    assert (bits(o)[w.mask == 0] == 0).all()
    T = int(cu_ref[-1])
    ref_pk = ref.reshape(-1, H, w.d)[oracle.kept_index(w.mask)]
    assert max_err(f64(o2[:T]), ref_pk) <= TOL[w.dtype]


@pytest.mark.parametrize("split", SPLITS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_every_length(device, dtype, split):
    """Every kept count from 0 to 224, four images each (900 images, 3
    heads, so the fused form pairs heads and ends on single-head
    workgroups): every exit of the whole-sequence tile loop, every ragged
    tail, and the chunked form past 208 rows.  Fused and packed forms
    against the oracle, every row."""
    rva = _rva()
    N, H = 224, 3
    counts = [n for n in range(N + 1) for _ in range(4)]
    B = len(counts)
    w = W.random_workload(33 if dtype == "f16" else 34, B=B, N=N, H=H, dtype=dtype,
                          counts=counts, name=f"every_length_{dtype}")
    _say(f"[every length] {dtype} B={B} N={N} H={H} split={split}")
    q, k, v, mask = upload(w, device)
    o = torch.full_like(q, float("nan"))
    pk = rva.pack(q, k, v, mask)
    o2 = torch.full_like(pk["q"], float("nan"))
    with _split(split):
        rva.fused(q, k, v, mask, out=o, max_seqlen_hint=N)
        rva.ragged_attend(pk["q"], pk["k"], pk["v"], pk["cu_seqlens"], N, out=o2)
    torch.cuda.synchronize()
    ref, cu_ref, _, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype)
    err = max_err(f64(o), ref)
    _say(f"   fused max abs err {err:.3e}")
    assert err <= TOL[w.dtype]
    assert (bits(o)[w.mask == 0] == 0).all()
    T = int(cu_ref[-1])
    ref_pk = ref.reshape(-1, H, w.d)[oracle.kept_index(w.mask)]
    assert max_err(f64(o2[:T]), ref_pk) <= TOL[w.dtype]


def test_explicit_scale(device):
    rva = _rva()
    w = _get("deit_b_224_p80")
    q, k, v, mask = upload(w, device)
    o = rva.fused(q, k, v, mask, scale=0.05)
    torch.cuda.synchronize()
    ref, _, _, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype, scale=0.05)
    assert max_err(f64(o), ref) <= TOL[w.dtype]


def test_staged_equals_fused_and_unpack_of_packed(device):
    """unpack(attend(pack(x))) and the fused kernel agree bit for bit (same
    arithmetic in the same order)."""
    rva = _rva()
    w = _get("deit_b_224_p50")
    q, k, v, mask = upload(w, device)
    pk = rva.pack(q, k, v, mask)
    o_pk = rva.ragged_attend(pk["q"], pk["k"], pk["v"], pk["cu_seqlens"], w.N)
    o_st = rva.unpack(o_pk, pk["cu_seqlens"], mask)
    o_fu = rva.fused(q, k, v, mask)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o_st), bits(o_fu))


def test_deterministic(device):
    rva = _rva()
    w = _get("deit_b_224_p20")
    q, k, v, mask = upload(w, device)
    a = rva.fused(q, k, v, mask)
    b = rva.fused(q, k, v, mask)
    torch.cuda.synchronize()
    assert np.array_equal(bits(a), bits(b))


LATE_KEY_SHAPES = {"resident": (197, [197, 150, 100, 70, 40, 33]),
                   "streamed": (600, [577, 300, 209])}


@pytest.mark.parametrize("shape", sorted(LATE_KEY_SHAPES))
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_late_dominant_key(device, dtype, shape):
    """Scores in a later key tile far above every score of the first tile
    (queries aligned with one late key and scaled up): the fixed reference
    max from the first tile is exceeded by much more than its headroom, so
    those query blocks are computed again exactly (against their exact max
    in the whole-sequence form; with a running max from memory in the
    streamed form, sequences longer than the staging).  Fused and packed
    forms against the oracle."""
    rva = _rva()
    N, counts = LATE_KEY_SHAPES[shape]
    B, H = len(counts), 2
    w = W.random_workload((41 if dtype == "f16" else 42) + (10 if shape == "streamed" else 0), B=B,
                          N=N, H=H, dtype=dtype, counts=counts, name=f"late_key_{dtype}_{shape}")
    q = oracle.decode(w.q, dtype)
    k = oracle.decode(w.k, dtype)
    for b in range(B):
        keep = np.flatnonzero(w.mask[b])
        late = keep[-1]  # the last kept key lies in the sequence's last tile
        for h in range(H):
            kv = k[b, late, h]
            # every query of the image points at that key, 3x its length
            q[b, :, h] = 3.0 * kv / np.linalg.norm(kv) * 8.0
    w.q = W._cast(q.astype(np.float32), dtype)
    qd, kd, vd, md = upload(w, device)
    o = rva.fused(qd, kd, vd, md)
    pk = rva.pack(qd, kd, vd, md)
    o2 = rva.ragged_attend(pk["q"], pk["k"], pk["v"], pk["cu_seqlens"], N)
    torch.cuda.synchronize()
    ref, cu_ref, _, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype)
    assert np.isfinite(f64(o)).all()
    err = max_err(f64(o), ref)
    _say(f"[late key] {dtype} {shape} max abs err {err:.3e}")
    assert err <= TOL[w.dtype]
    T = int(cu_ref[-1])
    ref_pk = ref.reshape(-1, H, w.d)[oracle.kept_index(w.mask)]
    assert max_err(f64(o2[:T]), ref_pk) <= TOL[w.dtype]


def test_runs_on_the_callers_stream(device):
    """The launch goes to the current stream (a side stream entered with
    torch.cuda.stream) or to an explicit stream argument: work queued on
    that stream before the call (a fill of the inputs) is seen, and the
    default stream need not be synchronised."""
    rva = _rva()
    w = _get("deit_b_224_p50")
    q, k, v, mask = upload(w, device)
    ref = rva.fused(q, k, v, mask)
    torch.cuda.synchronize()
    for explicit in (False, True):
        side = torch.cuda.Stream()
        q2, k2, v2 = (torch.empty_like(t) for t in (q, k, v))
        o = torch.full_like(q, float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            # inputs written on the side stream just before the call
            q2.copy_(q)
            k2.copy_(k)
            v2.copy_(v)
            if explicit:
                rva.fused(q2, k2, v2, mask, out=o, stream=side)
        if not explicit:
            with torch.cuda.stream(side):
                rva.fused(q2, k2, v2, mask, out=o)
        side.synchronize()
        assert np.array_equal(bits(o), bits(ref)), explicit


def test_independent_images(device):
    """Perturbing one image leaves every other image's output bitwise equal."""
    rva = _rva()
    w = _get("deit_b_224_p50")
    q, k, v, mask = upload(w, device)
    a = rva.fused(q, k, v, mask)
    q2, v2 = q.clone(), v.clone()
    q2[5] = q2[5] * 2 + 1
    v2[5] = -v2[5]
    b = rva.fused(q2, k, v2, mask)
    torch.cuda.synchronize()
    ba, bb = bits(a), bits(b)
    keep = np.ones(w.B, dtype=bool)
    keep[5] = False
    assert np.array_equal(ba[keep], bb[keep])
    assert not np.array_equal(ba[5], bb[5])


def test_q_zero_gives_mean_of_kept_v(device):
    rva = _rva()
    w = W.random_workload(21, B=4, N=197, H=2, dtype="f16", counts=[197, 50, 7, 1])
    q, k, v, mask = upload(w, device)
    q.zero_()
    o = rva.fused(q, k, v, mask)
    torch.cuda.synchronize()
    got = f64(o)
    vv = oracle.decode(w.v, "f16")
    for b in range(w.B):
        keep = np.flatnonzero(w.mask[b])
        mean = vv[b, keep].mean(axis=0)
        assert np.abs(got[b, keep] - mean[None]).max() <= 2e-3


def test_guard_bands(device):
    """Writes stay inside their buffers: poisoned margins around every output
    are unchanged, and packed rows beyond T keep their poison."""
    rva = _rva()
    w = _get("edge_f16")
    q, k, v, mask = upload(w, device)
    B, N, H, d = q.shape
    G = 4096
    cu_ref, _ = oracle.seqlens(w.mask)
    T = int(cu_ref[-1])

    def guarded(n_elem, dtype):
        buf = torch.full((n_elem + 2 * G,), 12345, dtype=torch.int16, device=device)
        return buf, buf[G:G + n_elem].view(dtype)

    ob, o = guarded(B * N * H * d, torch.float16)
    rva.fused(q, k, v, mask, out=o.view(B, N, H, d))
    pbufs = {}
    outs = {}
    for nm in ("q", "k", "v"):
        pbufs[nm], outs[nm] = guarded(B * N * H * d, torch.float16)
        outs[nm] = outs[nm].view(B * N, H, d)
    rva.pack(q, k, v, mask, outputs=dict(outs))
    torch.cuda.synchronize()
    for buf in [ob] + list(pbufs.values()):
        h = buf.cpu().numpy()
        assert (h[:G] == 12345).all() and (h[-G:] == 12345).all()
    for nm in ("q", "k", "v"):
        tail = pbufs[nm][G + T * H * d:G + B * N * H * d].cpu().numpy()
        assert (tail == 12345).all()


@pytest.mark.parametrize("B,N", [(10007, 7), (9001, 20)])
def test_many_images(device, B, N):
    """More images than one scan segment (4096) of the offsets workgroup:
    byte-wise counting (N < 16) and 16-byte chunks straddling image
    boundaries with a partial final chunk (N = 20, B*N not a multiple of
    16); a grid of B*H workgroups.  Offsets and largest count bit-exact
    through rva_pack and rva_fused; every row against the oracle."""
    rva = _rva()
    H = 2
    w = W.random_workload(36 + N, B=B, N=N, H=H, dtype="f16", keep_prob=0.5,
                          name=f"many_images_{B}x{N}")
    _say(f"[many images] B={B} N={N} H={H}")
    q, k, v, mask = upload(w, device)
    cu = torch.empty(B + 1, dtype=torch.int32, device=device)
    mx = torch.empty(1, dtype=torch.int32, device=device)
    o = rva.fused(q, k, v, mask, cu_seqlens=cu, max_seqlen=mx)
    pk = rva.pack(q, k, v, mask)
    torch.cuda.synchronize()
    ref, cu_ref, mx_ref, idx_ref = oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype)
    assert np.array_equal(cu.cpu().numpy(), cu_ref)
    assert int(mx.item()) == int(mx_ref)
    assert np.array_equal(pk["cu_seqlens"].cpu().numpy(), cu_ref)
    assert int(pk["max_seqlen"].item()) == int(mx_ref)
    assert max_err(f64(o), ref) <= TOL["f16"]
    assert not bits(o)[w.mask == 0].any()


@pytest.mark.parametrize("name", ["tiny", "long_f32", "edge_f32", "deit_s_224", "deit_b_384",
                                  "deit_b_224_p50", "edge_f16", "edge_bf16"])
def test_split_forms_agree(device, name):
    """The query-tile split only changes which workgroup computes a query
    block: for fp32 and for 16-bit sequences staged whole, the fused and
    packed outputs are identical bit for bit under every forced split, and
    each matches the oracle."""
    rva = _rva()
    w = _get(name)
    q, k, v, mask = upload(w, device)
    pk = rva.pack(q, k, v, mask)
    ref, cu_ref, _, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype)
    T = int(cu_ref[-1])
    ref_pk = ref.reshape(-1, w.H, w.d)[oracle.kept_index(w.mask)]
    hint = max(int(w.counts.max()), 1)
    first = None
    # split 0 lets the launch choose, which for small 16-bit launches may be
    # the key-split form (another order of summation): checked against the
    # oracle only; every forced split must give the same bits
    for split in [0, 1, 2, 3, 5, 64]:
        _say(f"[split] {name} split={split}")
        with _split(split):
            o = rva.fused(q, k, v, mask, max_seqlen_hint=hint)
            o2 = rva.ragged_attend(pk["q"], pk["k"], pk["v"], pk["cu_seqlens"], hint)
        torch.cuda.synchronize()
        assert max_err(f64(o), ref) <= TOL[w.dtype]
        assert max_err(f64(o2[:T]), ref_pk) <= TOL[w.dtype]
        if split == 0:
            continue
        got = (bits(o), bits(o2[:T]))
        if first is None:
            first = got
        assert np.array_equal(got[0], first[0]) and np.array_equal(got[1], first[1]), split


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_key_split_every_length(device, dtype):
    """Small 16-bit launches whose one-block-per-workgroup grid fits one
    slot-fill take the key-split form (a block's key tiles split over the
    four waves, partial results combined through LDS): every kept count from
    0 to 208 (16 images of 3 heads per launch, 14 launches), fused and packed
    forms against the oracle, every row."""
    rva = _rva()
    N, H, per = 208, 3, 16
    counts = list(range(0, N + 1))
    counts += [N] * (-len(counts) % per)
    for i in range(0, len(counts), per):
        cs = counts[i:i + per]
        w = W.random_workload((61 if dtype == "f16" else 62) + i, B=per, N=N, H=H, dtype=dtype,
                              counts=cs, name=f"key_split_{dtype}_{i}")
        _say(f"[key split] {dtype} counts {cs[0]}..{cs[-1]}")
        q, k, v, mask = upload(w, device)
        o = torch.full_like(q, float("nan"))
        rva.fused(q, k, v, mask, out=o)
        pk = rva.pack(q, k, v, mask)
        o2 = torch.full_like(pk["q"], float("nan"))
        rva.ragged_attend(pk["q"], pk["k"], pk["v"], pk["cu_seqlens"], N, out=o2)
        torch.cuda.synchronize()
        ref, cu_ref, _, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype)
        assert max_err(f64(o), ref) <= TOL[w.dtype], i
        assert (bits(o)[w.mask == 0] == 0).all(), i
        T = int(cu_ref[-1])
        ref_pk = ref.reshape(-1, H, w.d)[oracle.kept_index(w.mask)]
        assert max_err(f64(o2[:T]), ref_pk) <= TOL[w.dtype], i


def test_split_setting_rejects_negative(device):
    rva = _rva()
    with pytest.raises(rva.RVAError):
        rva.set_query_split(-1)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_vit_l_mixed_batch(device, dtype):
    """A ViT-L/14 shape (257 tokens, 16 heads) with per-image pruning rates
    uniform in [0, 0.9], 256 images: head pairs, sequences staged whole and
    (past the whole-sequence capacity) in chunks within one launch.  Fused
    and packed forms against the oracle, every row."""
    rva = _rva()
    B, N, H = 256, 257, 16
    rng = np.random.Generator(np.random.PCG64(71 if dtype == "f16" else 72))
    p = rng.uniform(0.0, 0.9, size=B)
    counts = np.clip(np.rint((1.0 - p) * N), 1, N).astype(int).tolist()
    w = W.random_workload(73 if dtype == "f16" else 74, B=B, N=N, H=H, dtype=dtype, counts=counts,
                          name=f"vit_l_{dtype}")
    _say(f"[vit-l] {dtype} B={B} N={N} H={H}")
    q, k, v, mask = upload(w, device)
    o = torch.full_like(q, float("nan"))
    pk = rva.pack(q, k, v, mask)
    o2 = torch.full_like(pk["q"], float("nan"))
    rva.fused(q, k, v, mask, out=o, max_seqlen_hint=max(counts))
    rva.ragged_attend(pk["q"], pk["k"], pk["v"], pk["cu_seqlens"], max(counts), out=o2)
    torch.cuda.synchronize()
    ref, cu_ref, _, _ = oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype)
    err = max_err(f64(o), ref)
    _say(f"   fused max abs err {err:.3e}")
    assert err <= TOL[w.dtype]
    assert (bits(o)[w.mask == 0] == 0).all()
    T = int(cu_ref[-1])
    ref_pk = ref.reshape(-1, H, w.d)[oracle.kept_index(w.mask)]
    assert max_err(f64(o2[:T]), ref_pk) <= TOL[w.dtype]
