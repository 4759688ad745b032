"""QKV and output projections on the device against the fp64 oracle.  Every
element is checked against its own bound derived from the arithmetic
(gpu_util.linear_bound / check_linear)."""
import sys

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import TOL, check_linear, f64, linear_bound, max_err, to_dev  # noqa: E402

_bound = linear_bound
_check = check_linear


def _rva():
    import ragged_variable_length_amd as rva
    rva.lib()
    return rva


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _mask(seed, B, N, lo=0.0, hi=1.0, empty_image=False):
    rng = np.random.Generator(np.random.PCG64(seed))
    keep = rng.uniform(lo, hi, size=(B, 1))
    m = (rng.random((B, N)) < keep).astype(np.uint8)
    m[:, 0] = 1
    if empty_image:
        m[B // 2] = 0
    return m


def _weights(C, dtype, seed=5):
    return W.projection_weights(seed=seed, C=C, dtype=dtype)


def _dev_w(wts, dtype, device):
    return {k: to_dev(v, dtype, device) for k, v in wts.items()}


CASES = [
    # (seed, B, N, C, dtype)
    (1, 4, 197, 384, "f16"),
    (2, 3, 197, 768, "bf16"),
    (3, 5, 50, 64, "f16"),       # one head, K = 64 (single K stage)
    (4, 2, 577, 192, "bf16"),    # 384x384 token count, DeiT-T width
    (5, 7, 33, 320, "f16"),      # Nout = 960, C not a multiple of 128
    (6, 2, 197, 1024, "bf16"),   # ViT-L width: 16 K stages, Nout = 3072 (12 column tiles)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}_B{c[1]}_N{c[2]}_C{c[3]}_{c[4]}")
def test_qkv_gather(device, case):
    rva = _rva()
    seed, B, N, C, dtype = case
    _say(f"[qkv] {case}")
    x = W._cast(np.random.Generator(np.random.PCG64(seed)).standard_normal((B, N, C), dtype=np.float32), dtype)
    mask = _mask(seed + 100, B, N, empty_image=True)
    wts = _weights(C, dtype, seed)
    dw = _dev_w(wts, dtype, device)
    xd = to_dev(x, dtype, device)
    idx = rva.index(torch.from_numpy(mask).to(device))
    T = int(mask.sum())
    sentinel = -7.0
    outs = tuple(torch.full((B * N, C), sentinel, dtype=xd.dtype, device=device) for _ in range(3))
    q, k, v = rva.qkv_projection(xd, idx["cu_seqlens"], dw["w_qkv"], dw["b_qkv"],
                                 kept_index=idx["kept_index"], out=outs)
    torch.cuda.synchronize()
    ref = oracle.qkv_projection(x, mask, wts["w_qkv"], wts["b_qkv"], dtype)
    xs = oracle.pack_rows(oracle.decode(x, dtype), mask)
    wf, bf = oracle.decode(wts["w_qkv"], dtype), oracle.decode(wts["b_qkv"], dtype)
    for t, (got, r) in enumerate(zip((q, k, v), ref)):
        g = f64(got)
        mb = _bound(xs, wf[t * C:(t + 1) * C], bf[t * C:(t + 1) * C], None, dtype)
        _check(g[:T], r, mb, dtype, f"part {t}")
        assert np.all(g[T:] == sentinel), "rows past T written"


def test_qkv_packed_input_no_bias(device):
    rva = _rva()
    B, N, C, dtype = 3, 100, 256, "f16"
    rng = np.random.Generator(np.random.PCG64(9))
    mask = _mask(10, B, N)
    T = int(mask.sum())
    xp = W._cast(rng.standard_normal((B * N, C), dtype=np.float32), dtype)
    wts = _weights(C, dtype, 11)
    dw = _dev_w(wts, dtype, device)
    idx = rva.index(torch.from_numpy(mask).to(device))
    q, k, v = rva.qkv_projection(to_dev(xp, dtype, device), idx["cu_seqlens"], dw["w_qkv"], None,
                                 B=B, N=N)
    ref = oracle.qkv_projection(xp[:T], None, wts["w_qkv"], None, dtype)
    xs, wf = oracle.decode(xp[:T], dtype), oracle.decode(wts["w_qkv"], dtype)
    for t, (got, r) in enumerate(zip((q, k, v), ref)):
        _check(f64(got)[:T], r, _bound(xs, wf[t * C:(t + 1) * C], None, None, dtype), dtype, t)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}_B{c[1]}_N{c[2]}_C{c[3]}_{c[4]}")
def test_out_scatter_residual(device, case):
    rva = _rva()
    seed, B, N, C, dtype = case
    _say(f"[out] {case}")
    rng = np.random.Generator(np.random.PCG64(seed + 50))
    mask = _mask(seed + 200, B, N, empty_image=True)
    T = int(mask.sum())
    o = W._cast(rng.standard_normal((B * N, C), dtype=np.float32), dtype)  # capacity rows
    res = W._cast(rng.standard_normal((B, N, C), dtype=np.float32), dtype)
    wts = _weights(C, dtype, seed + 1)
    dw = _dev_w(wts, dtype, device)
    md = torch.from_numpy(mask).to(device)
    idx = rva.index(md)
    y = torch.full((B, N, C), 3.0, dtype=dw["w_o"].dtype, device=device)
    rva.out_projection(to_dev(o, dtype, device), idx["cu_seqlens"], dw["w_o"], dw["b_o"],
                       kept_index=idx["kept_index"], mask=md, residual=to_dev(res, dtype, device),
                       out=y)
    torch.cuda.synchronize()
    ref = oracle.out_projection(o[:T], mask, wts["w_o"], wts["b_o"], dtype, residual=res)
    g = f64(y)
    keep = mask != 0
    os_, wf, bf = (oracle.decode(a, dtype) for a in (o[:T], wts["w_o"], wts["b_o"]))
    mb = _bound(os_, wf, bf, oracle.pack_rows(oracle.decode(res, dtype), mask), dtype)
    _check(g[keep], ref[keep], mb, dtype, "kept rows")
    # pruned rows are +0 bit patterns
    bits = y.view(torch.int16).cpu().numpy()
    assert np.all(bits[~keep] == 0)


def test_out_packed_inplace_residual(device):
    """Packed output with the residual read from and written to the same buffer."""
    rva = _rva()
    B, N, C, dtype = 4, 120, 384, "bf16"
    rng = np.random.Generator(np.random.PCG64(12))
    mask = _mask(13, B, N)
    T = int(mask.sum())
    o = W._cast(rng.standard_normal((B * N, C), dtype=np.float32), dtype)
    res = W._cast(rng.standard_normal((B * N, C), dtype=np.float32), dtype)
    wts = _weights(C, dtype, 14)
    dw = _dev_w(wts, dtype, device)
    idx = rva.index(torch.from_numpy(mask).to(device))
    y = to_dev(res, dtype, device)
    rva.out_projection(to_dev(o, dtype, device), idx["cu_seqlens"], dw["w_o"], None, B=B, N=N,
                       residual=y, out=y)
    ref = oracle.out_projection(o[:T], None, wts["w_o"], None, dtype, residual=res[:T])
    os_, wf = oracle.decode(o[:T], dtype), oracle.decode(wts["w_o"], dtype)
    g = f64(y)
    _check(g[:T], ref, _bound(os_, wf, None, oracle.decode(res[:T], dtype), dtype), dtype, "packed")
    assert np.array_equal(y.view(torch.int16).cpu().numpy()[T:],
                          res.view(np.int16)[T:]), "rows past T touched"


def test_block_stagewise_full_size(device):
    """The attention block on the mixed 1024-image batch at DeiT-B width:
    offsets + kept index, QKV gather-product, ragged attention, output
    product with scatter.  Each stage is checked on every row of every image
    against the oracle applied to that stage's device inputs."""
    rva = _rva()
    w = W.mixed_peak()
    B, N, H = w.B, w.N, w.H
    C = H * 64
    _say(f"[block] B={B} N={N} C={C}")
    x = W.embeddings(B=B, N=N, C=C)
    wts = _weights(C, "f16", 21)
    dw = _dev_w(wts, "f16", device)
    md = torch.from_numpy(w.mask).to(device)
    xd = to_dev(x, "f16", device)
    idx = rva.index(md)
    q, k, v = rva.qkv_projection(xd, idx["cu_seqlens"], dw["w_qkv"], dw["b_qkv"],
                                 kept_index=idx["kept_index"])
    cu = idx["cu_seqlens"]
    o = torch.empty_like(q)
    rva.ragged_attend(q.view(-1, H, 64), k.view(-1, H, 64), v.view(-1, H, 64), cu, 197,
                      out=o.view(-1, H, 64))
    y = torch.empty((B, N, C), dtype=torch.float16, device=device)
    rva.out_projection(o, cu, dw["w_o"], dw["b_o"], kept_index=idx["kept_index"], mask=md, out=y)
    torch.cuda.synchronize()
    cu_h = cu.cpu().numpy()
    T = int(cu_h[-1])
    assert T == w.total_kept
    imgs = np.arange(B)
    qh, kh, vh, oh = (a.cpu().numpy()[:T] for a in (q, k, v, o))
    # stage 1: QKV rows of every image
    rows = np.concatenate([np.arange(cu_h[b], cu_h[b + 1]) for b in imgs])
    kept = oracle.kept_index(w.mask)
    xs = oracle.decode(x.reshape(B * N, C)[kept[rows]], "f16")
    wf, bf = oracle.decode(wts["w_qkv"], "f16"), oracle.decode(wts["b_qkv"], "f16")
    for t, part in enumerate((qh, kh, vh)):
        ref = oracle.linear(xs, wf[t * C:(t + 1) * C], bf[t * C:(t + 1) * C])
        got = part[rows].astype(np.float64)
        _check(got, ref, _bound(xs, wf[t * C:(t + 1) * C], bf[t * C:(t + 1) * C], None, "f16"),
               "f16", f"qkv {t}")
    # stage 2: attention of every image on the device's own q/k/v
    for b in imgs:
        lo, hi = int(cu_h[b]), int(cu_h[b + 1])
        sl = lambda a: oracle.decode(a[lo:hi].reshape(hi - lo, H, 64), "f16")
        ref = oracle.attend(sl(qh), sl(kh), sl(vh), np.array([0, hi - lo]))
        assert max_err(oh[lo:hi].reshape(hi - lo, H, 64).astype(np.float64), ref) <= TOL["f16"]
    # stage 3: output rows of every image on the device's own o
    os_ = oracle.decode(oh[rows], "f16")
    wo, bo = oracle.decode(wts["w_o"], "f16"), oracle.decode(wts["b_o"], "f16")
    ref = oracle.linear(os_, wo, bo)
    yh = y.cpu().numpy().reshape(B * N, C)
    _check(yh[kept[rows]].astype(np.float64), ref, _bound(os_, wo, bo, None, "f16"), "f16", "out")
    assert np.all(y.view(torch.int16).cpu().numpy()[w.mask == 0] == 0)
