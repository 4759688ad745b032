"""Multi-layer plan: one pack, L attention sub-layers on the packed residual
stream, one unpack, replayed as one graph.

Checks: the plan's output equals, bit for bit, the same sequence of direct
calls; and every stage of that sequence, layer by layer, matches the oracle
applied to the stage's own device inputs (projection bounds derived from the
arithmetic, attention tolerance as for the attention kernel)."""
import sys

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import TOL, check_linear, linear_bound, max_err, to_dev  # noqa: E402


def _rva():
    import ragged_variable_length_amd as rva
    rva.lib()
    return rva


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _mask(seed, B, N):
    rng = np.random.Generator(np.random.PCG64(seed))
    m = (rng.random((B, N)) < rng.uniform(0.2, 1.0, size=(B, 1))).astype(np.uint8)
    m[:, 0] = 1
    return m


def _layer_weights(L, C, dtype, device, seed=60):
    host = [W.projection_weights(seed=seed + l, C=C, dtype=dtype) for l in range(L)]
    dev = [{k: to_dev(v, dtype, device) for k, v in h.items()} for h in host]
    return host, dev


def _eager(rva, x, mask_d, wdev, H, record=None):
    """The plan's sequence as direct calls; optionally records every stage."""
    B, N, C = x.shape
    pk = rva.pack(x.view(B, N, H, 64), None, None, mask_d)
    cu = pk["cu_seqlens"]
    resid = pk["q"].view(B * N, C)
    for l, wd in enumerate(wdev):
        if record is not None:
            record.append({"in": resid.clone()})
        q, k, v = rva.qkv_projection(resid, cu, wd["w_qkv"], wd["b_qkv"], B=B, N=N)
        o = torch.empty_like(q)
        rva.ragged_attend(q.view(-1, H, 64), k.view(-1, H, 64), v.view(-1, H, 64), cu, N,
                          out=o.view(-1, H, 64))
        rva.out_projection(o, cu, wd["w_o"], wd["b_o"], B=B, N=N, residual=resid, out=resid)
        if record is not None:
            record[-1].update(q=q.clone(), k=k.clone(), v=v.clone(), o=o.clone(), out=resid.clone())
    return rva.unpack(resid.view(B * N, H, 64), cu, mask_d).view(B, N, C), cu


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_layers_plan_matches_stages(device, dtype):
    rva = _rva()
    B, N, H, L = 3, 50, 2, 3
    C = H * 64
    _say(f"[layers] {dtype} B={B} N={N} C={C} L={L}")
    rng = np.random.Generator(np.random.PCG64(61))
    x_h = W._cast(rng.standard_normal((B, N, C), dtype=np.float32), dtype)
    mask = _mask(62, B, N)
    x = to_dev(x_h, dtype, device)
    md = torch.from_numpy(mask).to(device)
    host, wdev = _layer_weights(L, C, dtype, device)
    plan = rva.LayersPlan(x, md, wdev, max_seqlen_hint=N)
    plan.launch()
    torch.cuda.synchronize()
    rec = []
    y_eager, cu = _eager(rva, x, md, wdev, H, record=rec)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(plan.out), _bits(y_eager)), "plan differs from direct calls"
    cu_h = cu.cpu().numpy()
    T = int(cu_h[-1])
    dec = lambda t: oracle.decode(t.cpu().numpy()[:T] if dtype == "f16" else
                                  t.view(torch.int16).cpu().numpy().view(np.uint16)[:T], dtype)
    for l, st in enumerate(rec):
        wf = oracle.decode(host[l]["w_qkv"], dtype)
        bf = oracle.decode(host[l]["b_qkv"], dtype)
        xin = dec(st["in"])
        for t, nm in enumerate("qkv"):
            ref = oracle.linear(xin, wf[t * C:(t + 1) * C], bf[t * C:(t + 1) * C])
            check_linear(dec(st[nm]), ref, linear_bound(xin, wf[t * C:(t + 1) * C],
                                                        bf[t * C:(t + 1) * C], None, dtype),
                         dtype, f"layer {l} {nm}")
        att = oracle.attend(dec(st["q"]).reshape(T, H, 64), dec(st["k"]).reshape(T, H, 64),
                            dec(st["v"]).reshape(T, H, 64), cu_h)
        assert max_err(dec(st["o"]).reshape(T, H, 64), att) <= TOL[dtype], f"layer {l} attention"
        wo, bo = oracle.decode(host[l]["w_o"], dtype), oracle.decode(host[l]["b_o"], dtype)
        ob = dec(st["o"])
        ref = oracle.linear(ob, wo, bo, xin)
        check_linear(dec(st["out"]), ref, linear_bound(ob, wo, bo, xin, dtype), dtype,
                     f"layer {l} out")
    # the unpacked output holds the last residual stream at kept positions, +0 elsewhere
    yb = _bits(plan.out)
    keep = mask != 0
    assert np.array_equal(yb[keep], _bits(rec[-1]["out"])[:T])
    assert np.all(yb[~keep] == 0)
    plan.close()


def test_layers_plan_replays_follow_inputs(device):
    """Replays after new embeddings and a new mask, with direct calls between."""
    rva = _rva()
    B, N, H, L = 4, 197, 6, 2
    C = H * 64
    x = torch.empty((B, N, C), dtype=torch.float16, device=device)
    md = torch.empty((B, N), dtype=torch.uint8, device=device)
    _, wdev = _layer_weights(L, C, "f16", device, seed=70)
    plan = rva.LayersPlan(x, md, wdev, max_seqlen_hint=N)
    for rep in range(3):
        rng = np.random.Generator(np.random.PCG64(80 + rep))
        x.copy_(torch.from_numpy(rng.standard_normal((B, N, C), dtype=np.float32).astype(np.float16)))
        md.copy_(torch.from_numpy(_mask(90 + rep, B, N)))
        plan.launch()
        torch.cuda.synchronize()
        y_eager, _ = _eager(rva, x, md, wdev, H)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(plan.out), _bits(y_eager)), rep
    plan.close()


def test_layers_plan_full_size(device):
    """The mixed 1024-image batch at DeiT-B width through two layers: the
    plan equals the direct calls bit for bit, and pruned rows are +0."""
    rva = _rva()
    w = W.mixed_peak()
    B, N, H = w.B, w.N, w.H
    C = H * 64
    _say(f"[layers] full size B={B}")
    x = to_dev(W.embeddings(B=B, N=N, C=C), "f16", device)
    md = torch.from_numpy(w.mask).to(device)
    _, wdev = _layer_weights(2, C, "f16", device, seed=100)
    plan = rva.LayersPlan(x, md, wdev, max_seqlen_hint=197)
    plan.launch()
    torch.cuda.synchronize()
    y_eager, cu = _eager(rva, x, md, wdev, H)
    torch.cuda.synchronize()
    assert int(cu[-1].item()) == w.total_kept
    yb = _bits(plan.out)
    assert np.array_equal(yb, _bits(y_eager))
    assert np.all(yb[w.mask == 0] == 0)
    assert np.isfinite(plan.out.float().cpu().numpy()).all()
    plan.close()
