"""The Python binding checks every tensor argument before a pointer reaches
the library: device tensors on the current device, contiguous, the right
dtype and shape (mask [B, N], cu_seqlens int32 [B+1], max_seqlen int32,
k/v/out matching q).  A rejected call raises and launches nothing (the GPU
cases check the output buffer is untouched)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")


def _rva():
    import ragged_variable_length_amd as rva
    rva.lib()
    return rva


# ---------------------------------------------------------------- host only

def test_host_tensors_are_rejected_without_a_gpu():
    rva = _rva()
    q = torch.zeros(2, 8, 1, 64, dtype=torch.float16)
    m = torch.ones(2, 8, dtype=torch.uint8)
    with pytest.raises(ValueError, match="device tensor"):
        rva.fused(q, q, q, m)
    with pytest.raises(ValueError, match="device tensor"):
        rva.pack(q, None, None, m)
    with pytest.raises(ValueError, match="device tensor"):
        rva.ragged_attend(q[0], q[0], q[0], torch.zeros(3, dtype=torch.int32), 8)
    with pytest.raises(TypeError, match="mask must be uint8 or bool"):
        rva.index(m.float())
    with pytest.raises(ValueError, match=r"mask must be \[B, N\]"):
        rva.index(m[0])
    with pytest.raises(TypeError, match="torch tensor"):
        rva.threshold_l2_mask(np.zeros((2, 8, 64), np.float16), 0.5)


# ---------------------------------------------------------------- on the GPU

def _inputs(device, B=3, N=20, H=2, dtype=torch.float16):
    g = torch.Generator(device="cpu").manual_seed(3)
    q, k, v = (torch.randn(B, N, H, 64, generator=g).to(dtype).to(device) for _ in range(3))
    mask = (torch.rand(B, N, generator=g) < 0.6).to(torch.uint8).to(device)
    return q, k, v, mask


@pytest.mark.gpu
def test_fused_rejects_each_bad_argument(device):
    rva = _rva()
    q, k, v, mask = _inputs(device)
    B, N, H, d = q.shape
    out = torch.full_like(q, 7.0)
    cu = torch.full((B + 1,), -5, dtype=torch.int32, device=device)
    mx = torch.full((1,), -5, dtype=torch.int32, device=device)
    good = dict(q=q, k=k, v=v, mask=mask)
    bad = [
        ("q", q.cpu(), ValueError), ("k", k[:, :N - 1].contiguous(), ValueError),
        ("v", v.to(torch.bfloat16), TypeError), ("k", k.transpose(1, 2), ValueError),
        ("mask", mask.cpu(), ValueError), ("mask", mask[:, :N - 1], ValueError),
        ("mask", mask.to(torch.int32), TypeError), ("mask", mask[: B - 1], ValueError),
        ("q", q.float(), TypeError),
    ]
    for name, value, exc in bad:
        args = dict(good, **{name: value})
        with pytest.raises(exc):
            rva.fused(args["q"], args["k"], args["v"], args["mask"], out=out, cu_seqlens=cu,
                      max_seqlen=mx)
    for kw, exc in ((dict(out=out[:, :N - 1]), ValueError), (dict(out=out.float()), TypeError),
                    (dict(cu_seqlens=cu[:B]), ValueError),
                    (dict(cu_seqlens=cu.to(torch.int64)), TypeError),
                    (dict(cu_seqlens=cu.cpu()), ValueError),
                    (dict(max_seqlen=mx.to(torch.int64)), TypeError)):
        call = dict(out=out, cu_seqlens=cu, max_seqlen=mx)
        call.update(kw)
        with pytest.raises(exc):
            rva.fused(q, k, v, mask, **call)
    work = torch.zeros(2, dtype=torch.int32, device=device)
    with pytest.raises(ValueError):
        rva.fused_persistent(q, k, v, mask, work[:1], out=out)
    with pytest.raises(TypeError):
        rva.fused_persistent(q, k, v, mask, work.to(torch.int64), out=out)
    torch.cuda.synchronize()
    assert (out == 7.0).all(), "a rejected call wrote its output"
    assert (cu == -5).all() and int(mx.item()) == -5


@pytest.mark.gpu
def test_packed_calls_reject_bad_arguments(device):
    rva = _rva()
    q, k, v, mask = _inputs(device)
    B, N, H, d = q.shape
    pk = rva.pack(q, k, v, mask)
    cu = pk["cu_seqlens"]
    o = torch.full_like(pk["q"], 7.0)
    with pytest.raises(ValueError):
        rva.ragged_attend(pk["q"], pk["k"][:-1], pk["v"], cu, N, out=o)
    with pytest.raises(TypeError):
        rva.ragged_attend(pk["q"], pk["k"], pk["v"], cu.to(torch.int64), N, out=o)
    with pytest.raises(ValueError):
        rva.ragged_attend(pk["q"], pk["k"], pk["v"], cu, N, out=o[:-1])
    o_pad = torch.full((B, N, H, d), 7.0, dtype=q.dtype, device=device)
    with pytest.raises(ValueError):
        rva.unpack(pk["q"], cu[:B], mask, out=o_pad)
    with pytest.raises(ValueError):
        rva.unpack(pk["q"], cu, mask, out=o_pad[:, :N - 1])
    with pytest.raises(ValueError):
        rva.pack(q, k, v, mask, outputs={"q": torch.empty(3, H, d, dtype=q.dtype, device=device)})
    with pytest.raises(ValueError):
        rva.pack(q, k, v, mask[:, :5])
    with pytest.raises(ValueError):
        rva.index(mask, out={"kept_index": torch.empty(3, dtype=torch.int32, device=device)})
    torch.cuda.synchronize()
    assert (o == 7.0).all() and (o_pad == 7.0).all()


@pytest.mark.gpu
def test_projection_and_mask_calls_reject_bad_arguments(device):
    rva = _rva()
    B, N, C = 2, 10, 128
    x = torch.randn(B, N, C, device=device).half()
    mask = torch.ones(B, N, dtype=torch.uint8, device=device)
    idx = rva.index(mask)
    w = torch.randn(3 * C, C, device=device).half()
    with pytest.raises(ValueError):
        rva.qkv_projection(x, idx["cu_seqlens"], w[:C], kept_index=idx["kept_index"])
    with pytest.raises(TypeError):
        rva.qkv_projection(x, idx["cu_seqlens"], w.float(), kept_index=idx["kept_index"])
    with pytest.raises(ValueError):
        rva.qkv_projection(x, idx["cu_seqlens"], w, torch.zeros(C, device=device).half(),
                           kept_index=idx["kept_index"])
    wo = torch.randn(C, C, device=device).half()
    o = torch.randn(B * N, C, device=device).half()
    with pytest.raises(ValueError):
        rva.out_projection(o, idx["cu_seqlens"], wo, kept_index=idx["kept_index"])  # no mask
    with pytest.raises(ValueError):
        rva.out_projection(o, idx["cu_seqlens"], wo, kept_index=idx["kept_index"], mask=mask,
                           residual=torch.zeros(B * N, C, device=device).half())
    m_out = torch.full((B, N), 9, dtype=torch.uint8, device=device)
    with pytest.raises(ValueError):
        rva.threshold_l2_mask(x, 0.5, out=m_out[:, :5])
    with pytest.raises(TypeError):
        rva.threshold_l2_mask(x, 0.5, out=m_out.to(torch.int32))
    torch.cuda.synchronize()
    assert (m_out == 9).all()
