"""The library's ceiling probes produce exactly what they are documented to
produce: the copy moves every byte, the read probe's per-thread folds match
a host fold of the same pieces, and the gather probe writes q ^ k ^ v into
every kept row's slice and zero into every pruned row (odd head counts
included).  Their timings stand beside the attention's in the bench, so
they are checked like any other kernel."""
import sys

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import upload  # noqa: E402


def _rva():
    import ragged_variable_length_amd as rva
    rva.lib()
    return rva


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_copy_probe_moves_every_byte(device):
    rva = _rva()
    n = (1 << 20) + 16 * 37  # not a multiple of the grid's stride
    src = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device=device)
    dst = torch.zeros_like(src)
    _say("[probe] copy")
    rva.probe_copy(src, dst, 8)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_read_probe_folds_what_it_reads(device):
    rva = _rva()
    grid = 6
    n = 4 * (1 << 16) + 4 * 123  # 32-bit words: whole 16-byte pieces, a partial last stride
    host = np.random.default_rng(5).integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(device)
    sink = torch.zeros(grid * 256, dtype=torch.int32, device=device)
    _say("[probe] read")
    rva.probe_read(src, sink, grid)
    torch.cuda.synchronize()
    # thread t folds pieces t, t + S, t + 2S, ... (S = grid * 256 threads),
    # each piece's four words XORed together
    words = host.reshape(-1, 4)
    piece = words[:, 0] ^ words[:, 1] ^ words[:, 2] ^ words[:, 3]
    S = grid * 256
    pad = np.zeros((-len(piece)) % S, dtype=np.uint32)
    want = np.bitwise_xor.reduce(np.concatenate([piece, pad]).reshape(-1, S), axis=0)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)


@pytest.mark.parametrize("B,N,H,dtype", [(9, 197, 5, "f16"), (6, 40, 12, "bf16"), (3, 577, 1, "f16")])
def test_gather_probe_writes_its_pattern(device, B, N, H, dtype):
    rva = _rva()
    counts = [0, N, 1] + [int(c) for c in np.random.default_rng(B).integers(1, N + 1, size=B - 3)]
    w = W.random_workload(70 + B, B=B, N=N, H=H, dtype=dtype, counts=counts[:B])
    q, k, v, mask = upload(w, device)
    idx = rva.index(mask)
    out = torch.full_like(q, float("nan"))
    _say(f"[probe] gather B={B} N={N} H={H} {dtype}")
    rva.probe_gather(q, k, v, mask, idx["cu_seqlens"], idx["kept_index"], out)
    torch.cuda.synchronize()
    b = lambda t: t.view(torch.int16).cpu().numpy()
    want = b(q) ^ b(k) ^ b(v)
    want[w.mask == 0] = 0
    assert np.array_equal(b(out), want)


def test_gather_probe_mixed_batch(device):
    """The bench's configuration: the 1024-image mixed batch, every row."""
    rva = _rva()
    w = W.mixed_peak()
    q, k, v, mask = upload(w, device)
    idx = rva.index(mask)
    out = torch.full_like(q, float("nan"))
    _say("[probe] gather mixed batch")
    rva.probe_gather(q, k, v, mask, idx["cu_seqlens"], idx["kept_index"], out)
    torch.cuda.synchronize()
    b = lambda t: t.view(torch.int16).cpu().numpy()
    want = b(q) ^ b(k) ^ b(v)
    want[w.mask == 0] = 0
    assert np.array_equal(b(out), want)
