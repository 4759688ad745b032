"""Seeded synthetic inputs for the pack -> ragged attention -> unpack path.

The paper ("Dispatch-Aware Ragged Attention for Pruned Vision Transformers",
arXiv 2604.15408) evaluates DeiT-T/S/B on ImageNet-1k val with four pruning
policies (aissential.tech summary, "Summary"; sota2.com page, "Recorded
benchmark results").  Neither the dataset nor trained weights are used here:
these generators only reproduce the *shapes* of that workload (224x224 images
give 197 tokens = CLS + 14x14 patches, 384x384 give 577 = CLS + 24x24; DeiT-S
has 6 heads, DeiT-B 12, head_dim 64) and a ragged keep-mask per image.

This module is shared by the tests, the bench and the smoke check.  It holds
none of the method's arithmetic (no packing, no attention): it only draws
padded Q/K/V tensors and a keep-mask.  The oracle and the HIP path both
consume what it returns and neither is imported here.

Every array is a plain numpy array with the exact bits the device sees:
  f32  -> np.float32
  f16  -> np.float16 (numpy's float32 -> float16 cast, round-to-nearest-even)
  bf16 -> np.uint16 holding bfloat16 bits (float32 -> bfloat16 rounding done
          here with integer round-to-nearest-even; inputs are finite)
Padded layout is [B, N, H, d] row-major; the mask is uint8 [B, N], 1 = keep.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 64

DTYPES = ("f32", "f16", "bf16")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits with round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # add 0x7FFF plus the lowest kept bit, then truncate: RNE on the top 16 bits
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(np.asarray(x, dtype=np.float32).astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass
class Workload:
    name: str
    B: int
    N: int
    H: int
    d: int
    dtype: str
    mask: np.ndarray  # uint8 [B, N]
    q: np.ndarray     # [B, N, H, d] in the dtype's bit container
    k: np.ndarray
    v: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def counts(self) -> np.ndarray:
        return self.mask.sum(axis=1).astype(np.int64)

    @property
    def total_kept(self) -> int:
        return int(self.mask.sum())


def _mask_from_counts(rng: np.random.Generator, counts: np.ndarray, N: int) -> np.ndarray:
    """CLS (token 0) always kept, plus (n_b - 1) patches drawn without
    replacement from 1..N-1, for each image."""
    B = counts.shape[0]
    mask = np.zeros((B, N), dtype=np.uint8)
    for b in range(B):
        n = int(counts[b])
        mask[b, 0] = 1
        if n > 1:
            pick = rng.choice(np.arange(1, N), size=n - 1, replace=False)
            mask[b, pick] = 1
    return mask


def _normal_qkv(rng: np.random.Generator, B: int, N: int, H: int, d: int, dtype: str):
    out = []
    for _ in range(3):
        x = rng.standard_normal((B, N, H, d), dtype=np.float32)
        out.append(_cast(x, dtype))
        del x
    return out


def random_workload(seed: int, B: int, N: int, H: int, dtype: str, counts=None,
                    d: int = HEAD_DIM, name: str = "random", keep_prob=None) -> Workload:
    """A general seeded workload (used for edge and property cases).

    counts: explicit kept counts per image (CLS-first subsets), or None.
    keep_prob: if given (and counts is None), each token is kept independently
    with this probability -- no CLS rule, so images may keep nothing.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if counts is not None:
        counts = np.asarray(counts, dtype=np.int64)
        mask = np.zeros((B, N), dtype=np.uint8)
        for b in range(B):
            n = int(counts[b])
            if n > 0:
                mask[b, rng.choice(np.arange(N), size=n, replace=False)] = 1
    elif keep_prob is not None:
        mask = (rng.random((B, N)) < keep_prob).astype(np.uint8)
    else:
        mask = np.ones((B, N), dtype=np.uint8)
    q, k, v = _normal_qkv(rng, B, N, H, d, dtype)
    return Workload(name, B, N, H, d, dtype, mask, q, k, v, {"seed": seed})


def tiny(seed: int = 1001) -> Workload:
    """Tiny: 2 images, 197 tokens, 3 heads, fp32, Q/K/V ~ N(0,1).
    Kept counts (CLS included) uniform on [40, 120]."""
    B, N, H = 2, 197, 3
    rng = np.random.Generator(np.random.PCG64(seed))
    counts = rng.integers(40, 121, size=B)
    mask = _mask_from_counts(rng, counts, N)
    q, k, v = _normal_qkv(rng, B, N, H, HEAD_DIM, "f32")
    return Workload("tiny_b2_n197_h3_f32", B, N, H, HEAD_DIM, "f32", mask, q, k, v,
                    {"seed": seed})


def deit_s_224_threshold_l2(seed: int = 1002) -> Workload:
    """DeiT-S-shaped 224x224, batch 4, 6 heads, bf16.

    Token embeddings x ~ N(0,1) of shape [4, 197, 384]; W_q, W_k, W_v ~ N(0, 1/384)
    (variance); Q/K/V = x W computed in fp64, rounded to fp32 then to bf16.
    Head h is columns 64h..64h+63.  Threshold-L2 pruning at a 50% keep rate:
    CLS plus every patch whose L2 norm is at or above the per-image 0.5-quantile
    (linear interpolation) of the 196 patch norms.
    """
    B, N, H, d = 4, 197, 6, HEAD_DIM
    C = H * d
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((B, N, C))
    ws = [rng.standard_normal((C, C)) / np.sqrt(C) for _ in range(3)]
    norms = np.sqrt((x * x).sum(axis=2))
    mask = np.zeros((B, N), dtype=np.uint8)
    mask[:, 0] = 1
    for b in range(B):
        thr = np.quantile(norms[b, 1:], 0.5)
        mask[b, 1:] = (norms[b, 1:] >= thr).astype(np.uint8)
    q, k, v = [_cast((x @ w).astype(np.float32).reshape(B, N, H, d), "bf16") for w in ws]
    return Workload("deit_s_224_b4_h6_bf16_thresholdL2", B, N, H, d, "bf16", mask, q, k, v,
                    {"seed": seed, "x": x.astype(np.float32), "keep_quantile": 0.5})


DEIT_B_224_RATES = (0.0, 0.2, 0.5, 0.8)


def deit_b_224(rate: float, seed: int | None = None) -> Workload:
    """DeiT-B-shaped 224x224, batch 64, 12 heads, fp16 ~ N(0,1).

    Pruning rate p: at p = 0 every token is kept.  Otherwise
    n_b = clip(rint((1 - p) * 197 * u_b), 1, 197) with u_b ~ U[0.9, 1.1]
    (the +-10% jitter), CLS plus (n_b - 1) random patches.
    """
    B, N, H = 64, 197, 12
    i = DEIT_B_224_RATES.index(rate)
    if seed is None:
        seed = 1003 + 10 * i
    rng = np.random.Generator(np.random.PCG64(seed))
    if rate == 0.0:
        mask = np.ones((B, N), dtype=np.uint8)
    else:
        u = rng.uniform(0.9, 1.1, size=B)
        counts = np.clip(np.rint((1.0 - rate) * N * u), 1, N).astype(np.int64)
        mask = _mask_from_counts(rng, counts, N)
    q, k, v = _normal_qkv(rng, B, N, H, HEAD_DIM, "f16")
    return Workload(f"deit_b_224_b64_h12_f16_p{int(round(rate * 100))}", B, N, H, HEAD_DIM,
                    "f16", mask, q, k, v, {"seed": seed, "rate": rate})


def deit_b_384(seed: int = 1004) -> Workload:
    """DeiT-B-shaped 384x384, batch 32, 577 tokens, 12 heads, bf16 ~ N(0,1).
    80% pruning with kept counts (CLS included) uniform on [92, 139]."""
    B, N, H = 32, 577, 12
    rng = np.random.Generator(np.random.PCG64(seed))
    counts = rng.integers(92, 140, size=B)
    mask = _mask_from_counts(rng, counts, N)
    q, k, v = _normal_qkv(rng, B, N, H, HEAD_DIM, "bf16")
    return Workload("deit_b_384_b32_h12_bf16_p80", B, N, H, HEAD_DIM, "bf16", mask, q, k, v,
                    {"seed": seed})


def mixed_peak(seed: int = 1005, B: int = 1024) -> Workload:
    """Peak-throughput mixed batch: 1024 DeiT-B-shaped sequences (197 tokens,
    12 heads, fp16 ~ N(0,1)).  Per-image pruning rate p_b ~ U[0, 0.9],
    n_b = clip(rint((1 - p_b) * 197), 1, 197), so lengths span 20..197."""
    N, H = 197, 12
    rng = np.random.Generator(np.random.PCG64(seed))
    p = rng.uniform(0.0, 0.9, size=B)
    counts = np.clip(np.rint((1.0 - p) * N), 1, N).astype(np.int64)
    mask = _mask_from_counts(rng, counts, N)
    q, k, v = _normal_qkv(rng, B, N, H, HEAD_DIM, "f16")
    return Workload(f"mixed_b{B}_n197_h12_f16", B, N, H, HEAD_DIM, "f16", mask, q, k, v,
                    {"seed": seed})


def embeddings(seed: int = 1006, B: int = 1024, N: int = 197, C: int = 768,
               dtype: str = "f16") -> np.ndarray:
    """Token embeddings x ~ N(0, 1) of shape [B, N, C] in the dtype's bit
    container: the input of the Threshold-l2 keep-mask at DeiT-B width."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _cast(rng.standard_normal((B, N, C), dtype=np.float32), dtype)


def projection_weights(seed: int = 1007, C: int = 768, dtype: str = "f16") -> dict:
    """Synthetic attention-block weights in nn.Linear layout: W_qkv [3C, C] and
    W_o [C, C] ~ N(0, 1/C) (variance), biases ~ N(0, 0.02^2), in the dtype's
    bit container."""
    rng = np.random.Generator(np.random.PCG64(seed))
    s = np.float32(1.0 / np.sqrt(C))
    w_qkv = rng.standard_normal((3 * C, C), dtype=np.float32) * s
    b_qkv = rng.standard_normal(3 * C, dtype=np.float32) * np.float32(0.02)
    w_o = rng.standard_normal((C, C), dtype=np.float32) * s
    b_o = rng.standard_normal(C, dtype=np.float32) * np.float32(0.02)
    return {k: _cast(v, dtype) for k, v in
            (("w_qkv", w_qkv), ("b_qkv", b_qkv), ("w_o", w_o), ("b_o", b_o))}


def all_configs():
    """The five workloads in order; the DeiT-B 224 sweep contributes one per rate."""
    yield tiny()
    yield deit_s_224_threshold_l2()
    for r in DEIT_B_224_RATES:
        yield deit_b_224(r)
    yield deit_b_384()
    yield mixed_peak()


CONFIG_BUILDERS = {
    "tiny": tiny,
    "deit_s_224": deit_s_224_threshold_l2,
    "deit_b_224_p0": lambda: deit_b_224(0.0),
    "deit_b_224_p20": lambda: deit_b_224(0.2),
    "deit_b_224_p50": lambda: deit_b_224(0.5),
    "deit_b_224_p80": lambda: deit_b_224(0.8),
    "deit_b_384": deit_b_384,
    "mixed": mixed_peak,
}
