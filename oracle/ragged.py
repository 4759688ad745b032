"""fp64 CPU oracle for pack -> ragged bidirectional attention -> unpack.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module.  The HIP library never calls it and
shares no code with it; the product path has no CPU fallback.

What the method computes comes from "Dispatch-Aware Ragged Attention for
Pruned Vision Transformers" (arXiv 2604.15408): token pruning leaves each
image with a variable number of tokens; those tokens are packed into one
ragged buffer, bidirectional (non-causal) attention runs independently over
each image's tokens, and the result is returned to the padded layout (sota2.com
page, "Abstract": the pack-attend-unpack pipeline; aissential.tech summary,
"Method": a packer feeding a bidirectional ragged attention kernel).  The pages
write no formula; the plain reading used here is standard scaled dot-product
attention softmax(Q K^T / sqrt(d)) V per image and per head, with the
varlen convention of offsets ("cu_seqlens") the abstract's comparison to
FlashAttention-2 varlen implies.

Readings where the pages are silent (each listed in the design notes):
  * kept tokens keep their original order inside a packed sequence;
  * cu_seqlens is int32[B+1], cu[0] = 0, cu[b+1] = cu[b] + n_b;
  * the kept-index list holds flat b*N + j (int32);
  * pruned rows of the unpacked output are +0;
  * an image that keeps nothing contributes no rows and its output is zeros;
  * scale defaults to 1/sqrt(d).

Every function is the plain definition written out: no tiling, no online
softmax, no fusion.  Floating point is fp64 throughout.

Pins (tests/test_oracle.py): brute-force scalar attention on tiny inputs,
masked-dense equivalence with torch's SDPA in fp64, closed forms (Q = 0 gives
the mean of kept V; one kept token gives its V row; equal keys give the mean),
hand-derived rational fixtures under tests/golden/, invariants (permutation
equivariance, independence across images, key-shift invariance, linearity
in V, convex-hull bounds) and brute-force pack/unpack loops.  No function
here is parity unpinned.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- decoding

def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Bits as the device sees them -> float64.

    f32: IEEE binary32; f16: IEEE binary16; bf16: the top 16 bits of a
    binary32 (uint16 container), so the value is the binary32 whose low 16
    bits are zero.
    """
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------- pack

def seqlens(mask: np.ndarray):
    """Per-image kept counts -> (cu_seqlens int32[B+1], max_seqlen int).

    n_b is the number of kept tokens of image b; cu is its exclusive prefix
    sum with cu[B] = total kept tokens T.
    """
    mask = np.asarray(mask)
    n = (mask != 0).sum(axis=1).astype(np.int64)
    cu = np.zeros(mask.shape[0] + 1, dtype=np.int64)
    cu[1:] = np.cumsum(n)
    max_seqlen = int(n.max()) if n.size else 0
    return cu.astype(np.int32), max_seqlen


def kept_index(mask: np.ndarray) -> np.ndarray:
    """int32[T]: for packed row cu[b] + r, the flat padded position b*N + j of
    the r-th kept token of image b (kept tokens in ascending j)."""
    mask = np.asarray(mask)
    B, N = mask.shape
    parts = [b * N + np.flatnonzero(mask[b]) for b in range(B)]
    if not parts:
        return np.zeros(0, dtype=np.int32)
    return np.concatenate(parts).astype(np.int32)


def pack_rows(x: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Padded [B, N, ...] -> packed [T, ...]: kept rows copied bit for bit in
    kept-index order."""
    B, N = mask.shape
    flat = np.asarray(x).reshape((B * N,) + x.shape[2:])
    return flat[kept_index(mask).astype(np.int64)].copy()


# ---------------------------------------------------------------- attend

def attend(qp: np.ndarray, kp: np.ndarray, vp: np.ndarray, cu: np.ndarray,
           scale: float | None = None) -> np.ndarray:
    """Ragged bidirectional attention over packed fp64 rows.

    qp, kp, vp: [T, H, d] float64 (already decoded); cu: [B+1] offsets.
    For every image b (rows cu[b]..cu[b+1]) and head h independently:
        S = Q K^T * scale,  P = softmax over keys of S,  O = P V.
    No causal mask: every kept query sees every kept key of its own image
    and nothing of any other image.  The row maximum is subtracted before
    exponentiation only to keep exp finite; it cancels in the ratio.
    """
    qp = np.asarray(qp, dtype=np.float64)
    kp = np.asarray(kp, dtype=np.float64)
    vp = np.asarray(vp, dtype=np.float64)
    T, H, d = qp.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((T, H, vp.shape[2]), dtype=np.float64)
    cu = np.asarray(cu, dtype=np.int64)
    for b in range(cu.shape[0] - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi <= lo:
            continue
        for h in range(H):
            q = qp[lo:hi, h, :]
            k = kp[lo:hi, h, :]
            v = vp[lo:hi, h, :]
            s = (q @ k.T) * scale
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            out[lo:hi, h, :] = (p @ v) / p.sum(axis=1, keepdims=True)
    return out


# ---------------------------------------------------------------- unpack

def unpack(o_packed: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Packed [T, ...] -> padded [B, N, ...]: kept positions receive their
    packed row, pruned positions are +0."""
    mask = np.asarray(mask)
    B, N = mask.shape
    out = np.zeros((B * N,) + o_packed.shape[1:], dtype=o_packed.dtype)
    out[kept_index(mask).astype(np.int64)] = o_packed
    return out.reshape((B, N) + o_packed.shape[1:])


# ---------------------------------------------------------------- whole path

def pack_attend_unpack(q, k, v, mask, dtype: str, scale: float | None = None):
    """The full path on padded inputs (device bits): returns (O_pad float64
    [B,N,H,d], cu_seqlens, max_seqlen, kept_index)."""
    cu, mx = seqlens(mask)
    qp = decode(pack_rows(q, mask), dtype)
    kp = decode(pack_rows(k, mask), dtype)
    vp = decode(pack_rows(v, mask), dtype)
    o = attend(qp, kp, vp, cu, scale)
    return unpack(o, mask), cu, mx, kept_index(mask)


def attend_image_head(q, k, v, mask, dtype: str, b: int, h: int, scale: float | None = None):
    """Oracle output rows for one (image, head) of a padded workload, computed
    on their own (for sampled checks of large workloads).  Returns
    (kept positions j, O rows [n_b, d] float64)."""
    keep = np.flatnonzero(np.asarray(mask)[b])
    qq = decode(np.asarray(q)[b, keep, h, :], dtype)
    kk = decode(np.asarray(k)[b, keep, h, :], dtype)
    vv = decode(np.asarray(v)[b, keep, h, :], dtype)
    n = keep.shape[0]
    if n == 0:
        return keep, np.zeros((0, qq.shape[-1]))
    cu = np.array([0, n], dtype=np.int64)
    o = attend(qq[:, None, :], kk[:, None, :], vv[:, None, :], cu, scale)
    return keep, o[:, 0, :]
