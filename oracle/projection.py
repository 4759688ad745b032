"""fp64 CPU oracle for the projections around ragged attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module.  The HIP library never calls it and
shares no code with it.

The aissential.tech summary's "Method" has the packer feed the transformer
block and its "In practice" asks for attention and the rest of the block to
be timed apart.  The rest of an attention block is two affine maps of the
token rows (the standard ViT attention block; the pages write no formula):
  * the QKV projection  [q | k | v] = x W_qkv^T + b_qkv, W_qkv of shape
    [3C, C] (output features by input features), q, k, v each C = H * 64
    wide with head h in columns 64h .. 64h + 63;
  * the output projection y = o W_o^T + b_o (+ a residual term when given).
On the ragged path both act on the kept rows only: the QKV projection reads
the packed rows of the padded embeddings, and the output projection's rows
return to their padded positions with pruned rows +0 (the unpack's rule).

Every function is the definition written out with a matrix product as its
one library step; floating point is fp64 on the decoded input bits, with no
intermediate rounding.

Pins (tests/test_oracle_projection.py): a scalar triple loop on tiny
inputs, closed forms (identity weight, zero weight, one-hot weight picks a
column), linearity in x, the column-group split, and the packed/padded
relations with pack_rows / unpack.
"""
from __future__ import annotations

import numpy as np

from .ragged import decode, pack_rows, unpack


def linear(x: np.ndarray, w: np.ndarray, b: np.ndarray | None = None,
           residual: np.ndarray | None = None) -> np.ndarray:
    """y = x w^T + b (+ residual) in fp64; x [M, K], w [Nout, K], b [Nout]."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
    if b is not None:
        y = y + np.asarray(b, dtype=np.float64)
    if residual is not None:
        y = y + np.asarray(residual, dtype=np.float64)
    return y


def qkv_projection(x_pad: np.ndarray, mask: np.ndarray | None, w_qkv: np.ndarray,
                   b_qkv: np.ndarray | None, dtype: str):
    """Device bits in -> fp64 packed (q, k, v), each [T, C].  With mask None
    the input rows are already packed ([T, C])."""
    x = decode(x_pad, dtype)
    xp = pack_rows(x, mask) if mask is not None else x
    w = decode(w_qkv, dtype)
    b = decode(b_qkv, dtype) if b_qkv is not None else None
    y = linear(xp, w, b)
    C = w.shape[1]
    return y[:, :C], y[:, C:2 * C], y[:, 2 * C:]


def out_projection(o_packed: np.ndarray, mask: np.ndarray | None, w_o: np.ndarray,
                   b_o: np.ndarray | None, dtype: str, residual: np.ndarray | None = None):
    """Device bits in -> fp64 output.  With a mask: padded [B, N, C], kept
    rows are the projected packed rows (plus the padded residual rows), pruned
    rows +0.  With mask None: packed [T, C] (plus the packed residual)."""
    o = decode(o_packed, dtype)
    w = decode(w_o, dtype)
    b = decode(b_o, dtype) if b_o is not None else None
    if mask is None:
        r = decode(residual, dtype) if residual is not None else None
        return linear(o, w, b, r)
    y = unpack(linear(o, w, b), mask)
    if residual is not None:
        y = y + np.where(mask[..., None] != 0, decode(residual, dtype), 0.0)
    return y
