"""Randomized blockwise Walsh-Hadamard rotation, written out in float32.

E8-QAT applies Hadamard transforms to the weights before the lattice projection
but leaves them out of its overview figure [E8-QAT, Figure 2 caption].  The
reading used here (the pages give no formula): flip each column by a seeded
+-1 sign, then apply the natural-order (Sylvester) Walsh-Hadamard transform to
every block of ``b`` consecutive columns of a row, un-normalized, one butterfly
stage at a time with the stride ``h = 1, 2, 4, ..., b/2`` in ascending order;
each butterfly maps ``(p, q)`` to ``(fl32(p + q), fl32(p - q))``.  The
orthonormal factor ``kappa_b = fl32(1/sqrt(b))`` is applied afterwards, folded
into the scale (see ``pipeline.row_coefficients``).
"""

import numpy as np


def kappa(b):
    """``fl32(1/sqrt(b))`` computed in float64 and rounded once more to float32.

    Equals 2^-k exactly when b = 4^k.  ``b == 0`` means "no rotation" -> 1.
    """
    if b == 0:
        return np.float32(1.0)
    return np.float32(1.0 / np.sqrt(float(b)))


def fwht_blocks(v, b):
    """Un-normalized Sylvester WHT of every length-``b`` block of the last axis.

    ``v`` is float32 [..., cols] with ``cols % b == 0``; ``b`` a power of two.
    Stage order: ascending stride, as stated in the module docstring.
    """
    v = np.asarray(v, dtype=np.float32)
    cols = v.shape[-1]
    if b < 1 or b & (b - 1) or cols % b:
        raise ValueError("block must be a power of two dividing cols")
    lead = v.shape[:-1]
    out = v.reshape(lead + (cols // b, b)).copy()
    h = 1
    while h < b:
        out = out.reshape(lead + (cols // b, b // (2 * h), 2, h))
        p = out[..., 0, :]
        q = out[..., 1, :]
        out = np.stack([p + q, p - q], axis=-2)
        h *= 2
    return out.reshape(lead + (cols,))


def sylvester_matrix(b):
    """Dense Sylvester Hadamard matrix H_b (float64): H_1 = [1],
    H_2n = [[H_n, H_n], [H_n, -H_n]].  Used only to pin ``fwht_blocks``."""
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < b:
        h = np.block([[h, h], [h, -h]])
    return h
