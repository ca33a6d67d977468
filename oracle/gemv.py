"""Products of the exported weights with activations (the decode-time GEMV).

TEST INFRASTRUCTURE ONLY (see the package docstring).

E8-QAT reports decode throughput of its 2-bit representation against BF16
(abstract); the product it serves is ``y = W_hat x`` with ``W_hat`` the
restored weights of the exported form [E8-QAT, Figure 2(c) caption].  The
reference here is that product in float64 from the exact restored weights
``w_hat = sigma * H_b (s z) / sqrt(b)`` (no rounding anywhere), together with
the magnitude sum that bounds the float32 rounding error of any evaluation
order (used by the tests to state their tolerance).
"""

import numpy as np

from .hadamard import sylvester_matrix


def exact_restored(two_z, s, signs=None, had_block=0):
    """``W_hat`` [batch, rows, cols] in float64, exactly (2z is an integer
    array [batch, rows, cols]; s float32 [batch*rows])."""
    two_z = np.asarray(two_z, dtype=np.float64)
    batch, rows, cols = two_z.shape
    sc = np.asarray(s, dtype=np.float64).reshape(batch, rows, 1)
    z = two_z * 0.5 * sc
    if signs is None or had_block == 0:
        return z
    b = int(had_block)
    H = sylvester_matrix(b)
    blk = z.reshape(batch, rows, cols // b, b) @ H.T
    return blk.reshape(batch, rows, cols) / np.sqrt(float(b)) * np.asarray(signs, dtype=np.float64)


def gemv_reference(two_z, s, x, signs=None, had_block=0):
    """``y[b, t, r] = sum_c W_hat[b, r, c] x[b, t, c]`` in float64 and the
    magnitude ``sum_c |W_hat[b, r, c]| * |x[b, t, c]|`` (same shape).

    ``x``: [batch, m, cols] float values (bf16 activations given as their
    float values).
    """
    W = exact_restored(two_z, s, signs, had_block)
    x = np.asarray(x, dtype=np.float64)
    y = np.einsum("brc,btc->btr", W, x)
    mag = np.einsum("brc,btc->btr", np.abs(W), np.abs(x))
    return y, mag


def rotated_bound(x, signs=None, had_block=0):
    """``xbar``: the block sums of ``|x|`` scaled by 1/sqrt(b) (``|x|`` with no
    rotation), a bound on every ``|x_tilde_i|`` of the rotated activation
    ``x_tilde = H_b (sigma * x) / sqrt(b)`` (each entry is a signed sum over
    the block)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    if signs is None or had_block == 0:
        return x
    b = int(had_block)
    lead = x.shape[:-1]
    cols = x.shape[-1]
    return np.repeat(x.reshape(lead + (cols // b, b)).sum(-1), b, axis=-1) / np.sqrt(float(b))


def rotated_magnitude(two_z, s, x, signs=None, had_block=0):
    """``s_r * sum_g sum_i |z_gi| * xbar_gi`` with ``xbar`` the block sums of
    ``|x|`` scaled by 1/sqrt(b): a bound on the terms of the rotated-basis
    evaluation ``y_r = s_r sum z . x_tilde`` (``|x_tilde_i| <= xbar_i``)."""
    two_z = np.asarray(two_z, dtype=np.float64)
    batch, rows, cols = two_z.shape
    x = np.abs(np.asarray(x, dtype=np.float64))
    if signs is None or had_block == 0:
        xbar = x
    else:
        b = int(had_block)
        xbar = np.repeat(x.reshape(batch, -1, cols // b, b).sum(-1), b, axis=-1) / np.sqrt(float(b))
    sc = np.asarray(s, dtype=np.float64).reshape(batch, rows)
    return np.einsum("brc,btc->btr", np.abs(two_z) * 0.5, xbar) * sc[:, None, :]
