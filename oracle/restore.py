"""Inverse rotation: lattice points back to the original weight basis, and
gradients from the rotated basis back to the latent weights.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The forward rotation of a row block is ``u = R w`` with
``R = kappa_b * H_b * diag(sigma)`` (sign flip, natural-order Walsh-Hadamard
transform, ``kappa_b = fl32(1/sqrt(b))``).  ``H_b`` is symmetric with
``H_b H_b = b I``, so ``R`` is orthogonal and ``R^T = diag(sigma) H_b kappa_b``:
the inverse applies the transform first and the signs last.  E8-QAT applies
Hadamard transforms around its projection and leaves them out of the overview
figure [E8-QAT, Figure 2 caption]; these functions are the plainest readings of
undoing that rotation, which the pages do not write out:

* restored weights ``w_hat = R^T (s z) = sigma * fl32(T * c2)`` with
  ``T = H_b (2z)`` (float32 butterflies in the forward stage order; exact for
  every realistic ``2z``) and ``c2 = fl32(fl32(s * kappa_b) * 0.5)``;
* the rotated-basis gradient ``dL/dw = R^T dL/du = sigma * fl32(kappa_b * H_b g)``
  (the identity straight-through estimator through the rounding, with the exact
  Jacobian of the rotation [E8-QAT, Figure 2(b) caption: identity STE]).

Zeros: the product is taken as ``fl32(T * c2) + 0`` so that every zero is +0
before the sign flip (the flip then gives ``sigma * +0``).  Rows whose scale is
invalid (the projection's bad-row rule) restore to ``sigma * +0``.
"""

import numpy as np

from .hadamard import fwht_blocks, kappa
from .pipeline import (_shape3, _widen, f32_to_bf16, project)


def restore_coefficients(s, had_block):
    """``c2_r = fl32(fl32(s_r * kappa_b) * 0.5)`` for valid rows."""
    s = np.asarray(s, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        return ((s * kappa(had_block)).astype(np.float32) * np.float32(0.5)).astype(np.float32)


def restore_original(two_z, s, signs, had_block, bad_row_of_rows=None):
    """Restored weights ``[batch, rows, cols]`` (float32) from ``2z``.

    ``two_z``: integer [batch, rows, cols] (or [G, 8] with the shape given by
    ``s`` and ``signs``); ``s``: float32 [batch*rows]; ``signs``: +-1 [cols];
    ``bad_row_of_rows``: bool [batch*rows] rows restored to ``sigma * +0``.
    """
    sig = np.asarray(signs, dtype=np.int8).astype(np.float32)
    cols = sig.shape[0]
    s = np.asarray(s, dtype=np.float32).reshape(-1)
    t = np.asarray(two_z).astype(np.float32).reshape(s.shape[0], cols)   # exact: |2z| < 2^15
    T = fwht_blocks(t, int(had_block))
    c2 = restore_coefficients(s, had_block)
    if bad_row_of_rows is not None:
        c2 = np.where(np.asarray(bad_row_of_rows), np.float32(0.0), c2).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (T * c2[:, None]).astype(np.float32) + np.float32(0.0)
    return (y * sig).astype(np.float32)


def project_restore(w, s, signs, had_block, w_is_bf16=True, core_bound=-1):
    """Forward projection with the output restored to the original basis.

    Returns the ``project`` dict plus ``w_hat_f32`` and ``w_hat_bf16``
    ([batch, rows, cols]).
    """
    out = project(w, s, signs, had_block, w_is_bf16, core_bound)
    batch, rows, cols = _shape3(w)
    s32 = np.asarray(s, dtype=np.float32).reshape(batch * rows)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        c = kappa(had_block) * (np.float32(1.0) / s32)
    bad = ~(s32 > 0) | np.isinf(s32) | np.isinf(c)
    wh = restore_original(out["two_z"].reshape(batch, rows, cols), s32, signs, had_block, bad)
    out["w_hat_f32"] = wh.reshape(batch, rows, cols)
    out["w_hat_bf16"] = f32_to_bf16(out["w_hat_f32"])
    return out


def rotate_grad(grad_q, signs, had_block, is_bf16=True):
    """``sigma * (fl32(kappa_b * H_b g) + 0)`` per row block, float32
    [..., cols]; ``grad_q`` as bf16 bits or float32."""
    g = _widen(grad_q, is_bf16)
    sig = np.asarray(signs, dtype=np.int8).astype(np.float32)
    T = fwht_blocks(g, int(had_block))
    with np.errstate(over="ignore", invalid="ignore"):
        y = (T * kappa(had_block)).astype(np.float32) + np.float32(0.0)
    return (y * sig).astype(np.float32)


def ste_backward_hadamard(grad_q, signs, had_block, is_bf16=True, w_latent=None, lr=None):
    """Gradient of the latent weights through the rotation, and optionally the
    SGD step ``w <- fl32(w - fl32(lr * g))`` on it (``g`` in float32, before
    any rounding of the returned gradient).

    Returns ``(grad_w, w_new)``: ``grad_w`` in the dtype of ``grad_q`` (bf16
    bits by round-to-nearest-even, every NaN as 0x7FC0), ``w_new`` likewise or
    None.
    """
    g = rotate_grad(grad_q, signs, had_block, is_bf16)
    grad_w = f32_to_bf16(g) if is_bf16 else g
    w_new = None
    if w_latent is not None:
        wf = _widen(w_latent, is_bf16)
        with np.errstate(over="ignore", invalid="ignore"):
            new = (wf - (np.float32(lr) * g).astype(np.float32)).astype(np.float32)
        w_new = f32_to_bf16(new) if is_bf16 else new
    return grad_w, w_new
