"""PTQ initialization onto the fixed core.

TEST INFRASTRUCTURE ONLY (see the package docstring).

E8-QAT initializes its latent weights by post-training quantization onto a
fixed E8 core before QAT starts [E8-QAT, Figure 2(a) caption], so that training
begins with no escapes (Table 9: the escape fraction is exactly zero at the
first checkpoint).  The pages do not give the PTQ procedure; the plainest
reading, used here:

* finite-core projection: the nearest E8 point of the normalized group
  (``lattice.nearest_e8_two_z``, the projection's own rule) when it lies in the
  core C(B); otherwise the nearest point of C(B) by exhaustive search, where the
  comparison key of a core point 2z = t is ``x.t - ||t||^2 / 4`` (maximal for
  the nearest point) evaluated in float64 in one fixed order -- products
  ``x_i t_i`` (exact), pairwise sums ((0+1)+(2+3))+((4+5)+(6+7)), then minus
  ``||t||^2 / 4`` (exact) -- and equal keys go to the lower core index;
* per-row scale search: candidate scales ``s_k = fl32(alpha_k * s0_r)`` for
  given multipliers ``alpha_k``; the row's squared error in the rotated basis
  (equal to the weight-space error, the rotation being orthogonal) is the
  exact rational number ``E_k = sum_i (kappa_b v_i - s_k t_i / 2)^2`` over the
  row (``v`` the un-normalized float32 transform, ``kappa_b`` and ``s_k`` their
  float32 values, ``t`` the finite-core projection at ``s_k``).  The candidate
  with the smallest ``E_k`` wins, ties go to the smaller k; a candidate whose
  scale is invalid (the projection's bad-row rule) has ``E_k = +inf``; a row
  with a non-finite ``v`` has no defined error (NaN), which counts as +inf.
  The errors are computed exactly with scaled integers: every float32 value is
  a multiple of 2^-149, so ``2^300 (2 kappa_b v_i - s_k t_i)`` is an integer.
"""

from fractions import Fraction

import numpy as np

from .core import core_points, core_rank
from .hadamard import fwht_blocks, kappa
from .lattice import nearest_e8_two_z
from .pipeline import (STATUS_BAD_SCALE, STATUS_NONFINITE, STATUS_X_RANGE, X_LIMIT, _shape3, _widen,
                       row_coefficients)

def core_search_two_z(x, core_bound, chunk=4096):
    """Nearest point of C(B) to each row of ``x`` (float32 [G, 8]) by the
    float64 key described in the module docstring; 2z as int64 [G, 8]."""
    pts = core_points(core_bound).astype(np.int64)              # rank order
    tf = pts.astype(np.float64)
    n4 = (pts * pts).sum(1).astype(np.float64) / 4.0
    out = np.zeros((len(x), 8), dtype=np.int64)
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    for lo in range(0, len(x), chunk):
        xs = x64[lo:lo + chunk]
        p = xs[:, None, :] * tf[None, :, :]                     # exact
        key = ((p[..., 0] + p[..., 1]) + (p[..., 2] + p[..., 3])) + \
              ((p[..., 4] + p[..., 5]) + (p[..., 6] + p[..., 7]))
        key = key - n4[None, :]
        out[lo:lo + chunk] = pts[np.argmax(key, axis=1)]         # first maximum = lowest rank
    return out


def core_project_two_z(x, core_bound):
    """Finite-core projection of valid groups ``x`` (float32 [G, 8])."""
    tz = nearest_e8_two_z(x)
    esc = (tz * tz).sum(1) > core_bound
    if esc.any():
        tz[esc] = core_search_two_z(x[esc], core_bound)
    return tz


def _rotated(w, signs, had_block, w_is_bf16):
    v = _widen(w, w_is_bf16)
    if v.ndim == 2:
        v = v[None]
    if signs is not None:
        v = fwht_blocks(v * np.asarray(signs, dtype=np.int8).astype(np.float32), int(had_block))
    return v.astype(np.float32)


def _project_rows(v, s, had_block, core_bound):
    """Finite-core projection of every group of the rows ``v`` [R, cols] at
    scales ``s`` [R].  Returns (2z int64 [R, cols/8, 8], bad_row [R],
    nonfinite_row [R], xrange_row [R])."""
    rows, cols = v.shape
    c, bad = row_coefficients(s, had_block)
    with np.errstate(over="ignore", invalid="ignore"):
        x = (v * c[:, None]).astype(np.float32).reshape(rows, cols // 8, 8)
    finite = np.isfinite(x).all(-1)
    with np.errstate(invalid="ignore"):
        small = (np.abs(np.where(np.isfinite(x), x, 0)) < X_LIMIT).all(-1)
    valid = ~bad[:, None] & finite & small
    tz = np.zeros((rows, cols // 8, 8), dtype=np.int64)
    if valid.any():
        tz[valid] = core_project_two_z(x[valid], core_bound)
    nonfinite = (~bad[:, None] & ~finite).any(1)
    xrange = (~bad[:, None] & finite & ~small).any(1)
    return tz, bad, nonfinite, xrange


_SHIFT = 300      # 2^300 * (2 kappa v - s t) is an integer for float32 kappa, v, s


def _scaled(x):
    """``x * 2^_SHIFT`` as an exact integer for a finite float that is a
    multiple of 2^-_SHIFT."""
    n, d = float(x).as_integer_ratio()          # d is a power of two
    return (n << _SHIFT) // d


def exact_row_errors(v, s, tz, had_block):
    """Exact ``E = sum_i (kappa_b v_i - s t_i / 2)^2`` of every row, as a
    ``Fraction`` (None for a row with a non-finite ``v``): rows ``v`` float32
    [R, cols], scales ``s`` float32 [R], points ``tz`` (2z) [R, cols/8, 8].
    With ``U_i = 2^300 (2 kappa_b v_i - s t_i)`` (an integer),
    ``E = sum_i U_i^2 / (4 * 2^600)``."""
    rows, cols = v.shape
    k = float(kappa(had_block))
    kn, kd = k.as_integer_ratio()
    t_all = np.asarray(tz, dtype=np.int64).reshape(rows, cols)
    out = []
    for r in range(rows):
        vr = np.asarray(v[r], dtype=np.float32)
        if not np.isfinite(vr).all():
            out.append(None)
            continue
        a = []
        for x in vr.astype(np.float64):
            n, d = float(x).as_integer_ratio()
            a.append(((2 * kn * n) << _SHIFT) // (kd * d))     # 2^300 * 2 kappa v, exact
        sc = _scaled(np.float32(s[r]))
        total = 0
        for ai, ti in zip(a, t_all[r].tolist()):
            u = ai - sc * ti
            total += u * u
        out.append(Fraction(total, 4 << (2 * _SHIFT)))
    return out


def ptq_init(w, s0, alphas, signs=None, had_block=0, core_bound=16, w_is_bf16=True):
    """Per-row scale search and finite-core projection.

    ``w`` [batch, rows, cols] (bf16 bits or float32), ``s0`` float32
    [batch*rows], ``alphas`` float32 [K].  Returns a dict with ``scale``
    (float32 [batch*rows]), ``k`` (int64), ``err_exact`` (per row, per k: a
    Fraction, ``inf`` for an invalid scale, None for a row with a non-finite
    transform), ``err`` (float64 [batch*rows, K]: the nearest float64 to each
    exact error, +inf, or NaN), ``two_z`` (int64 [G, 8]), ``core_idx``
    (uint16 [G]) and ``status``.
    """
    batch, rows, cols = _shape3(w)
    R = batch * rows
    v = _rotated(w, signs, had_block, w_is_bf16).reshape(R, cols)
    s0 = np.asarray(s0, dtype=np.float32).reshape(-1)
    alphas = np.asarray(alphas, dtype=np.float32)
    K = len(alphas)
    exact = [[None] * K for _ in range(R)]
    err = np.zeros((R, K), dtype=np.float64)
    for k in range(K):
        with np.errstate(over="ignore", invalid="ignore"):
            sk = (alphas[k] * s0).astype(np.float32)
        tz, bad, _, _ = _project_rows(v, sk, had_block, core_bound)
        e = exact_row_errors(v, sk, tz, had_block)
        for r in range(R):
            exact[r][k] = float("inf") if bad[r] else e[r]
            err[r, k] = np.nan if exact[r][k] is None else float(exact[r][k])
    kbest = np.zeros(R, dtype=np.int64)
    for r in range(R):
        keys = [float("inf") if x is None else x for x in exact[r]]     # NaN counts as +inf
        kbest[r] = min(range(K), key=lambda j: (keys[j], j))           # ties: smaller k
    with np.errstate(over="ignore", invalid="ignore"):
        scale = (alphas[kbest] * s0).astype(np.float32)
    tz, bad, nonfinite, xrange = _project_rows(v, scale, had_block, core_bound)
    status = 0
    if bad.any():
        status |= STATUS_BAD_SCALE
    if nonfinite.any():
        status |= STATUS_NONFINITE
    if xrange.any():
        status |= STATUS_X_RANGE
    tz = tz.reshape(-1, 8)
    core_idx = core_rank(tz, core_bound).astype(np.uint16)
    return {"scale": scale, "k": kbest, "err": err, "err_exact": exact, "two_z": tz, "core_idx": core_idx,
            "status": status}
