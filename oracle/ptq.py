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
  (equal to the weight-space error, the rotation being orthogonal) is
  ``E = sum_g sum_i d_gi^2`` with ``d = fl64(kappa_b * v) - s_k * z`` (``v`` the
  un-normalized transform, ``kappa_b`` the float32 value, every product exact
  in float64, one rounding per subtraction and square, group sums in the fixed
  pairwise order), summed over the groups of the row as 64 interleaved partial
  sums (group g into partial g mod 64, in increasing g) combined by a butterfly
  (offsets 32, 16, ..., 1); the candidate with the smallest E wins, NaN counts
  as +inf, ties go to the smaller k, a candidate whose scale is invalid (the
  projection's bad-row rule) has E = +inf.
"""

import numpy as np

from .core import core_points, core_rank
from .hadamard import fwht_blocks, kappa
from .lattice import nearest_e8_two_z
from .pipeline import (STATUS_BAD_SCALE, STATUS_NONFINITE, STATUS_X_RANGE, X_LIMIT, _shape3, _widen,
                       row_coefficients)

LANES = 64


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


def row_error(v, s, tz, had_block):
    """E per row (float64 [R]) for rows ``v`` [R, cols], scales ``s`` [R] and
    points ``tz`` [R, cols/8, 8], in the fixed order of the module docstring."""
    rows, cols = v.shape
    gpr = cols // 8
    k64 = np.float64(kappa(had_block))
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        d = k64 * v.astype(np.float64).reshape(rows, gpr, 8) - s64[:, None, None] * (0.5 * tz.astype(np.float64))
        q = d * d
        e = ((q[..., 0] + q[..., 1]) + (q[..., 2] + q[..., 3])) + ((q[..., 4] + q[..., 5]) + (q[..., 6] + q[..., 7]))
    part = np.zeros((rows, LANES), dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        for g in range(gpr):
            part[:, g % LANES] = part[:, g % LANES] + e[:, g]
        lanes = np.arange(LANES)
        off = LANES // 2
        while off >= 1:
            part = part + part[:, lanes ^ off]
            off //= 2
    return part[:, 0]


def ptq_init(w, s0, alphas, signs=None, had_block=0, core_bound=16, w_is_bf16=True):
    """Per-row scale search and finite-core projection.

    ``w`` [batch, rows, cols] (bf16 bits or float32), ``s0`` float32
    [batch*rows], ``alphas`` float32 [K].  Returns a dict with ``scale``
    (float32 [batch*rows]), ``k`` (int64), ``err`` (float64 [batch*rows, K]),
    ``two_z`` (int64 [G, 8]), ``core_idx`` (uint16 [G]) and ``status``.
    """
    batch, rows, cols = _shape3(w)
    v = _rotated(w, signs, had_block, w_is_bf16).reshape(batch * rows, cols)
    s0 = np.asarray(s0, dtype=np.float32).reshape(-1)
    alphas = np.asarray(alphas, dtype=np.float32)
    K = len(alphas)
    err = np.zeros((batch * rows, K), dtype=np.float64)
    for k in range(K):
        with np.errstate(over="ignore", invalid="ignore"):
            sk = (alphas[k] * s0).astype(np.float32)
        tz, bad, _, _ = _project_rows(v, sk, had_block, core_bound)
        e = row_error(v, sk, tz, had_block)
        err[:, k] = np.where(bad, np.inf, e)
    key = np.where(np.isnan(err), np.inf, err)
    kbest = np.argmin(key, axis=1)
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
    return {"scale": scale, "k": kbest.astype(np.int64), "err": err, "two_z": tz, "core_idx": core_idx,
            "status": status}
