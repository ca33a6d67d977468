"""The finite 2-bit core: a ball of E8 points and its dense index.

E8-QAT stores each group as a 16-bit index into a fixed finite core of lattice
points and keeps groups that leave the core as sparse exact records [E8-QAT,
abstract; Figure 2(c) caption; Figure 6(c) caption gives the payload
2 + 20 rho bits per weight].  The pages do not say how their 65,536-point core
is built.  Reading taken here (parity unpinned: any bijection would satisfy the
pages):

* core ``C(B) = { z in E8 : ||2z||^2 <= B }`` with an integer bound ``B``
  (0 <= B <= 40 so that |C(B)| <= 65,535 fits a 16-bit slot with one value
  spare);
* the index of ``z`` is its position when ``C(B)`` is sorted lexicographically
  by ``2z`` as a signed tuple, coordinate 0 most significant;
* the spare slot value 0xFFFF marks a group stored as an escape record.

Everything is computed by enumeration, sorting and search.
"""

import numpy as np

ESCAPE_SLOT = 0xFFFF
MAX_CORE_BOUND = 40

_cache = {}


def core_points(bound):
    """All ``2z`` of ``C(bound)``, int64 [N, 8], sorted lexicographically.

    Enumeration: extend prefixes one coordinate at a time over the box
    ``|2z_i| <= floor(sqrt(bound))``, drop prefixes whose squared norm already
    exceeds the bound, and keep complete vectors that are E8 points
    (all coordinates of one parity, sum = 0 mod 4) [SPLAG ch. 4 sec. 8.1].
    """
    bound = int(bound)
    if bound < 0 or bound > MAX_CORE_BOUND:
        raise ValueError("core bound must be in [0, 40]")
    if bound in _cache:
        return _cache[bound]
    tmax = int(np.floor(np.sqrt(bound)))
    vals = np.arange(-tmax, tmax + 1, dtype=np.int64)
    pts = vals[:, None]
    for _ in range(7):
        ext = np.concatenate(
            [np.repeat(pts, len(vals), axis=0),
             np.tile(vals, len(pts))[:, None]], axis=1)
        # a prefix survives if it still fits the ball and keeps one parity
        ok = ((ext * ext).sum(axis=1) <= bound) & ((ext[:, -1] & 1) == (ext[:, 0] & 1))
        pts = ext[ok]
    par = pts & 1
    keep = (par == par[:, :1]).all(axis=1) & ((pts.sum(axis=1) % 4) == 0)
    pts = pts[keep]
    order = np.lexsort(pts.T[::-1])      # last key is primary -> coordinate 0
    pts = pts[order]
    _cache[bound] = pts
    return pts


def core_size(bound):
    return int(core_points(bound).shape[0])


def _keys(t, tmax):
    """Map signed tuples with |t_i| <= tmax to integers that sort like the tuples."""
    base = 2 * tmax + 1
    k = np.zeros(t.shape[0], dtype=np.int64)
    for i in range(8):
        k = k * base + (t[:, i] + tmax)
    return k


def core_rank(two_z, bound):
    """Dense lexicographic index of each ``2z`` in ``C(bound)``; -1 if outside."""
    pts = core_points(bound)
    t = np.asarray(two_z, dtype=np.int64).reshape(-1, 8)
    tmax = max(int(np.floor(np.sqrt(bound))), 0)
    inside = (t * t).sum(axis=1) <= bound
    out = np.full(t.shape[0], -1, dtype=np.int64)
    if inside.any():
        keys = _keys(pts, tmax)
        q = _keys(t[inside], tmax)
        pos = np.searchsorted(keys, q)
        pos_ok = np.minimum(pos, len(keys) - 1)
        hit = keys[pos_ok] == q
        res = np.where(hit, pos_ok, -1)
        out[inside] = res
    return out


def core_unrank(idx, bound):
    """Inverse of ``core_rank``: the ``2z`` stored at each index."""
    pts = core_points(bound)
    idx = np.asarray(idx, dtype=np.int64)
    if (idx < 0).any() or (idx >= len(pts)).any():
        raise ValueError("index outside the core")
    return pts[idx]
