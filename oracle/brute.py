"""Exact nearest E8 point by exhaustive search of the local neighbourhood.

This is the check for ``lattice.nearest_e8_two_z`` and shares none of its
reasoning: it lists every E8 point in a box around ``x`` and measures every
distance.  E8 has covering radius 1 [SPLAG ch. 4 sec. 8.1], so a nearest point
``y`` satisfies ``|x_i - y_i| <= 1`` in every coordinate.  Integer coordinates
within 1 of ``x_i`` lie in ``{r-1, r, r+1}`` with ``r = rint(x_i)``;
half-integer ones lie in ``{f-1/2, f+1/2, f+3/2}`` with ``f = floor(x_i)``.
All 2 x 3^8 combinations are listed, non-lattice ones dropped (parity), and the
distances are computed in float64 to screen, then exactly with ``Fraction`` for
every candidate within a relative 1e-9 of the screened minimum.

Slow by design: intended for a few thousand groups.
"""

from fractions import Fraction
import itertools

import numpy as np

_OFF = np.array(list(itertools.product((-1, 0, 1), repeat=8)), dtype=np.int64)


def _exact_d2(xrow, two_y):
    return sum((Fraction(float(xi)) - Fraction(int(ti), 2)) ** 2
               for xi, ti in zip(xrow, two_y))


def brute_nearest_e8(x, chunk=32):
    """For each row of ``x`` (float32 [G, 8], finite) return ``(d2, best)``:
    the exact minimum squared distance to E8 (a list of ``Fraction``) and the
    list of all minimizers as ``2z`` tuples."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, 8)
    x64 = x.astype(np.float64)
    d2_out, best_out = [], []
    for lo in range(0, x.shape[0], chunk):
        xs = x64[lo:lo + chunk]
        base_int = 2 * np.rint(xs).astype(np.int64)                # 2r
        base_half = 2 * np.floor(xs).astype(np.int64) + 1          # 2f + 1
        cand = np.concatenate(
            [base_int[:, None, :] + 2 * _OFF[None], base_half[:, None, :] + 2 * _OFF[None]],
            axis=1)                                                 # [c, 2*6561, 8]
        member = (cand.sum(axis=2) % 4) == 0                        # one parity per coset already
        diff = xs[:, None, :] - 0.5 * cand
        d = (diff * diff).sum(axis=2)
        d = np.where(member, d, np.inf)
        dmin = d.min(axis=1)
        for j in range(xs.shape[0]):
            near = np.nonzero(d[j] <= dmin[j] * (1 + 1e-9) + 1e-300)[0]
            exact = [(_exact_d2(x[lo + j], cand[j, c]), tuple(int(t) for t in cand[j, c]))
                     for c in near]
            m = min(e for e, _ in exact)
            best = sorted({t for e, t in exact if e == m})
            d2_out.append(m)
            best_out.append(best)
    return d2_out, best_out
