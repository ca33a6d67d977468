"""Nearest point of the E8 lattice, written out as the textbook decoder.

E8 is the union of two cosets: D8 (integer vectors with an even coordinate sum)
and D8 + 1/2 (the same shifted by one half in every coordinate)  [SPLAG ch. 4
sec. 8.1].  E8-QAT replaces a stored codebook by this lattice and maps each group
of eight normalized coordinates to a lattice point by arithmetic alone
[E8-QAT, abstract; Figure 1(c) and Figure 2(b) captions].

The decoder is the one of [CS82] / [SPLAG ch. 20]: find the nearest point of
each coset (round every coordinate; if the parity is wrong, re-round the worst
coordinate the other way) and keep the nearer of the two.  It is written in
terms of quantities that are exact in float32 so that the result is a pure
function of the float32 input bits:

* ``n_i = rint(x_i)`` (round half to even), ``a_i = |x_i - n_i|`` (exact),
  ``s_i = +1 if x_i >= n_i else -1``;
* the nearest integer vector is ``n``; the nearest half-integer vector is
  ``n + s/2`` (the half-integer next to ``x_i`` on the side of ``x_i``);
* D8 candidate: if ``sum(n)`` is odd, move coordinate ``k`` (largest ``a``) by
  ``s_k`` -- the cheapest re-rounding, costing ``1 - 2 a_k``;
* D8+1/2 candidate: if ``sum(2y)`` is not a multiple of 4, move coordinate
  ``m`` (smallest ``a``) by ``-s_m`` -- costing ``2 a_m``;
* the squared-distance difference of the two candidates is exactly
  ``sum(a) - 2 + [odd0](1 - 2 a_k) - [odd1] 2 a_m``; it is evaluated in float64
  in one fixed order (exact whenever every non-zero ``a_i`` is at least 2^-26),
  and the D8 candidate wins when it is <= 0.

Tie rules (a reading: the pages give none; parity unpinned beyond brute-force
optimality): rint ties go to even; ``s_i = +1`` when ``x_i`` is an integer;
``k`` / ``m`` are the lowest index among equal ``a``; a zero difference picks D8.

Lattice points are returned as ``2z`` (integers), which is exact for both cosets.
"""

import numpy as np


def nearest_e8_two_z(x):
    """Return ``2z`` (int64, shape [G, 8]) for the nearest E8 point of each row of ``x``.

    ``x`` is float32 [G, 8], finite.  Follows [CS82] / [SPLAG ch. 20] with the
    tie rules in the module docstring.
    """
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, 8)
    if not np.isfinite(x).all():
        raise ValueError("nearest_e8_two_z needs finite input")
    g = x.shape[0]
    rows = np.arange(g)

    n = np.rint(x)                       # float32, round half to even
    a = np.abs(x - n)                    # exact in float32
    s = np.where(x >= n, 1, -1).astype(np.int64)
    n_int = n.astype(np.int64)

    # Nearest point of D8.
    y0 = 2 * n_int
    odd0 = (n_int.sum(axis=1) & 1) == 1
    k = np.argmax(a, axis=1)             # first (lowest) index of the largest a
    y0[rows[odd0], k[odd0]] += 2 * s[rows[odd0], k[odd0]]

    # Nearest point of D8 + 1/2 (all arithmetic on 2y).
    y1 = 2 * n_int + s
    odd1 = (y1.sum(axis=1) % 4) != 0
    m = np.argmin(a, axis=1)             # first (lowest) index of the smallest a
    y1[rows[odd1], m[odd1]] -= 2 * s[rows[odd1], m[odd1]]

    # Which coset point is nearer: float64, fixed evaluation order.
    a64 = a.astype(np.float64)
    total = ((a64[:, 0] + a64[:, 1]) + (a64[:, 2] + a64[:, 3])) + \
            ((a64[:, 4] + a64[:, 5]) + (a64[:, 6] + a64[:, 7]))
    t = total - 2.0
    t = np.where(odd0, t + (1.0 - 2.0 * a64[rows, k]), t)
    t = np.where(odd1, t - 2.0 * a64[rows, m], t)
    return np.where((t <= 0.0)[:, None], y0, y1)


def is_e8_two_z(two_z):
    """Membership test on ``2z`` [SPLAG ch. 4 sec. 8.1].

    ``z`` is in E8 iff all ``2z_i`` are even (z in Z^8) or all are odd
    (z in Z^8 + 1/2), and ``sum(z)`` is even, i.e. ``sum(2z) = 0 mod 4``.
    """
    t = np.asarray(two_z, dtype=np.int64).reshape(-1, 8)
    par = t & 1
    same_coset = (par == par[:, :1]).all(axis=1)
    return same_coset & ((t.sum(axis=1) % 4) == 0)
