"""Constructed PTQ rows whose candidate errors tie exactly or nearly.

Input generators only (no part of the method's arithmetic): one row, no
rotation, scales s_0 = 1 and s_1 = 1 + 2^-22 (float32 neighbours two ulps
apart), midpoint s* = 1 + 2^-23.  64 groups are the half-integer E8 points
z = (+-1/2)^8 scaled by s* (exact in float32), perturbed by +-j 2^-24 in pairs
of groups so that sum_g v_g . z_g = s* sum_g ||z_g||^2; 1024 groups are small
(|v_i| < 0.245, inside the Voronoi cell of the origin at both scales).  Both
candidates then project every group to the same point, and with
P = sum v.z, N = sum ||z||^2,
    E_0 - E_1 = (s_0 - s_1) ((s_0 + s_1) N - 2 P) = 0.
``eta_units = 1`` moves one coordinate by 2^-24 along z (v.z grows by 2^-25),
which makes E_0 - E_1 = 2^-21 * 2^-25 = 2^-46 exactly: the second candidate
is better, by far less than one float64 ulp of E (about 160).
"""

import numpy as np

ALPHAS = np.array([1.0, 1.0 + 2.0 ** -22], np.float32)
TIE_SEED = 12          # a seed whose float64 sums in forward and reverse order rank the candidates differently


def tie_row(seed=TIE_SEED, eta_units=0, small_groups=1024, z_groups=64):
    rng = np.random.default_rng(seed)
    sstar = 1.0 + 2.0 ** -23
    ulp = 2.0 ** -24
    G = small_groups + z_groups
    v = np.zeros((G, 8), np.float64)
    zset = set(rng.permutation(G)[:z_groups].tolist())
    zs = []
    for g in range(G):
        if g in zset:
            sg = np.where(rng.integers(0, 2, 8) == 1, -1.0, 1.0)
            if (sg < 0).sum() % 2:
                sg[0] = -sg[0]
            v[g] = sstar * 0.5 * sg
            zs.append((g, sg))
        else:
            v[g] = rng.uniform(-0.245, 0.245, 8).astype(np.float32)
    for (g1, s1), (g2, s2) in zip(zs[0::2], zs[1::2]):
        j = int(rng.integers(1, 1 << 12))
        v[g1, 0] += j * ulp * s1[0]
        v[g2, 0] -= j * ulp * s2[0]
    v[zs[0][0], 2] += eta_units * ulp * zs[0][1][2]
    v32 = v.astype(np.float32)
    assert np.array_equal(v32.astype(np.float64), v)
    return v32.reshape(1, 1, G * 8), np.ones(1, np.float32), ALPHAS.copy()
