"""Pins for the oracle's nearest-E8 decoder against facts it does not use itself:
exhaustive search (brute force), lattice membership, the covering radius, the
normalized second moment of E8, and hand-worked special vectors."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.brute import brute_nearest_e8


def _adversarial(rng):
    """Near-tie inputs: exact half-integers, quarter values, deep holes, lattice
    points, and their +-1 ulp neighbours."""
    base = [
        [1, 0, 0, 0, 0, 0, 0, 0],            # deep hole of E8
        [0.25] * 8,                          # coset tie (0 vs (1/2)^8)
        [0.5, 0.5, 0, 0, 0, 0, 0, 0],        # RNE tie
        [0.5] * 8,
        [0.75] * 8,
        [1.5, -0.5, 0.5, 0.5, -1.5, 0.5, 0.5, 0.5],
        [-0.25, 0.25, -0.25, 0.25, -0.25, 0.25, -0.25, 0.25],
        [0.5, -0.5, 0.5, -0.5, 0.5, -0.5, 0.5, 0.5],
        [1, 1, 0, 0, 0, 0, 0, 0],
        [2.5, 0.5, 0.5, 0.5, 0.5, 0.5, 0.5, 0.5],
        [-1e-30, 0, 0, 0, 0, 0, 0, 0],
        [0.3, 0.3, 0.3, 0.3, 0.3, 0.3, 0.3, 0.3],
        [0.49999997, 0.5, 0.50000006, 0, 0, 0, 0, 1],
    ]
    xs = []
    for b in base:
        b = np.array(b, dtype=np.float32)
        xs.append(b)
        for i in range(8):
            for d in (np.float32(np.inf), np.float32(-np.inf)):
                v = b.copy()
                v[i] = np.nextafter(v[i], d)
                xs.append(v)
    # random half/quarter grids produce many exact ties
    xs.append((rng.integers(-8, 9, size=(400, 8)) / 4).astype(np.float32))
    return np.vstack(xs)


def _check_against_brute(x):
    tz = oracle.nearest_e8_two_z(x)
    d2, best = brute_nearest_e8(x)
    bad = [i for i in range(len(x)) if tuple(int(t) for t in tz[i]) not in best[i]]
    assert not bad, f"not a nearest point for rows {bad[:5]}: x={x[bad[0]]} got {tz[bad[0]]} want one of {best[bad[0]]}"
    return tz, d2, best


def test_brute_force_random_gaussian():
    rng = np.random.default_rng(1)
    x = np.vstack([rng.normal(size=(600, 8)), rng.normal(scale=1 / 3, size=(300, 8)),
                   rng.normal(scale=4.0, size=(300, 8))]).astype(np.float32)
    _check_against_brute(x)


def test_brute_force_adversarial_ties():
    rng = np.random.default_rng(2)
    _check_against_brute(_adversarial(rng))


@pytest.mark.slow
def test_brute_force_all_groups_of_small_workload():
    """Every one of the 8,192 groups of the 256x256 float32 workload."""
    import torch
    from bit_e8_lattice_amd import workloads
    b = workloads.small_f32("cpu")
    x, _, bad, _ = oracle.normalized_groups(b.w.numpy(), b.scale.numpy(), w_is_bf16=False)
    assert not bad.any()
    assert x.shape == (8192, 8)
    _check_against_brute(x)


def test_outputs_are_lattice_points():
    rng = np.random.default_rng(3)
    x = np.vstack([rng.normal(scale=s, size=(20000, 8)) for s in (0.1, 1, 10, 500)]).astype(np.float32)
    tz = oracle.nearest_e8_two_z(x)
    assert oracle.is_e8_two_z(tz).all()


def test_membership_rule_on_known_points():
    good = [[0] * 8, [2, 2, 0, 0, 0, 0, 0, 0], [1] * 8, [-1, 1, 1, 1, 1, 1, 1, -1],
            [3, 1, 1, 1, 1, 1, 1, -1], [4, 0, 0, 0, 0, 0, 0, 0]]
    bad = [[2, 0, 0, 0, 0, 0, 0, 0], [1, 1, 1, 1, 1, 1, 1, -1], [1, 1, 0, 0, 0, 0, 0, 0],
           [3, 1, 1, 1, 1, 1, 1, 1]]
    assert oracle.is_e8_two_z(np.array(good)).all()
    assert not oracle.is_e8_two_z(np.array(bad)).any()


def test_idempotent_on_lattice_points():
    rng = np.random.default_rng(4)
    t = 2 * rng.integers(-20, 21, size=(5000, 8))
    t[:, 0] += 2 * (((t // 2).sum(axis=1)) % 2)          # make sum(z) even
    h = 2 * rng.integers(-20, 21, size=(5000, 8)) + 1
    h[:, 0] += 2 * (((h.sum(axis=1) % 4) != 0).astype(np.int64))
    pts = np.vstack([t, h])
    assert oracle.is_e8_two_z(pts).all()
    x = (pts / 2).astype(np.float32)
    assert (oracle.nearest_e8_two_z(x) == pts).all()


def test_covering_radius_one():
    """E8 (minimal norm 2) has covering radius 1: every x is within distance 1."""
    rng = np.random.default_rng(5)
    x = rng.uniform(-6, 6, size=(200000, 8)).astype(np.float32)
    tz = oracle.nearest_e8_two_z(x)
    d2 = ((x.astype(np.float64) - tz / 2.0) ** 2).sum(axis=1)
    assert d2.max() <= 1.0 + 1e-12
    # deep hole: exactly distance 1
    deep = np.array([[1, 0, 0, 0, 0, 0, 0, 0]], dtype=np.float32)
    tz = oracle.nearest_e8_two_z(deep)
    assert sum((Fraction(float(a)) - Fraction(int(b), 2)) ** 2 for a, b in zip(deep[0], tz[0])) == 1


def test_second_moment_matches_e8():
    """Mean squared error per dimension for uniform input equals the normalized
    second moment of E8, G = 929/12960 (unit-volume lattice, SPLAG ch. 2/21)."""
    rng = np.random.default_rng(6)
    x = rng.uniform(-40, 40, size=(400000, 8)).astype(np.float32)
    tz = oracle.nearest_e8_two_z(x)
    mse = (((x.astype(np.float64) - tz / 2.0) ** 2).sum(axis=1) / 8).mean()
    assert abs(mse - 929 / 12960) < 4e-4


def test_special_vectors_tie_rules():
    # deep hole: 16 nearest points at distance 1; the tie rules pick (2, 0^7)
    x = np.array([[1, 0, 0, 0, 0, 0, 0, 0]], dtype=np.float32)
    d2, best = brute_nearest_e8(x)
    assert d2[0] == 1 and len(best[0]) == 16
    assert tuple(oracle.nearest_e8_two_z(x)[0]) == (4, 0, 0, 0, 0, 0, 0, 0)
    # (1/4)^8 is equidistant from 0 and (1/2)^8: a zero difference keeps D8
    x = np.full((1, 8), 0.25, dtype=np.float32)
    d2, best = brute_nearest_e8(x)
    assert (0,) * 8 in best[0] and (1,) * 8 in best[0]
    assert (oracle.nearest_e8_two_z(x) == 0).all()
    # (1/2, 1/2, 0^6): 0 and (1, 1, 0^6) tie; rint ties to even -> 0
    x = np.array([[0.5, 0.5, 0, 0, 0, 0, 0, 0]], dtype=np.float32)
    assert (oracle.nearest_e8_two_z(x) == 0).all()
    # one ulp above 1/2 in both leading coordinates breaks the tie towards (1,1,0^6)
    up = np.nextafter(np.float32(0.5), np.float32(1))
    x = np.array([[up, up, 0, 0, 0, 0, 0, 0]], dtype=np.float32)
    assert tuple(oracle.nearest_e8_two_z(x)[0]) == (2, 2, 0, 0, 0, 0, 0, 0)


def test_tiny_negative_coordinate_picks_near_half_point():
    """x = (-2^-30, 0.5^7...) style inputs: the half-integer next to a tiny
    negative coordinate is -1/2, not +1/2 (the literal D8(x - 1/2) + 1/2 form
    gets this wrong in float32)."""
    x = np.array([[-2.0 ** -30, 0.5, 0.5, 0.5, 0.5, 0.5, 0.5, 0.5]], dtype=np.float32)
    tz = oracle.nearest_e8_two_z(x)
    d2, best = brute_nearest_e8(x)
    assert tuple(int(t) for t in tz[0]) in best[0]
