"""Pins for the oracle's PTQ initialization: the finite-core search against
exact rational distances, the finite-core projection's agreement with the
unconstrained projection inside the core, the exact row error against plain
Fraction arithmetic and the float64 weight-space error, the scale choice on a
constructed exact tie and near tie (where float64 sums disagree with each
other), and the scale search recovering an exact lattice scale."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from ptq_cases import tie_row


def _exact_best(x, pts):
    """Lowest-rank point of pts (2z, rank order) minimizing the exact ||x - t/2||^2."""
    xf = [Fraction(float(v)) for v in x]
    best, arg = None, None
    for i, t in enumerate(pts):
        d = sum((xi - Fraction(int(ti), 2)) ** 2 for xi, ti in zip(xf, t))
        if best is None or d < best:
            best, arg = d, i
    return pts[arg]


@pytest.mark.parametrize("bound", [8, 16])
def test_core_search_is_the_exact_nearest_core_point(bound):
    rng = np.random.default_rng(bound)
    pts = oracle.core_points(bound)
    x = np.concatenate([rng.normal(size=(40, 8)) * 2.5,          # mostly outside the core
                        rng.normal(size=(20, 8)) * 0.6,
                        np.round(rng.normal(size=(10, 8)) * 2) / 2 + 0.25]).astype(np.float32)
    got = oracle.core_search_two_z(x, bound)
    for i in range(len(x)):
        assert np.array_equal(got[i], _exact_best(x[i], pts)), i


def test_core_projection_matches_the_projection_inside_the_core():
    rng = np.random.default_rng(1)
    x = (rng.normal(size=(5000, 8)) * 0.7).astype(np.float32)
    tz = oracle.core_project_two_z(x, 16)
    free = oracle.nearest_e8_two_z(x)
    inside = (free * free).sum(1) <= 16
    assert inside.mean() > 0.5 and (~inside).sum() > 50
    assert np.array_equal(tz[inside], free[inside])
    assert ((tz * tz).sum(1) <= 16).all()
    assert oracle.is_e8_two_z(tz).all()
    # outside: no core point is nearer (exact check on a sample)
    pts = oracle.core_points(16)
    for i in np.nonzero(~inside)[0][:30]:
        assert np.array_equal(tz[i], _exact_best(x[i], pts))


def _fraction_error(v_row, s, t_row, hb):
    """sum (kappa v - s t/2)^2 in Fractions, term by term."""
    k = Fraction(float(oracle.kappa(hb)))
    sf = Fraction(float(np.float32(s)))
    return sum(((k * Fraction(float(x)) - sf * Fraction(int(t), 2)) ** 2 for x, t in zip(v_row, t_row)),
               Fraction(0))


@pytest.mark.parametrize("hb", [0, 64, 128])
def test_exact_row_error_against_fractions(hb):
    """Rows of ordinary, tiny (subnormal) and huge values; points from the
    projection and arbitrary small integers; a non-finite row gives None."""
    rng = np.random.default_rng(10 + hb)
    rows, cols = 5, 128
    v = (rng.standard_normal((rows, cols)) * 0.05).astype(np.float32)
    v[1, :4] = [1e-45, -3e-42, 7e-39, 1e-30]
    v[2] = (rng.standard_normal(cols) * 2.0 ** rng.integers(-100, 100, cols)).astype(np.float32)
    v[3, 7] = np.inf
    s = np.array([0.01, 2.0 ** -130, 3.0e10, 0.5, 1e-3], np.float32)
    tz = rng.integers(-6, 7, size=(rows, cols // 8, 8))
    got = oracle.exact_row_errors(v, s, tz, hb)
    for r in range(rows):
        if r == 3:
            assert got[r] is None
            continue
        assert got[r] == _fraction_error(v[r], s[r], tz[r].reshape(-1), hb), r


@pytest.mark.parametrize("hb,rtol", [(0, 1e-12), (64, 1e-6), (128, 1e-5)])
def test_row_error_is_the_weight_space_error(hb, rtol):
    """Exact up to float64 rounding without rotation; with it, within the
    float32 rounding of the transform (and of kappa_b when b is not 4^k)."""
    rng = np.random.default_rng(2)
    rows, cols = 6, 512
    w = (rng.normal(size=(rows, cols)) * 0.02).astype(np.float32)
    sig = np.where(rng.integers(0, 2, cols) == 1, 1, -1).astype(np.int8) if hb else None
    s = oracle.rms_scale(w, 1.5)
    out = oracle.project(w[None], s, sig, hb, w_is_bf16=False)
    v = w if not hb else oracle.fwht_blocks(w * sig.astype(np.float32), hb)
    tz = out["two_z"].reshape(rows, cols // 8, 8)
    e = np.array([float(x) for x in oracle.exact_row_errors(v.astype(np.float32), s, tz, hb)])
    W = oracle.exact_restored(tz.reshape(1, rows, cols), s, sig, hb)[0]
    plain = ((w.astype(np.float64) - W) ** 2).sum(1)
    assert np.allclose(e, plain, rtol=rtol, atol=0)


def _float64_sums(w, alphas):
    """Each candidate's float64 terms (exact here: no rotation, products of
    float32 values near 1) summed forward and in reverse."""
    v = w.reshape(-1).astype(np.float64)
    fwd, rev = [], []
    for a in alphas:
        tz = oracle.core_project_two_z(w.reshape(-1, 8), 16).reshape(-1)
        d = v - float(a) * 0.5 * tz
        q = (d * d).tolist()
        fwd.append(sum(q))
        rev.append(sum(q[::-1]))
    return fwd, rev


def test_scale_choice_on_a_constructed_exact_tie():
    """Exactly equal errors (tie: the smaller k) that float64 sums in forward
    and reverse order rank in opposite ways."""
    w, s0, al = tie_row()
    out = oracle.ptq_init(w, s0, al, None, 0, 16, w_is_bf16=False)
    e = [_fraction_error(w.reshape(-1), np.float32(a), out["two_z"].reshape(-1), 0) for a in al]
    assert e[0] == e[1] and out["err_exact"][0] == e
    fwd, rev = _float64_sums(w, al)
    assert (fwd[0] < fwd[1]) != (rev[0] < rev[1]) or (fwd[0] == fwd[1]) != (rev[0] == rev[1])
    assert out["k"][0] == 0 and out["scale"][0] == al[0]


def test_scale_choice_on_a_constructed_near_tie():
    """E_0 - E_1 = 2^-46 exactly (closed form of the construction), half a
    float64 ulp of E: the second candidate wins, though a float64 sum in one
    of the two orders ranks it last."""
    w, s0, al = tie_row(eta_units=1)
    out = oracle.ptq_init(w, s0, al, None, 0, 16, w_is_bf16=False)
    e = out["err_exact"][0]
    assert e[0] - e[1] == Fraction(1, 2 ** 46)
    assert 128 < e[1] < 256                     # float64 ulp 2^-45
    fwd, rev = _float64_sums(w, al)
    assert not (fwd[0] > fwd[1] and rev[0] > rev[1])
    assert out["k"][0] == 1 and out["scale"][0] == al[1]
    # the points are the same at both scales
    for a in al:
        tz = oracle.core_project_two_z((w.reshape(-1, 8) / np.float32(a)).astype(np.float32), 16)
        assert np.array_equal(tz, out["two_z"])


def test_scale_search_recovers_an_exact_lattice_scale():
    """Weights that are exactly s_true * z (z in the core, b = 64 so kappa is
    exact) give error 0 at the candidate s_true, which must win."""
    rng = np.random.default_rng(3)
    rows, cols, hb = 8, 256, 64
    pts = oracle.core_points(16)
    tz = pts[rng.integers(0, len(pts), size=rows * cols // 8)].reshape(rows, cols)
    sig = np.where(rng.integers(0, 2, cols) == 1, 1, -1).astype(np.int8)
    s_true = np.full(rows, 2.0 ** -5, np.float32)
    w = oracle.exact_restored(tz[None], s_true, sig, hb)[0]
    w32 = w.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), w)
    s0 = np.full(rows, 2.0 ** -6, np.float32)
    alphas = np.array([1.0, 1.5, 2.0, 2.5, 3.0], np.float32)
    out = oracle.ptq_init(w32[None], s0, alphas, sig, hb, 16, w_is_bf16=False)
    assert (out["k"] == 2).all()
    assert (out["err"][:, 2] == 0).all() and (out["err"][:, [0, 1, 3, 4]] > 0).all()
    assert np.array_equal(out["two_z"].reshape(rows, cols), tz)
    assert out["status"] == 0
    assert np.array_equal(oracle.core_unrank(out["core_idx"].astype(np.int64), 16), out["two_z"])


def test_scale_search_invalid_rows():
    rng = np.random.default_rng(4)
    w = (rng.normal(size=(1, 4, 128)) * 0.02).astype(np.float32)
    s0 = oracle.rms_scale(w[0], 1.0)
    w[0, 1, 5] = np.nan
    s0[2] = 0.0
    out = oracle.ptq_init(w, s0, np.array([1.0, 2.0], np.float32), None, 0, 16, w_is_bf16=False)
    assert np.isnan(out["err"][1]).all() and np.isinf(out["err"][2]).all()
    assert out["k"][1] == 0 and out["k"][2] == 0
    assert out["status"] == (oracle.STATUS_NONFINITE | oracle.STATUS_BAD_SCALE)
    assert (out["two_z"].reshape(4, 16, 8)[2] == 0).all()


def test_nan_error_counts_as_infinite():
    """A row whose errors are [inf (bad scale), NaN (non-finite weights)] ties at
    +inf and keeps the first candidate."""
    rng = np.random.default_rng(5)
    w = (rng.normal(size=(1, 2, 64)) * 0.02).astype(np.float32)
    s0 = oracle.rms_scale(w[0], 1.0)
    w[0, 1, 3] = np.nan
    out = oracle.ptq_init(w, s0, np.array([0.0, 1.0], np.float32), None, 0, 16, w_is_bf16=False)
    assert np.isinf(out["err"][1, 0]) and np.isnan(out["err"][1, 1])
    assert out["k"][1] == 0 and out["k"][0] == 1
