"""Pins for the oracle's Hadamard rotation, scale handling and finite core."""

import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle


# --------------------------------------------------------------- Hadamard

@pytest.mark.parametrize("b", [8, 16, 32, 64, 128, 256, 1024, 4096])
def test_fwht_matches_dense_sylvester(b):
    rng = np.random.default_rng(b)
    v = rng.normal(size=(3, 2 * b)).astype(np.float32)
    got = oracle.fwht_blocks(v, b).astype(np.float64)
    H = oracle.sylvester_matrix(b)
    want = np.concatenate([v[:, :b].astype(np.float64) @ H.T, v[:, b:].astype(np.float64) @ H.T], axis=1)
    err = np.abs(got - want).max() / np.abs(want).max()
    assert err < 1e-6


@pytest.mark.parametrize("b", [8, 128, 4096])
def test_fwht_exact_on_integers(b):
    """Small integers make every float32 butterfly exact, so the result must equal
    the dense product exactly."""
    rng = np.random.default_rng(7)
    v = rng.integers(-50, 51, size=(2, b)).astype(np.float32)
    got = oracle.fwht_blocks(v, b)
    want = v.astype(np.float64) @ oracle.sylvester_matrix(b).T
    assert np.array_equal(got.astype(np.float64), want)


def test_fwht_involution_parseval_delta():
    b = 128
    rng = np.random.default_rng(8)
    v = rng.normal(size=(5, b)).astype(np.float32)
    w = oracle.fwht_blocks(v, b)
    back = oracle.fwht_blocks(w, b) / b
    assert np.allclose(back, v, rtol=0, atol=1e-5)
    assert np.allclose((w.astype(np.float64) ** 2).sum(1) / b, (v.astype(np.float64) ** 2).sum(1), rtol=1e-5)
    delta = np.zeros((1, b), np.float32)
    delta[0, 0] = 1
    assert (oracle.fwht_blocks(delta, b) == 1).all()
    const = np.ones((1, b), np.float32)
    out = oracle.fwht_blocks(const, b)
    assert out[0, 0] == b and (out[0, 1:] == 0).all()


def test_kappa():
    for k in range(0, 7):
        assert oracle.kappa(4 ** k) == np.float32(2.0 ** -k)
    assert oracle.kappa(128) == np.float32(1 / np.sqrt(128.0))
    assert oracle.kappa(0) == 1


# -------------------------------------------------------------- normalization

def _round_f32(fr):
    """Correct rounding of a positive Fraction to float32 (round half even),
    by integer arithmetic; independent of numpy's division."""
    assert fr > 0
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    while Fraction(2) ** e > fr:
        e -= 1
    while Fraction(2) ** (e + 1) <= fr:
        e += 1
    e = max(e, -126)
    scaled = fr / Fraction(2) ** (e - 23)
    q, r = divmod(scaled.numerator, scaled.denominator)
    if 2 * r > scaled.denominator or (2 * r == scaled.denominator and q & 1):
        q += 1
    return np.float32(float(Fraction(q) * Fraction(2) ** (e - 23)))


def test_reciprocal_scale_is_correctly_rounded():
    rng = np.random.default_rng(9)
    s = np.abs(rng.normal(size=300)).astype(np.float32) * np.float32(0.02) + np.float32(1e-6)
    c, bad = oracle.row_coefficients(s, 0)
    assert not bad.any()
    for si, ci in zip(s, c):
        assert ci == _round_f32(1 / Fraction(float(si)))
    c128, _ = oracle.row_coefficients(s, 128)
    k = oracle.kappa(128)
    for si, ci, c0 in zip(s, c128, c):
        assert ci == _round_f32(Fraction(float(k)) * Fraction(float(c0)))


def test_bad_scales_flagged():
    s = np.array([1.0, 0.0, -1.0, np.nan, np.inf, 1e-45, 3e38], dtype=np.float32)
    _, bad = oracle.row_coefficients(s, 0)
    assert bad.tolist() == [False, True, True, True, True, True, False]


def test_power_of_two_scale_divides_exactly():
    rng = np.random.default_rng(10)
    w = rng.normal(size=(1, 4, 64)).astype(np.float32)
    s = np.array([0.5, 0.25, 2.0, 0.125], dtype=np.float32)
    x, _, bad, row = oracle.normalized_groups(w, s, w_is_bf16=False)
    assert np.array_equal(x.reshape(4, 64), w[0] / s[:, None])


def test_rms_scale_closed_form():
    w = np.zeros((3, 16), np.float32)
    w[0] = 0.5
    w[1, ::2] = 3.0        # rms = 3 / sqrt(2)
    w[2] = -2.0
    s = oracle.rms_scale(w, alpha=3.0)
    assert s[0] == np.float32(1.5)
    assert s[1] == np.float32(3 * 3 / np.sqrt(2))
    assert s[2] == np.float32(6.0)


def test_workload_scale_matches_oracle_definition():
    import torch
    from bit_e8_lattice_amd import workloads
    w = workloads.normal((1, 64, 256), 123, "cpu")
    got = workloads.rms_scale(w, 3.0).numpy()
    want = oracle.rms_scale(w.float().numpy().reshape(64, 256), 3.0)
    ulps = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1


# ------------------------------------------------------------------- bf16

def test_bf16_conversions_match_torch():
    import torch
    rng = np.random.default_rng(11)
    f = np.concatenate([rng.normal(size=5000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 5000),
                        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, 1e-40], np.float32)]).astype(np.float32)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(f), want)
    back = oracle.bf16_to_f32(want)
    assert np.array_equal(back, torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())
    assert oracle.f32_to_bf16(np.array([np.nan], np.float32))[0] == 0x7FC0


# ------------------------------------------------------------------- core

def _sigma3(n):
    return sum(d ** 3 for d in range(1, n + 1) if n % d == 0)


@pytest.mark.parametrize("bound", [0, 8, 16, 24, 32, 40])
def test_core_size_is_e8_theta_series(bound):
    """|C(B)| = 1 + sum_{1 <= n <= B/8} 240 sigma_3(n): E8 has 240 sigma_3(n) vectors
    of norm 2n, i.e. ||2z||^2 = 8n (SPLAG ch. 4 sec. 8.3)."""
    want = 1 + sum(240 * _sigma3(n) for n in range(1, bound // 8 + 1))
    assert oracle.core_size(bound) == want


def test_core_order_against_plain_enumeration():
    """B = 8: list the whole box with itertools, keep E8 points of the ball,
    sort the tuples; must equal the oracle's core in the same order."""
    pts = [t for t in itertools.product(range(-2, 3), repeat=8)
           if sum(v * v for v in t) <= 8 and len({v & 1 for v in t}) == 1 and sum(t) % 4 == 0]
    pts.sort()
    assert np.array_equal(oracle.core_points(8), np.array(pts))


@pytest.mark.parametrize("bound", [8, 16, 40])
def test_core_codec_round_trip(bound):
    """Every index decodes to a core point and encodes back to itself (the
    'core decoding agreement' check of E8-QAT Table 3, applied to this core)."""
    n = oracle.core_size(bound)
    idx = np.arange(n)
    pts = oracle.core_unrank(idx, bound)
    assert oracle.is_e8_two_z(pts).all()
    assert ((pts * pts).sum(1) <= bound).all()
    assert np.array_equal(oracle.core_rank(pts, bound), idx)
    keys = [tuple(p) for p in pts]
    assert all(keys[i] < keys[i + 1] for i in range(len(keys) - 1))


def test_core_rank_rejects_outside_points():
    far = np.array([[4, 4, 0, 0, 0, 0, 0, 0], [3, 3, 1, 1, 1, 1, 1, 1]])
    assert (oracle.core_rank(far, 16) == -1).all()
    assert oracle.core_size(16) <= 0xFFFF


# ------------------------------------------------------------------- accounting

def test_payload_table10(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "payload_table10.json")))
    for row in g["rows"]:
        b = oracle.payload_bits(row["rho"], record_bytes=g["record_bytes"])
        assert abs((b - 2) - row["delta_b"]) <= 0.5e-3 * row["delta_b"] + 1e-9
        assert abs(b - row["b_payload"]) <= 1e-6


def test_escape_fraction_tables_3_4_9(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "escape_accounting.json")))
    rho = oracle.escape_fraction(g["escaped_groups_375_step_artifact"],
                                 g["quantized_weights"] // g["group_size"])
    assert abs(rho - g["rho_table9_step375"]) < 0.5e-9
    # per-weight would be 8x smaller and not match Table 9
    assert abs(rho / 8 - g["rho_table9_step375"]) > 1e-6
    assert g["core_codewords_table3"] == 2 ** 16
