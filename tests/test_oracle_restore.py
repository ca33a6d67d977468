"""Pins for the oracle's inverse rotation (restored weights) and the
rotated-basis gradient: dense products in float64, the exact round trip on
lattice points, and the adjoint identity against the forward rotation."""

import numpy as np
import pytest
import torch

import oracle


def _e8_two_z(rng, n, spread=3):
    """Random E8 points as 2z: 2y (+1 in the half-integer coset), sum(y) even."""
    y = rng.integers(-spread, spread + 1, size=(n, 8))
    y[:, 0] += y.sum(1) & 1
    half = rng.integers(0, 2, size=(n, 1))
    return 2 * y + half


def _signs(rng, cols):
    return np.where(rng.integers(0, 2, cols) == 1, 1, -1).astype(np.int8)


def _dense_rt(t, sig, b):
    """sigma * (H_b t) / sqrt(b) per block, float64 (t: [rows, cols])."""
    H = oracle.sylvester_matrix(b)
    rows, cols = t.shape
    blk = t.reshape(rows, cols // b, b).astype(np.float64) @ H.T
    return blk.reshape(rows, cols) / np.sqrt(float(b)) * sig.astype(np.float64)


@pytest.mark.parametrize("b", [8, 32, 128, 512, 4096])
def test_restore_matches_dense_product(b):
    rng = np.random.default_rng(b)
    rows, cols = 6, max(2 * b, 256)
    two_z = _e8_two_z(rng, rows * cols // 8).reshape(rows, cols)
    s = rng.uniform(0.01, 0.2, rows).astype(np.float32)
    sig = _signs(rng, cols)
    got = oracle.restore_original(two_z, s, sig, b).astype(np.float64)
    want = _dense_rt(two_z * 0.5 * s.astype(np.float64)[:, None], sig, b)
    # one rounding of T * c2, c2 rounded twice, kappa_b rounded once: < 4 ulp
    assert np.all(np.abs(got - want) <= 2.0 ** -21 * np.abs(want))


@pytest.mark.parametrize("b", [16, 64, 256, 1024, 4096])
def test_restore_inverts_the_forward_on_lattice_points(b):
    """For b = 4^k (kappa exact) and a power-of-two scale, w = R^T (s z) is exact
    in float32; projecting it must give z back and restoring must give w back,
    bit for bit."""
    rng = np.random.default_rng(100 + b)
    rows, cols = 5, 2 * b if b >= 128 else 256
    two_z = _e8_two_z(rng, rows * cols // 8, spread=2).reshape(rows, cols)
    s = np.full(rows, 2.0 ** -6, np.float32)
    sig = _signs(rng, cols)
    w = _dense_rt(two_z * 0.5 * 2.0 ** -6, sig, b)
    w32 = w.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), w)
    out = oracle.project_restore(w32[None], s, sig, b, w_is_bf16=False)
    assert np.array_equal(out["two_z"].reshape(rows, cols), two_z)
    assert np.array_equal(out["w_hat_f32"][0], w32)


@pytest.mark.parametrize("b", [8, 128, 2048])
def test_rotate_grad_is_the_adjoint_of_the_forward_rotation(b):
    """<R w, g> = <w, R^T g> with R the forward rotation the projection uses."""
    rng = np.random.default_rng(200 + b)
    rows, cols = 4, 2 * b
    w = rng.normal(size=(rows, cols)).astype(np.float32)
    g = rng.normal(size=(rows, cols)).astype(np.float32)
    sig = _signs(rng, cols)
    u = oracle.project(w[None], np.ones(rows, np.float32), sig, b, w_is_bf16=False)["u"][0]
    rt = oracle.rotate_grad(g, sig, b, is_bf16=False)
    lhs = (u.astype(np.float64) * g).sum()
    rhs = (w.astype(np.float64) * rt).sum()
    assert abs(lhs - rhs) <= 1e-5 * np.sqrt((w.astype(np.float64) ** 2).sum() * (g.astype(np.float64) ** 2).sum())
    # and R^T R = I
    back = oracle.rotate_grad(u, sig, b, is_bf16=False)
    assert np.abs(back - w).max() < 1e-5


@pytest.mark.parametrize("b", [8, 64, 1024])
def test_rotate_grad_matches_dense_product(b):
    rng = np.random.default_rng(300 + b)
    g = rng.normal(size=(3, 2 * b)).astype(np.float32)
    sig = _signs(rng, 2 * b)
    got = oracle.rotate_grad(g, sig, b, is_bf16=False).astype(np.float64)
    want = _dense_rt(g, sig, b)
    assert np.abs(got - want).max() <= 1e-6 * np.abs(want).max()


def test_zero_signs_and_bad_rows():
    """Every zero is sigma * (+0); a row with an invalid scale restores to it."""
    rng = np.random.default_rng(5)
    cols, b = 128, 128
    sig = _signs(rng, cols)
    two_z = np.zeros((3, cols), np.int64)
    two_z[1, :8] = [2, 2, 0, 0, 0, 0, 0, 0]   # H of this has zeros in half the columns
    s = np.array([0.1, 0.1, 0.1], np.float32)
    bad = np.array([False, False, True])
    two_z[2] = _e8_two_z(rng, cols // 8).reshape(-1)
    out = oracle.restore_original(two_z, s, sig, b, bad)
    zero = out == 0
    assert zero[0].all() and zero[2].all() and zero[1].any() and not zero[1].all()
    assert np.array_equal(np.signbit(out[zero]), np.broadcast_to(sig < 0, out.shape)[zero])


def test_bf16_outputs_follow_torch_rounding():
    rng = np.random.default_rng(6)
    w = torch.randn(4, 256, dtype=torch.float32).mul(0.02)
    wb = w.bfloat16().view(torch.int16).numpy().view(np.uint16)
    s = oracle.rms_scale(oracle.bf16_to_f32(wb), 1.0)
    sig = _signs(rng, 256)
    out = oracle.project_restore(wb[None], s, sig, 128)
    want = torch.from_numpy(out["w_hat_f32"]).bfloat16().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out["w_hat_bf16"], want)
    # gradient + fused SGD against torch's float32 arithmetic and bf16 rounding
    g = torch.randn(4, 256).mul(1e-3).bfloat16()
    gb = g.view(torch.int16).numpy().view(np.uint16)
    gw, wn = oracle.ste_backward_hadamard(gb, sig, 128, True, wb, 0.5)
    g32 = torch.from_numpy(oracle.rotate_grad(gb, sig, 128))
    assert np.array_equal(gw, g32.bfloat16().view(torch.int16).numpy().view(np.uint16))
    ref = (torch.from_numpy(oracle.bf16_to_f32(wb)) - g32 * 0.5).bfloat16()
    assert np.array_equal(wn, ref.view(torch.int16).numpy().view(np.uint16))
