"""Pins for the oracle's projection, encoding, invalid-data rules, STE and SGD."""

import numpy as np
import pytest

import oracle


def _bf16_matrix(rng, batch, rows, cols, std=0.02):
    f = (rng.normal(size=(batch, rows, cols)) * std).astype(np.float32)
    return oracle.f32_to_bf16(f)


def test_project_dequant_is_s_times_z():
    rng = np.random.default_rng(20)
    w = _bf16_matrix(rng, 2, 8, 128)
    s = np.full(16, 0.015625, np.float32)              # power of two: q / s exact
    signs = rng.choice([-1, 1], size=128).astype(np.int8)
    out = oracle.project(w, s, signs, 32, core_bound=16)
    z = out["two_z"].reshape(2, 8, 128) / 2.0
    assert np.array_equal(out["q_f32"].astype(np.float64) / 0.015625, z)
    import torch
    want = torch.from_numpy(out["q_f32"]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out["q_bf16"], want)
    assert out["status"] == 0
    norms = (out["two_z"] ** 2).sum(1).reshape(2, -1)
    assert out["esc_count"].tolist() == (norms > 16).sum(1).tolist()


def test_rotated_values_are_orthonormal_rotation():
    rng = np.random.default_rng(21)
    w = _bf16_matrix(rng, 1, 4, 256)
    signs = rng.choice([-1, 1], size=256).astype(np.int8)
    s = np.ones(4, np.float32)
    out = oracle.project(w, s, signs, 128)
    v = oracle.bf16_to_f32(w).astype(np.float64)[0] * signs
    H = oracle.sylvester_matrix(128) / np.sqrt(128)
    want = np.concatenate([v[:, :128] @ H.T, v[:, 128:] @ H.T], axis=1)
    assert np.abs(out["u"][0] - want).max() <= 1e-6 * np.abs(want).max()


def test_encode_decode_round_trip_and_order():
    rng = np.random.default_rng(22)
    w = _bf16_matrix(rng, 3, 16, 256)
    s = oracle.rms_scale(oracle.bf16_to_f32(w).reshape(48, 256), 1.3)
    signs = rng.choice([-1, 1], size=256).astype(np.int8)
    enc = oracle.encode_core_escape(w, s, signs, 128, core_bound=16)
    proj = oracle.project(w, s, signs, 128)
    assert np.array_equal(enc["two_z"], proj["two_z"])
    norms = (enc["two_z"] ** 2).sum(1)
    esc = norms > 16
    assert enc["counts"].sum() == esc.sum() > 0
    assert (enc["core_idx"][esc] == oracle.ESCAPE_SLOT).all()
    assert (enc["core_idx"][~esc] != oracle.ESCAPE_SLOT).all()
    dec = oracle.decode_core_escape(enc["core_idx"], enc["records"], enc["counts"], 16)
    assert np.array_equal(dec, enc["two_z"])
    assert oracle.ESCAPE_RECORD_DTYPE.itemsize == 20
    # records ascend within every batch item
    off = np.concatenate([[0], np.cumsum(enc["counts"])])
    for b in range(3):
        g = enc["records"]["group"][off[b]:off[b + 1]]
        assert (np.diff(g.astype(np.int64)) > 0).all()


def test_escape_capacity_truncates_in_order():
    rng = np.random.default_rng(23)
    w = _bf16_matrix(rng, 1, 8, 128)
    s = oracle.rms_scale(oracle.bf16_to_f32(w).reshape(8, 128), 1.0)
    full = oracle.encode_core_escape(w, s, None, 0, core_bound=8)
    n = len(full["records"])
    assert n > 10
    cut = oracle.encode_core_escape(w, s, None, 0, core_bound=8, esc_capacity=n - 5)
    assert cut["status"] & oracle.STATUS_ESC_OVERFLOW
    assert np.array_equal(cut["records"], full["records"][:n - 5])
    assert np.array_equal(cut["counts"], full["counts"])


def test_invalid_data_rules():
    w = np.zeros((1, 4, 16), np.float32)
    w[0, 0, :] = 1.0
    w[0, 1, 3] = np.nan
    w[0, 2, :] = 0.25
    w[0, 2, 9] = 1e6
    w[0, 3, :] = 0.5
    s = np.array([1.0, 1.0, 1.0, 0.0], np.float32)
    out = oracle.project(w, s, w_is_bf16=False)
    st = out["status"]
    assert st & oracle.STATUS_BAD_SCALE and st & oracle.STATUS_NONFINITE and st & oracle.STATUS_X_RANGE
    tz = out["two_z"].reshape(4, 2, 8)
    assert (tz[1, 0] == 0).all() and not (tz[1, 1] != 0).any()     # NaN group -> 0
    assert (tz[2, 1] == 0).all()                                    # huge group -> 0
    assert (tz[3] == 0).all() and (out["q_f32"][0, 3] == 0).all()   # bad row -> 0
    assert not np.signbit(out["q_f32"]).any()


def test_int8_saturation_flag():
    w = np.zeros((1, 1, 8), np.float32)
    w[0, 0, 0] = 100.0
    w[0, 0, 1] = 100.0
    out = oracle.project(w, np.ones(1, np.float32), w_is_bf16=False)
    assert out["two_z"][0, 0] == 200
    assert out["two_z_i8"][0, 0, 0] == 127
    assert out["status"] & oracle.STATUS_INT8_RANGE
    enc = oracle.encode_core_escape(w, np.ones(1, np.float32), core_bound=16, w_is_bf16=False)
    assert enc["records"]["two_z"][0, 0] == 200                     # records stay exact


def test_ste_identity_and_sgd():
    import torch
    rng = np.random.default_rng(24)
    g = _bf16_matrix(rng, 1, 4, 64, std=1e-4)
    assert np.array_equal(oracle.ste_backward(g), g)
    w = _bf16_matrix(rng, 1, 4, 64)
    new = oracle.sgd_update(w, g, 1.0)
    wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).float()
    gt = torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).float()
    want = (wt - 1.0 * gt).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(new, want)
    assert np.array_equal(oracle.sgd_update(w, np.zeros_like(w), 0.5), w)
    assert (oracle.bf16_to_f32(oracle.sgd_update(w, w, 1.0)) == 0).all()
    wf = oracle.bf16_to_f32(w)
    assert np.array_equal(oracle.sgd_update(wf, wf, 0.5, is_bf16=False), wf - np.float32(0.5) * wf)
