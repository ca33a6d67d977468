"""Pins for the oracle's decoder: the exported form decodes to exactly what the
projection computes (2z, q, restored weights), and malformed exports are
flagged."""

import numpy as np
import pytest

import oracle


def _weights(rng, batch, rows, cols, alpha):
    w = (rng.standard_t(4, size=(batch, rows, cols)) * 0.02 / np.sqrt(2)).astype(np.float32)
    s = oracle.rms_scale(w.reshape(batch * rows, cols), alpha)
    return w, s


@pytest.mark.parametrize("bound", [0, 8, 16, 40])
@pytest.mark.parametrize("alpha", [1.0, 3.0])
def test_decode_reproduces_the_projection(bound, alpha):
    rng = np.random.default_rng(bound + int(alpha * 10))
    batch, rows, cols, hb = 3, 9, 256, 128
    w, s = _weights(rng, batch, rows, cols, alpha)
    sig = np.where(rng.integers(0, 2, cols) == 1, 1, -1).astype(np.int8)
    enc = oracle.encode_core_escape(w, s, sig, hb, bound, w_is_bf16=False)
    dec = oracle.decode_outputs(enc["core_idx"], enc["records"], enc["counts"], bound,
                                (batch, rows, cols), s, sig, hb)
    prj = oracle.project_restore(w, s, sig, hb, w_is_bf16=False)
    assert np.array_equal(dec["two_z"], prj["two_z"])
    assert np.array_equal(dec["q_bf16"], prj["q_bf16"])
    assert np.array_equal(dec["q_f32"].view(np.uint32), prj["q_f32"].view(np.uint32))
    assert np.array_equal(dec["w_hat_f32"].view(np.uint32), prj["w_hat_f32"].view(np.uint32))
    assert np.array_equal(dec["two_z_i8"], prj["two_z_i8"])
    assert dec["status"] == 0
    if alpha == 1.0 and bound <= 16:
        assert len(enc["records"]) > 0


def test_decode_flags_malformed_exports():
    rng = np.random.default_rng(9)
    batch, rows, cols = 2, 8, 128
    w, s = _weights(rng, batch, rows, cols, 1.0)
    enc = oracle.encode_core_escape(w, s, None, 0, 16, w_is_bf16=False)
    recs, counts, core = enc["records"], enc["counts"], enc["core_idx"].copy()
    assert counts.min() > 2
    shape = (batch, rows, cols)
    # a truncated record list: the tail of the last batch item has no record
    cut = oracle.decode_outputs(core, recs[:-2], counts, 16, shape)
    assert cut["status"] == oracle.STATUS_ESC_MISSING
    missing = recs[-2:]["group"].astype(np.int64) + (batch - 1) * (rows * cols // 8)
    assert (cut["two_z"][missing] == 0).all()
    # an index past the core
    bad = core.copy()
    k = int(np.nonzero(bad != oracle.ESCAPE_SLOT)[0][0])
    bad[k] = oracle.core_size(16)
    out = oracle.decode_outputs(bad, recs, counts, 16, shape)
    assert out["status"] == oracle.STATUS_BAD_INDEX and (out["two_z"][k] == 0).all()
    # a record for a slot that is not escaped is ignored
    stray = core.copy()
    e = int(np.nonzero(stray == oracle.ESCAPE_SLOT)[0][0])
    stray[e] = 0
    out = oracle.decode_outputs(stray, recs, counts, 16, shape)
    assert out["status"] == 0
    assert np.array_equal(out["two_z"][e], oracle.core_unrank(np.array([0]), 16)[0])


def test_decode_bad_scale_rows():
    rng = np.random.default_rng(10)
    shape = (1, 4, 128)
    w, s = _weights(rng, *shape, 3.0)
    sig = np.where(rng.integers(0, 2, 128) == 1, 1, -1).astype(np.int8)
    enc = oracle.encode_core_escape(w, s, sig, 64, 16, w_is_bf16=False)
    s2 = s.copy()
    s2[1] = np.nan
    s2[2] = -1.0
    out = oracle.decode_outputs(enc["core_idx"], enc["records"], enc["counts"], 16, shape, s2, sig, 64)
    assert out["status"] == oracle.STATUS_BAD_SCALE
    assert (out["q_f32"][0, 1:3] == 0).all() and not np.signbit(out["q_f32"][0, 1:3]).any()
    assert np.array_equal(np.signbit(out["w_hat_f32"][0, 1:3]), np.broadcast_to(sig < 0, (2, 128)))


@pytest.mark.parametrize("hb", [0, 8, 128, 512])
def test_gemv_reference_is_the_restored_product(hb):
    """The float64 GEMV reference equals the oracle's float32 restored weights
    times x up to the rounding of those weights, and its exact weights are the
    restore's values before that rounding."""
    rng = np.random.default_rng(40 + hb)
    batch, rows, cols, m = 2, 12, 1024, 3
    w, s = _weights(rng, batch, rows, cols, 1.5)
    sig = np.where(rng.integers(0, 2, cols) == 1, 1, -1).astype(np.int8) if hb else None
    prj = oracle.project_restore(w, s, sig, hb, w_is_bf16=False) if hb else oracle.project(w, s, w_is_bf16=False)
    two_z = prj["two_z"].reshape(batch, rows, cols)
    W = oracle.exact_restored(two_z, s, sig, hb)
    w32 = prj["w_hat_f32"] if hb else prj["q_f32"]
    assert np.all(np.abs(W - w32) <= 2.0 ** -21 * np.abs(W))
    x = rng.normal(size=(batch, m, cols))
    y, mag = oracle.gemv_reference(two_z, s, x, sig, hb)
    want = np.einsum("brc,btc->btr", w32.astype(np.float64), x)
    assert np.all(np.abs(y - want) <= 2.0 ** -20 * mag)
    # the rotated-basis form s * sum z . x_tilde (x_tilde = H_b (sigma x) / sqrt(b))
    # gives the same product
    if hb:
        H = oracle.sylvester_matrix(hb)
        xt = ((x * sig).reshape(batch, m, cols // hb, hb) @ H.T).reshape(batch, m, cols) / np.sqrt(hb)
        y2 = np.einsum("brc,btc->btr", two_z * 0.5 * s.reshape(batch, rows, 1).astype(np.float64), xt)
        assert np.allclose(y2, y, rtol=0, atol=1e-12 * mag.max())
        rmag = oracle.rotated_magnitude(two_z, s, x, sig, hb)
        assert (rmag >= np.abs(y2) - 1e-12).all()


@pytest.mark.parametrize("hb", [0, 8, 128])
def test_rotated_bound_covers_the_rotated_activations(hb):
    """rotated_bound (the GEMV tolerance's xbar) bounds every |x_tilde_i| of the
    rotated activation H_b (sigma x) / sqrt(b) computed densely in float64, and
    is attained at position 0 of a block whose signed entries are all
    non-negative (that row of H_b is all ones)."""
    rng = np.random.default_rng(70 + hb)
    batch, m, cols = 2, 3, 512
    x = rng.normal(size=(batch, m, cols))
    sig = np.where(rng.integers(0, 2, cols) == 1, 1, -1).astype(np.int8) if hb else None
    xbar = oracle.rotated_bound(x, sig, hb)
    if hb:
        H = oracle.sylvester_matrix(hb)
        xt = ((x * sig).reshape(batch, m, cols // hb, hb) @ H.T).reshape(batch, m, cols) / np.sqrt(hb)
    else:
        xt = x
    assert (xbar >= np.abs(xt) * (1 - 1e-12)).all()
    if hb:
        y = np.abs(x) * sig                     # sigma * y >= 0 everywhere
        xb = oracle.rotated_bound(y, sig, hb)
        first = ((y * sig).reshape(batch, m, cols // hb, hb) @ oracle.sylvester_matrix(hb).T)[..., 0] / np.sqrt(hb)
        assert np.allclose(xb.reshape(batch, m, cols // hb, hb)[..., 0], first, rtol=1e-12, atol=0)
    else:
        assert np.array_equal(xbar, np.abs(x))
