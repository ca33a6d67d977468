"""GPU parity of e8q_decode_core_escape: the oracle's exported form decoded on
the device must equal the oracle's decode bit for bit (2z, q, restored
weights, status); and the device's own encode followed by its decode must give
back the oracle's projection of the original weights."""

import numpy as np
import pytest
import torch

import oracle
from bit_e8_lattice_amd import workloads
from gpu_util import (device, first_mismatch, run_decode, run_encode, run_project, run_restore,
                      upload_export, wbits)

pytestmark = pytest.mark.gpu


def _cmp(out, ref, q=None, w_hat=None):
    if "two_z_i8" in out:
        assert first_mismatch(out["two_z_i8"], ref["two_z_i8"]) is None
    if q is not None:
        key = "q_bf16" if q == torch.bfloat16 else "q_f32"
        want = ref[key] if q == torch.bfloat16 else ref[key].view(np.uint32)
        got = out["q"] if q == torch.bfloat16 else out["q"].view(np.uint32)
        m = first_mismatch(got, want)
        assert m is None, f"q: {m}"
    if w_hat is not None:
        key = "w_hat_bf16" if w_hat == torch.bfloat16 else "w_hat_f32"
        want = ref[key] if w_hat == torch.bfloat16 else ref[key].view(np.uint32)
        got = out["w_hat"] if w_hat == torch.bfloat16 else out["w_hat"].view(np.uint32)
        m = first_mismatch(got, want)
        assert m is None, f"w_hat: {m}"
    assert out["status"] == ref["status"], (out["status"], ref["status"])


@pytest.mark.parametrize("bound", [0, 8, 16, 24, 31, 40])
@pytest.mark.parametrize("alpha", [1.0, 3.0])
def test_decode_oracle_export(bound, alpha):
    """Point table in LDS (small bounds) and in global memory (large ones);
    alpha 1 gives thousands of records to search."""
    d = device()
    shape = (3, 29, 256)
    w = workloads.normal(shape, 1200 + bound, d)
    s = workloads.rms_scale(w, alpha)
    sg = workloads.signs(256, 1201, d)
    sn = sg.cpu().numpy()
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sn, 128, bound)
    ref = oracle.decode_outputs(enc["core_idx"], enc["records"], enc["counts"], bound, shape,
                                s.cpu().numpy(), sn, 128)
    core, esc, cnt = upload_export(enc, d)
    for qd, wd in ((torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32)):
        out = run_decode(core, esc, cnt, shape, bound, s, sg, 128, q_dtype=qd, w_hat_dtype=wd)
        _cmp(out, ref, qd, wd)
    out = run_decode(core, esc, cnt, shape, bound)
    _cmp(out, oracle.decode_outputs(enc["core_idx"], enc["records"], enc["counts"], bound, shape))


@pytest.mark.parametrize("hb", [8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_decode_restore_every_block(hb):
    d = device()
    cols = max(hb, 512)
    shape = (2, 13, cols)
    w = workloads.normal(shape, 1300 + hb, d)
    s = workloads.rms_scale(w, 1.5)
    sg = workloads.signs(cols, 1301 + hb, d)
    sn = sg.cpu().numpy()
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sn, hb, 16)
    ref = oracle.decode_outputs(enc["core_idx"], enc["records"], enc["counts"], 16, shape,
                                s.cpu().numpy(), sn, hb)
    core, esc, cnt = upload_export(enc, d)
    out = run_decode(core, esc, cnt, shape, 16, s, sg, hb, q_dtype=torch.bfloat16, w_hat_dtype=torch.bfloat16)
    _cmp(out, ref, torch.bfloat16, torch.bfloat16)


def test_decode_malformed_exports():
    """Truncated record list, an index past the core, a record for a slot that
    is not escaped, and rows with invalid scales."""
    d = device()
    shape = (2, 16, 128)
    w = workloads.normal(shape, 1400, d)
    s = workloads.rms_scale(w, 1.0)
    sg = workloads.signs(128, 1401, d)
    sn = sg.cpu().numpy()
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sn, 64, 16)
    core_np = enc["core_idx"].copy()
    k = int(np.nonzero(core_np != oracle.ESCAPE_SLOT)[0][3])
    core_np[k] = oracle.core_size(16) + 5
    e = int(np.nonzero(core_np == oracle.ESCAPE_SLOT)[0][1])
    core_np[e] = 7
    s_bad = s.clone()
    s_bad[3] = float("nan")
    s_bad[20] = -2.0
    recs = enc["records"][:-5]
    bad_enc = {"core_idx": core_np, "records": recs, "counts": enc["counts"]}
    ref = oracle.decode_outputs(core_np, recs, enc["counts"], 16, shape, s_bad.cpu().numpy(), sn, 64)
    assert ref["status"] == (oracle.STATUS_ESC_MISSING | oracle.STATUS_BAD_INDEX | oracle.STATUS_BAD_SCALE)
    core, esc, cnt = upload_export(bad_enc, d)
    out = run_decode(core, esc, cnt, shape, 16, s_bad, sg, 64, q_dtype=torch.float32, w_hat_dtype=torch.float32)
    _cmp(out, ref, torch.float32, torch.float32)
    # the same list cut by the capacity argument instead of by length
    core2, esc2, cnt2 = upload_export(enc, d)
    out = run_decode(core2, esc2, cnt2, shape, 16, esc_records=len(enc["records"]) - 5)
    ref2 = oracle.decode_outputs(enc["core_idx"], enc["records"][:-5], enc["counts"], 16, shape)
    _cmp(out, ref2)


def test_decode_int8_saturation_from_records():
    """Escape records with |2z| > 127 saturate in the int8 output only."""
    d = device()
    shape = (1, 8, 64)
    w = workloads.normal(shape, 1500, d, dtype=torch.float32)
    s = workloads.rms_scale(w, 0.01)     # |x| ~ 100: large escaped points
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), None, 0, 16, w_is_bf16=False)
    assert np.abs(enc["two_z"]).max() > 127
    ref = oracle.decode_outputs(enc["core_idx"], enc["records"], enc["counts"], 16, shape, s.cpu().numpy())
    core, esc, cnt = upload_export(enc, d)
    out = run_decode(core, esc, cnt, shape, 16, s, q_dtype=torch.float32)
    _cmp(out, ref, torch.float32)


def test_device_encode_then_decode_matches_projection():
    """Dense-decoder shapes, all three launches at full size as the benchmark
    runs them: the device's encode then decode must give back the oracle's
    projection (q and restored weights) of the original weights on sampled rows,
    and the device's own projection everywhere."""
    d = device()
    rng = np.random.default_rng(1)
    for b in workloads.dense_decoder(d):
        nb, rows, cols = b.w.shape
        shape = (nb, rows, cols)
        enc = run_encode(b.w, b.scale, 16, b.signs, 128, keep_device=True)
        core, esc, cnt = enc["dev"]
        out = run_decode(core, esc, cnt, shape, 16, b.scale, b.signs, 128, two_z=False,
                         q_dtype=None, w_hat_dtype=torch.bfloat16)
        assert out["status"] == 0
        for m in (0, nb - 1):
            rsel = np.unique(np.concatenate([[0, rows - 1], rng.integers(0, rows, 3)]))
            ref = oracle.project_restore(wbits(b.w[m])[rsel], b.scale[m * rows:(m + 1) * rows].cpu().numpy()[rsel],
                                         b.signs.cpu().numpy(), 128)
            got = out["w_hat"].reshape(shape)[m][rsel]
            assert first_mismatch(got, ref["w_hat_bf16"][0]) is None
        full = run_restore(b.w, b.scale, b.signs, 128, two_z=False)
        assert first_mismatch(out["w_hat"], full["w_hat"]) is None
        del enc, core, esc, cnt, out, full
        torch.cuda.empty_cache()


@pytest.mark.parametrize("bound", [0, 16, 40])
@pytest.mark.parametrize("alpha", [1.0, 3.0])
def test_decode_restore_only(bound, alpha):
    """Restored weights as the only output with 128-wide blocks (point table
    in LDS, and in global memory for C(40)); alpha 1 escapes most groups."""
    d = device()
    shape = (3, 37, 512)
    w = workloads.normal(shape, 1600 + bound, d)
    s = workloads.rms_scale(w, alpha)
    sg = workloads.signs(512, 1601, d)
    sn = sg.cpu().numpy()
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sn, 128, bound)
    ref = oracle.decode_outputs(enc["core_idx"], enc["records"], enc["counts"], bound, shape,
                                s.cpu().numpy(), sn, 128)
    core, esc, cnt = upload_export(enc, d)
    for wd in (torch.bfloat16, torch.float32):
        out = run_decode(core, esc, cnt, shape, bound, s, sg, 128, two_z=False, w_hat_dtype=wd)
        _cmp(out, ref, None, wd)


def test_decode_restore_only_large_escapes_and_malformed():
    """Restored weights only, with escaped points far outside bfloat16's exact
    integers (|2z| > 256), an index past the core, a missing record and
    invalid row scales."""
    d = device()
    shape = (2, 21, 256)
    w = workloads.normal(shape, 1610, d, dtype=torch.float32)
    s = workloads.rms_scale(w, 1.0)
    s = s * 0.004                              # |x| ~ 2000 after the rotation
    sg = workloads.signs(256, 1611, d)
    sn = sg.cpu().numpy()
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sn, 128, 16, w_is_bf16=False)
    assert np.abs(enc["two_z"]).max() > 256
    core_np = enc["core_idx"].copy()
    k = int(np.nonzero(core_np != oracle.ESCAPE_SLOT)[0][0]) if (core_np != oracle.ESCAPE_SLOT).any() else 0
    core_np[k] = oracle.core_size(16) + 3
    s_bad = s.clone()
    s_bad[4] = float("nan")
    s_bad[30] = -1.0
    recs = enc["records"][:-4]
    bad_enc = {"core_idx": core_np, "records": recs, "counts": enc["counts"]}
    ref = oracle.decode_outputs(core_np, recs, enc["counts"], 16, shape, s_bad.cpu().numpy(), sn, 128,
                                want_two_z=False)
    assert ref["status"] == (oracle.STATUS_ESC_MISSING | oracle.STATUS_BAD_INDEX | oracle.STATUS_BAD_SCALE)
    core, esc, cnt = upload_export(bad_enc, d)
    for wd in (torch.bfloat16, torch.float32):
        out = run_decode(core, esc, cnt, shape, 16, s_bad, sg, 128, two_z=False, w_hat_dtype=wd)
        _cmp(out, ref, None, wd)


@pytest.mark.parametrize("where", ["first_rows", "last_rows", "one_row", "two_ends"])
def test_decode_clustered_escapes(where):
    """Escape records bunched in a few rows of each batch item (the record
    search's interpolated probes land far from them and it falls back to
    halving): decoded 2z, q and restored weights still match the oracle."""
    d = device()
    shape = (3, 40, 512)
    w = workloads.normal(shape, 4321, d, dtype=torch.float32)
    s = workloads.rms_scale(w, 3.0)
    rows = {"first_rows": slice(0, 3), "last_rows": slice(37, 40), "one_row": slice(20, 21),
            "two_ends": [0, 39]}[where]
    w[:, rows, ::5] = 6.0 * s.view(3, 40, 1)[:, rows, :]
    sg = workloads.signs(512, 4322, d)
    sn = sg.cpu().numpy()
    wb = wbits(w)
    enc = oracle.encode_core_escape(wb, s.cpu().numpy(), sn, 128, 16, w_is_bf16=False)
    assert enc["counts"].min() > 10
    ref = oracle.decode_outputs(enc["core_idx"], enc["records"], enc["counts"], 16, shape, s.cpu().numpy(), sn, 128)
    core, esc, cnt = upload_export(enc, d)
    out = run_decode(core, esc, cnt, shape, 16, s, sg, 128, q_dtype=torch.float32, w_hat_dtype=torch.float32)
    _cmp(out, ref, torch.float32, torch.float32)
