"""GPU GEMV from the exported form against the float64 product of the exact
restored weights, within the documented bound (the evaluation order is the
kernel's own, so the bar is a derived tolerance, not bit equality).  Rows of
a multiple of 256 columns with 16-byte aligned indices take the int8
matrix-core kernel (cores below 4096 points whose table and activation
digits fit in LDS) or the bfloat16 matrix-core kernel; other shapes and
alignments the vector kernel."""

import numpy as np
import pytest
import torch

import oracle
from bit_e8_lattice_amd import workloads
from gpu_util import device, gemv_tolerance, run_encode, run_gemv, upload_export, wbits

pytestmark = pytest.mark.gpu


def _x(shape, seed, d, dtype=torch.bfloat16):
    g = torch.Generator(device=d).manual_seed(seed)
    return torch.randn(shape, generator=g, device=d).to(dtype)


def _xvals(x):
    return x.float().cpu().numpy().astype(np.float64)


def _check(out, two_z, s, x, sig, hb, cols):
    xv = _xvals(x)
    y, _ = oracle.gemv_reference(two_z, s, xv, sig, hb)
    tol = gemv_tolerance(two_z, s, xv, sig, hb, cols)
    err = np.abs(out["y"] - y)
    assert (err <= tol).all(), f"max err/tol {np.max(err / np.maximum(tol, 1e-300)):.3g}"
    return y


@pytest.mark.parametrize("m", [1, 2, 4])
@pytest.mark.parametrize("hb", [0, 8, 128, 1024])
@pytest.mark.parametrize("alpha", [1.0, 3.0])
def test_gemv_oracle_export(m, hb, alpha):
    d = device()
    shape = (3, 70, 2048)
    w = workloads.normal(shape, 1600 + hb, d)
    s = workloads.rms_scale(w, alpha)
    sg = workloads.signs(2048, 1601, d) if hb else None
    sn = None if sg is None else sg.cpu().numpy()
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sn, hb, 16)
    core, esc, cnt = upload_export(enc, d)
    x = _x((3, m, 2048), 1602 + m, d)
    out = run_gemv(core, esc, cnt, shape, 16, s, x, sg, hb)
    assert out["status"] == 0
    _check(out, enc["two_z"].reshape(shape), s.cpu().numpy(), x, sn, hb, 2048)


@pytest.mark.parametrize("bound", [0, 24, 40])
def test_gemv_bounds_and_f32_activations(bound):
    """Cores below 4096 points (the int8 kernel, table in LDS) and of 9121 and
    56881 points (the bfloat16 kernel, table in global memory); float32
    activations."""
    d = device()
    shape = (2, 33, 4096)
    w = workloads.normal(shape, 1700 + bound, d)
    s = workloads.rms_scale(w, 2.0)
    sg = workloads.signs(4096, 1701, d)
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), 4096, bound)
    core, esc, cnt = upload_export(enc, d)
    x = _x((2, 1, 4096), 1702, d, torch.float32)
    out = run_gemv(core, esc, cnt, shape, bound, s, x, sg, 4096)
    assert out["status"] == 0
    _check(out, enc["two_z"].reshape(shape), s.cpu().numpy(), x, sg.cpu().numpy(), 4096, 4096)


def test_gemv_malformed_and_bad_scale():
    d = device()
    shape = (2, 16, 1024)
    w = workloads.normal(shape, 1800, d)
    s = workloads.rms_scale(w, 1.0)
    sg = workloads.signs(1024, 1801, d)
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), 128, 16)
    core_np = enc["core_idx"].copy()
    k = int(np.nonzero(core_np != oracle.ESCAPE_SLOT)[0][0])
    core_np[k] = oracle.core_size(16)
    s_bad = s.clone()
    s_bad[5] = 0.0
    bad = {"core_idx": core_np, "records": enc["records"][:-3], "counts": enc["counts"]}
    core, esc, cnt = upload_export(bad, d)
    x = _x((2, 2, 1024), 1802, d)
    out = run_gemv(core, esc, cnt, shape, 16, s_bad, x, sg, 128)
    assert out["status"] == (oracle.STATUS_BAD_INDEX | oracle.STATUS_ESC_MISSING | oracle.STATUS_BAD_SCALE)
    dec = oracle.decode_core_escape(core_np, bad["records"], enc["counts"], 16)
    sb = s_bad.cpu().numpy().copy()
    xv = _xvals(x)
    sref = np.where(sb > 0, sb, 0).astype(np.float32)
    yref, _ = oracle.gemv_reference(dec.reshape(shape), sref, xv, sg.cpu().numpy(), 128)
    tol = gemv_tolerance(dec.reshape(shape), sref, xv, sg.cpu().numpy(), 128, 1024)
    assert (np.abs(out["y"] - yref) <= tol).all()
    assert (out["y"][0, :, 5] == 0).all()


def test_gemv_dense_decoder_shapes():
    """All 224 dense-decoder matrices in the benchmark's three launches (one
    activation vector per matrix); the first, middle and last matrix of each
    launch checked in full against the float64 product of the projection of
    the original weights."""
    d = device()
    for i, b in enumerate(workloads.dense_decoder(d)):
        nb, rows, cols = b.w.shape
        shape = (nb, rows, cols)
        enc = run_encode(b.w, b.scale, 16, b.signs, 128, keep_device=True)
        core, esc, cnt = enc["dev"]
        x = _x((nb, 1, cols), 1900 + i, d)
        out = run_gemv(core, esc, cnt, shape, 16, b.scale, x, b.signs, 128)
        assert out["status"] == 0
        sn = b.signs.cpu().numpy()
        for mi in (0, nb // 2, nb - 1):
            sm = b.scale[mi * rows:(mi + 1) * rows].cpu().numpy()
            prj = oracle.project(wbits(b.w[mi]), sm, sn, 128)
            tz = prj["two_z"].reshape(1, rows, cols)
            o = {"y": out["y"][mi:mi + 1]}
            _check(o, tz, sm, x[mi:mi + 1], sn, 128, cols)
        del enc, core, esc, cnt
        torch.cuda.empty_cache()


@pytest.mark.parametrize("m", [1, 2, 4])
def test_gemv_vector_path_shapes(m):
    """Rows whose group count is not a multiple of 8 (1000 columns), and a
    16-byte misaligned index pointer: the vector kernel."""
    d = device()
    shape = (2, 37, 1000)
    w = workloads.normal(shape, 1750 + m, d)
    s = workloads.rms_scale(w, 1.0)
    sg = workloads.signs(1000, 1751, d)
    sn = sg.cpu().numpy()
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sn, 8, 16)
    core, esc, cnt = upload_export(enc, d)
    x = _x((2, m, 1000), 1752 + m, d)
    out = run_gemv(core, esc, cnt, shape, 16, s, x, sg, 8)
    assert out["status"] == 0
    _check(out, enc["two_z"].reshape(shape), s.cpu().numpy(), x, sn, 8, 1000)
    # the same 2048-column export through a misaligned copy of its indices
    shape = (1, 9, 2048)
    w = workloads.normal(shape, 1760 + m, d)
    s = workloads.rms_scale(w, 1.0)
    sg = workloads.signs(2048, 1761, d)
    sn = sg.cpu().numpy()
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sn, 128, 16)
    core, esc, cnt = upload_export(enc, d)
    buf = torch.empty(core.numel() + 1, dtype=core.dtype, device=d)
    buf[1:].copy_(core)
    x = _x((1, m, 2048), 1762 + m, d)
    out = run_gemv(buf[1:], esc, cnt, shape, 16, s, x, sg, 128)
    assert out["status"] == 0
    _check(out, enc["two_z"].reshape(shape), s.cpu().numpy(), x, sn, 128, 2048)


@pytest.mark.parametrize("m,cols", [(4, 4096), (2, 11008)])
def test_gemv_wide_activations(m, cols):
    """The widest activation shapes the call takes (four vectors of 4096
    columns, two of 11008): the int8 kernel keeps their digits in LDS beside
    the point table."""
    d = device()
    shape = (2, 45, cols)
    w = workloads.normal(shape, 1770 + m, d)
    s = workloads.rms_scale(w, 2.0)
    sg = workloads.signs(cols, 1771, d)
    sn = sg.cpu().numpy()
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sn, 128, 16)
    core, esc, cnt = upload_export(enc, d)
    x = _x((2, m, cols), 1772 + m, d)
    out = run_gemv(core, esc, cnt, shape, 16, s, x, sg, 128)
    assert out["status"] == 0
    _check(out, enc["two_z"].reshape(shape), s.cpu().numpy(), x, sn, 128, cols)


@pytest.mark.parametrize("rows", [1, 3, 17])
def test_gemv_matrix_core_few_rows(rows):
    """Fewer rows than one tile (and one past a tile): the lanes of missing
    rows repeat the last row and write nothing."""
    d = device()
    shape = (2, rows, 256)
    w = workloads.normal(shape, 1780 + rows, d)
    s = workloads.rms_scale(w, 1.0)
    sg = workloads.signs(256, 1781, d)
    sn = sg.cpu().numpy()
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sn, 128, 16)
    core, esc, cnt = upload_export(enc, d)
    x = _x((2, 2, 256), 1782 + rows, d)
    out = run_gemv(core, esc, cnt, shape, 16, s, x, sg, 128)
    assert out["status"] == 0
    _check(out, enc["two_z"].reshape(shape), s.cpu().numpy(), x, sn, 128, 256)


@pytest.mark.parametrize("where", ["first_rows", "last_rows", "two_ends"])
def test_gemv_clustered_escapes(where):
    """Escape records bunched in a few rows (the record search falls back from
    interpolated probes to halving), on the matrix-core path."""
    d = device()
    shape = (3, 40, 2048)
    w = workloads.normal(shape, 4331, d, dtype=torch.float32)
    s = workloads.rms_scale(w, 3.0)
    rows = {"first_rows": slice(0, 3), "last_rows": slice(37, 40), "two_ends": [0, 39]}[where]
    w[:, rows, ::7] = 6.0 * s.view(3, 40, 1)[:, rows, :]
    sg = workloads.signs(2048, 4332, d)
    sn = sg.cpu().numpy()
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sn, 128, 16, w_is_bf16=False)
    assert enc["counts"].min() > 10
    core, esc, cnt = upload_export(enc, d)
    x = _x((3, 1, 2048), 4333, d)
    out = run_gemv(core, esc, cnt, shape, 16, s, x, sg, 128)
    assert out["status"] == 0
    _check(out, enc["two_z"].reshape(shape), s.cpu().numpy(), x, sn, 128, 2048)


@pytest.mark.parametrize("cols", [1024, 1000])
def test_gemv_duplicate_and_unused_records(cols):
    """A record repeated (same key and point) counts once, and a record whose
    slot is a core index is ignored: y is the product of the original export
    and no status bit is set (matrix-core and vector kernels)."""
    d = device()
    shape = (2, 40, cols)
    w = workloads.normal(shape, 2100 + cols, d)
    s = workloads.rms_scale(w, 1.5)
    sg = workloads.signs(cols, 2101, d)
    sn = sg.cpu().numpy()
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sn, 8, 16)
    rec, counts, gpb = enc["records"], enc["counts"].copy(), 40 * cols // 8
    assert counts.min() >= 2
    parts = []
    off = 0
    for b in range(2):
        r = rec[off:off + counts[b]].copy()
        off += counts[b]
        # a duplicate of the second record, right after it
        r = np.concatenate([r[:2], r[1:2], r[2:]])
        # a record for a core slot of this item, at its sorted position
        core_slots = np.nonzero(enc["core_idx"][b * gpb:(b + 1) * gpb] != oracle.ESCAPE_SLOT)[0]
        extra = np.zeros(1, dtype=oracle.ESCAPE_RECORD_DTYPE)
        extra["group"] = core_slots[len(core_slots) // 2]
        extra["two_z"] = 2
        pos = int(np.searchsorted(r["group"], extra["group"][0]))
        r = np.concatenate([r[:pos], extra, r[pos:]])
        parts.append(r)
        counts[b] = len(r)
    bad = {"core_idx": enc["core_idx"], "records": np.concatenate(parts), "counts": counts}
    core, esc, cnt = upload_export(bad, d)
    x = _x((2, 1, cols), 2102, d)
    out = run_gemv(core, esc, cnt, shape, 16, s, x, sg, 8)
    assert out["status"] == 0
    _check(out, enc["two_z"].reshape(shape), s.cpu().numpy(), x, sn, 8, cols)


@pytest.mark.parametrize("m", [1, 2])
def test_gemv_deterministic(m):
    """Two runs give the same y bit for bit (escaped slots at 2 x RMS go through
    the per-row record sums; no atomics decide an order)."""
    d = device()
    shape = (4, 96, 4096)
    w = workloads.normal(shape, 2200 + m, d)
    s = workloads.rms_scale(w, 2.0)
    sg = workloads.signs(4096, 2201, d)
    enc = run_encode(w, s, 16, sg, 128, keep_device=True)
    core, esc, cnt = enc["dev"]
    assert int(cnt.sum()) > 0
    x = _x((4, m, 4096), 2202, d)
    a = run_gemv(core, esc, cnt, shape, 16, s, x, sg, 128)
    b = run_gemv(core, esc, cnt, shape, 16, s, x, sg, 128)
    assert a["status"] == 0 and b["status"] == 0
    assert np.array_equal(a["y"].view(np.uint64), b["y"].view(np.uint64))


def test_gemv_many_batch_items():
    """More than 1024 batch items on the matrix-core path: the escape blocks
    take their record ranges from the offsets scan."""
    d = device()
    shape = (1100, 16, 256)
    w = workloads.normal(shape, 2300, d)
    s = workloads.rms_scale(w, 1.5)
    sg = workloads.signs(256, 2301, d)
    sn = sg.cpu().numpy()
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sn, 128, 16)
    assert (enc["counts"] > 0).sum() > 1000
    core, esc, cnt = upload_export(enc, d)
    x = _x((1100, 1, 256), 2302, d)
    out = run_gemv(core, esc, cnt, shape, 16, s, x, sg, 128)
    assert out["status"] == 0
    _check(out, enc["two_z"].reshape(shape), s.cpu().numpy(), x, sn, 128, 256)


def test_gemv_int8_zero_nonfinite_and_wide_range_vectors():
    """The int8 kernel's fixed point per activation vector: an all-zero vector
    gives y = 0 exactly; a vector holding a NaN gives NaN rows and the
    NONFINITE bit while the other vectors stay within the bound; a vector with
    one entry 10^6 times the rest stays within the bound, whose fixed-point
    term grows with the vector's largest entry; a vector of float32
    subnormals (scale exponent about -130) stays within it too."""
    d = device()
    shape = (3, 40, 2048)
    w = workloads.normal(shape, 1900, d)
    s = workloads.rms_scale(w, 2.0)
    sg = workloads.signs(2048, 1901, d)
    sn = sg.cpu().numpy()
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sn, 128, 16)
    core, esc, cnt = upload_export(enc, d)
    x = _x((3, 2, 2048), 1902, d, torch.float32)
    x[0, 1] = 0.0
    x[1, 0, 77] = float("nan")
    x[2, 1, 1500] = 1.0e6
    x[2, 0] *= 1.0e-39
    out = run_gemv(core, esc, cnt, shape, 16, s, x, sg, 128)
    assert out["status"] == 1   # NONFINITE
    assert np.all(out["y"][0, 1] == 0.0)
    assert np.all(np.isnan(out["y"][1, 0]))
    xv = _xvals(x)
    tz = enc["two_z"].reshape(shape)
    y, _ = oracle.gemv_reference(tz, s.cpu().numpy(), np.nan_to_num(xv), sn, 128)
    tol = gemv_tolerance(tz, s.cpu().numpy(), np.nan_to_num(xv), sn, 128, 2048)
    keep = np.ones((3, 2), dtype=bool)
    keep[1, 0] = False
    err = np.abs(out["y"] - y)[keep]
    assert (err <= tol[keep]).all(), f"max err/tol {np.max(err / np.maximum(tol[keep], 1e-300)):.3g}"
