"""GPU parity of e8q_project / e8q_project_hadamard against the CPU oracle.

Bit-exact on 2z (int8), bf16 q and float32 q.  Rotated values: the contract
allows 1e-6 relative; they are checked to be equal as values (the canonical
operation order makes every non-zero value bit-identical; an exact zero may
differ in sign)."""

import numpy as np
import pytest
import torch

import oracle
from bit_e8_lattice_amd import workloads
from gpu_util import device, first_mismatch, run_project, wbits

pytestmark = pytest.mark.gpu


def _compare(out, ref, q_bf16=True, rotated=False):
    m = first_mismatch(out["two_z_i8"].reshape(-1, 8), ref["two_z_i8"].reshape(-1, 8))
    assert m is None, f"2z: {m}"
    if "q" in out:
        want = ref["q_bf16"] if q_bf16 else ref["q_f32"]
        if q_bf16:
            m = first_mismatch(out["q"].reshape(-1), want.reshape(-1))
        else:
            m = first_mismatch(out["q"].reshape(-1).view(np.uint32), want.reshape(-1).view(np.uint32))
        assert m is None, f"q: {m}"
    if rotated:
        u, v = out["u"].reshape(-1), ref["u"].reshape(-1)
        rel = np.abs(u.astype(np.float64) - v) / np.maximum(np.abs(v.astype(np.float64)), 1e-30)
        assert rel.max() <= 1e-6
        # equal as values (the contract's bar is 1e-6 relative); the sign of an
        # exact zero is the only freedom left
        assert np.array_equal(u, v)
    assert out["status"] == ref["status"], (out["status"], ref["status"])


def test_small_f32_workload_project():
    """256x256 float32, per-row RMS scale, no rotation: q float32 and 2z."""
    d = device()
    b = workloads.small_f32(d)
    out = run_project(b.w, b.scale, q_dtype=torch.float32)
    ref = oracle.project(wbits(b.w), b.scale.cpu().numpy(), w_is_bf16=False)
    _compare(out, ref, q_bf16=False)
    out = run_project(b.w, b.scale, q_dtype=torch.bfloat16)
    _compare(out, ref, q_bf16=True)


def test_linear_4096_project_hadamard():
    """4096x4096 bf16, random signs, 128-wide Walsh-Hadamard, per-row RMS."""
    d = device()
    b = workloads.linear_4096(d)
    out = run_project(b.w, b.scale, b.signs, 128, rotated=True, core_bound=16)
    ref = oracle.project(wbits(b.w), b.scale.cpu().numpy(), b.signs.cpu().numpy(), 128, core_bound=16)
    _compare(out, ref, rotated=True)
    assert out["esc_count"].tolist() == ref["esc_count"].tolist()


@pytest.mark.parametrize("hb", [8, 16, 32, 64, 128])
@pytest.mark.parametrize("wdtype", [torch.bfloat16, torch.float32])
def test_blocks_ragged_batch(hb, wdtype):
    """Several tiles with a ragged tail: 3 x 37 x 384 (5,328 groups)."""
    d = device()
    w = workloads.normal((3, 37, 384), 1000 + hb, d, dtype=wdtype)
    s = workloads.rms_scale(w, 1.0)
    sg = workloads.signs(384, 2000 + hb, d)
    out = run_project(w, s, sg, hb, rotated=True, core_bound=8)
    ref = oracle.project(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), hb, core_bound=8,
                         w_is_bf16=wdtype == torch.bfloat16)
    _compare(out, ref, rotated=True)
    assert out["esc_count"].tolist() == ref["esc_count"].tolist()


@pytest.mark.parametrize("rows,cols", [(1, 8), (1, 16), (5, 24), (63, 40), (65, 8)])
def test_tiny_shapes_no_rotation(rows, cols):
    d = device()
    w = workloads.normal((rows, cols), rows * 100 + cols, d, std=1.0)
    s = torch.full((rows,), 0.37, dtype=torch.float32, device=d)
    out = run_project(w, s, core_bound=0)
    ref = oracle.project(wbits(w), s.cpu().numpy(), core_bound=0)
    _compare(out, ref)
    assert out["esc_count"].tolist() == ref["esc_count"].tolist()


def test_heavy_tails_and_scales():
    """Student-t weights at several scale multipliers (large |2z|)."""
    d = device()
    w = workloads.student_t4((16, 1024), 77, d)
    for alpha in (0.05, 0.3, 1.0, 3.0):
        s = workloads.rms_scale(w, alpha)
        out = run_project(w, s, core_bound=16)
        ref = oracle.project(wbits(w), s.cpu().numpy(), core_bound=16)
        _compare(out, ref)


def test_invalid_data_status_bits():
    d = device()
    w = torch.zeros((4, 64), dtype=torch.float32)
    w[0] = 0.3
    w[1, 5] = float("nan")
    w[1, 20] = float("inf")
    w[2, :] = 0.25
    w[2, 9] = 1e6
    w[3, :] = 100.0                   # |2z| = 200 saturates int8
    s = torch.tensor([1.0, 1.0, 1.0, 1.0])
    wd, sd = w.to(d), s.to(d)
    out = run_project(wd, sd, q_dtype=torch.float32)
    ref = oracle.project(w.numpy(), s.numpy(), w_is_bf16=False)
    _compare(out, ref, q_bf16=False)
    assert out["status"] == (oracle.STATUS_NONFINITE | oracle.STATUS_X_RANGE | oracle.STATUS_INT8_RANGE)
    for bad in (0.0, -2.0, float("nan"), float("inf"), 1e-45):
        s2 = torch.tensor([1.0, bad, 1.0, 1.0])
        out = run_project(wd, s2.to(d), q_dtype=torch.float32, two_z=True)
        ref = oracle.project(w.numpy(), s2.numpy(), w_is_bf16=False)
        _compare(out, ref, q_bf16=False)
        assert out["status"] & oracle.STATUS_BAD_SCALE


def test_bad_scales_wide_rows():
    """Rows of 128 groups (row coefficients computed once per tile and row),
    40 rows over two tiles, bf16 with a 128-wide rotation: every kind of bad
    scale on rows of both tiles; each bad row projects to 0 with BAD_SCALE."""
    d = device()
    w = workloads.normal((40, 1024), 120, d)
    s = workloads.rms_scale(w, 1.0)
    sc = s.cpu()
    for r, bad in zip((1, 8, 31, 32, 39), (0.0, -2.0, float("nan"), float("inf"), 1e-45)):
        sc[r] = bad
    sg = workloads.signs(1024, 121, d)
    out = run_project(w, sc.to(d), sg, 128)
    ref = oracle.project(wbits(w), sc.numpy(), sg.cpu().numpy(), 128)
    _compare(out, ref)
    assert out["status"] == oracle.STATUS_BAD_SCALE


def test_exact_ties_and_lattice_points():
    """Quarter/half grids and exact lattice points: tie rules must match."""
    d = device()
    rng = np.random.default_rng(5)
    x = (rng.integers(-12, 13, size=(4096, 8)) / 4).astype(np.float32)
    x[:64] = np.float32(0.25)
    x[64:128] = np.array([1, 0, 0, 0, 0, 0, 0, 0], np.float32)
    x[128:192] = np.array([0.5, 0.5, 0, 0, 0, 0, 0, 0], np.float32)
    w = torch.from_numpy(x.reshape(64, 512))
    s = torch.ones(64, dtype=torch.float32)
    out = run_project(w.to(d), s.to(d), q_dtype=torch.float32)
    ref = oracle.project(w.numpy(), s.numpy(), w_is_bf16=False)
    _compare(out, ref, q_bf16=False)


def test_near_decision_boundary_float64_path():
    """Inputs whose coset decision lies within float32 rounding of zero force the
    float64 path: (1/4 + eps)^8 style vectors at many eps."""
    d = device()
    eps = np.float32(2.0) ** -np.arange(10, 40, dtype=np.float32)
    x = np.full((len(eps) * 4, 8), 0.25, dtype=np.float32)
    for i, e in enumerate(eps):
        x[4 * i] += e
        x[4 * i + 1] -= e
        x[4 * i + 2, 0] += e
        x[4 * i + 3, 7] -= e
    w = torch.from_numpy(x.reshape(-1, 64))
    s = torch.ones(w.shape[0], dtype=torch.float32)
    out = run_project(w.to(d), s.to(d), q_dtype=torch.float32)
    ref = oracle.project(w.numpy(), s.numpy(), w_is_bf16=False)
    _compare(out, ref, q_bf16=False)


def test_deterministic_repeat():
    d = device()
    b = workloads.linear_4096(d, rows=512)
    a1 = run_project(b.w, b.scale, b.signs, 128)
    a2 = run_project(b.w, b.scale, b.signs, 128)
    assert first_mismatch(a1["q"], a2["q"]) is None
    assert first_mismatch(a1["two_z_i8"], a2["two_z_i8"]) is None


@pytest.mark.parametrize("hb", [256, 512, 1024, 2048, 4096])
@pytest.mark.parametrize("wdtype", [torch.bfloat16, torch.float32])
def test_wide_blocks_lds_stages(hb, wdtype):
    """Blocks wider than 128 columns (LDS stages): 2 x 9 x 4096, a ragged last
    tile, rotated values, q and 2z."""
    d = device()
    w = workloads.normal((2, 9, 4096), 3000 + hb, d, dtype=wdtype)
    s = workloads.rms_scale(w, 1.0)
    sg = workloads.signs(4096, 4000 + hb, d)
    out = run_project(w, s, sg, hb, rotated=True, core_bound=16)
    ref = oracle.project(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), hb, core_bound=16,
                         w_is_bf16=wdtype == torch.bfloat16)
    _compare(out, ref, rotated=True)
    assert out["esc_count"].tolist() == ref["esc_count"].tolist()


def test_decoder_shapes_full_row_blocks():
    """The secondary reading of the dense decoder: the largest power-of-two block
    dividing each row (4096 for 4096-column rows, 256 for 11008-column rows)."""
    d = device()
    for rows, cols, hb in ((64, 4096, 4096), (24, 11008, 256)):
        w = workloads.normal((2, rows, cols), rows + cols, d)
        s = workloads.rms_scale(w, 3.0)
        sg = workloads.signs(cols, 4001 if cols == 4096 else 4002, d)
        out = run_project(w, s, sg, hb, core_bound=16)
        ref = oracle.project(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), hb, core_bound=16)
        _compare(out, ref)
        assert out["esc_count"].tolist() == ref["esc_count"].tolist()


@pytest.mark.parametrize("shape", [(5000, 1, 8), (250, 37, 8), (900, 1, 72), (40, 300, 64)])
def test_escape_counts_many_batch_items(shape):
    """Per-batch escape counts when waves and blocks span many batch items
    (each wave holds its count while its items stay in one batch item)."""
    d = device()
    w = workloads.normal(shape, 17 * shape[0] + shape[2], d)
    s = workloads.rms_scale(w, 1.0)
    for bound in (0, 16):
        out = run_project(w, s, core_bound=bound)
        ref = oracle.project(wbits(w), s.cpu().numpy(), core_bound=bound)
        assert out["esc_count"].tolist() == ref["esc_count"].tolist()
        assert int(out["esc_count"].sum()) > 0
