"""GPU parity of e8q_encode_core_escape against the CPU oracle: core indices,
escape records and their order, per-batch counts and status bits, all
bit-exact."""

import numpy as np
import pytest
import torch

import oracle
from bit_e8_lattice_amd import workloads
from gpu_util import device, first_mismatch, run_encode, wbits

pytestmark = pytest.mark.gpu


def _compare(out, ref):
    m = first_mismatch(out["core_idx"], ref["core_idx"])
    assert m is None, f"core index: {m}"
    assert out["counts"].tolist() == ref["counts"].tolist()
    assert len(out["records"]) == len(ref["records"])
    m = first_mismatch(out["records"]["group"], ref["records"]["group"])
    assert m is None, f"record groups: {m}"
    m = first_mismatch(out["records"]["two_z"], ref["records"]["two_z"])
    assert m is None, f"record 2z: {m}"
    assert out["status"] == ref["status"], (out["status"], ref["status"])


@pytest.mark.parametrize("bound", [0, 8, 16, 24, 31, 32, 40])
def test_bounds_ragged(bound):
    """Every table layout (LDS up to 31, global memory above), ragged tail."""
    d = device()
    w = workloads.normal((3, 41, 256), 500 + bound, d)
    s = workloads.rms_scale(w, 1.5)
    sg = workloads.signs(256, 600 + bound, d)
    out = run_encode(w, s, bound, sg, 128)
    ref = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), 128, bound)
    _compare(out, ref)
    dec = oracle.decode_core_escape(out["core_idx"], out["records"], out["counts"], bound)
    assert np.array_equal(dec, ref["two_z"])


@pytest.mark.parametrize("hb", [0, 8, 32, 128])
@pytest.mark.parametrize("alpha", [1.0, 3.0])
def test_moe_shapes_reduced(hb, alpha):
    """Expert-FFN shapes (8 experts of gate 768x2048 / down 2048x768), Student-t
    weights, dense (alpha 1) and sparse (alpha 3) escape regimes."""
    d = device()
    for kind in ("gate", "down"):
        b = workloads.moe_experts(d, kind, experts=8, alpha=alpha, had_block=hb or 128)
        sg = b.signs if hb else None
        out = run_encode(b.w, b.scale, 16, sg, hb)
        ref = oracle.encode_core_escape(wbits(b.w), b.scale.cpu().numpy(),
                                        None if sg is None else sg.cpu().numpy(), hb, 16)
        _compare(out, ref)


def test_moe_full_sampled_experts():
    """Full 128-expert stacks in the launch configuration the benchmark uses;
    experts 0, 63 and 127 compared in full against the oracle."""
    d = device()
    for kind in ("gate", "up", "down"):
        b = workloads.moe_experts(d, kind)
        out = run_encode(b.w, b.scale, 16, b.signs, 128)
        off = np.concatenate([[0], np.cumsum(out["counts"])])
        gpe = b.w.shape[1] * b.w.shape[2] // 8
        for e in (0, 63, 127):
            ref = oracle.encode_core_escape(wbits(b.w[e]), b.scale[e * b.w.shape[1]:(e + 1) * b.w.shape[1]].cpu().numpy(),
                                            b.signs.cpu().numpy(), 128, 16)
            assert first_mismatch(out["core_idx"][e * gpe:(e + 1) * gpe], ref["core_idx"]) is None
            assert out["counts"][e] == ref["counts"][0]
            seg = out["records"][off[e]:off[e + 1]]
            assert np.array_equal(seg, ref["records"])
        assert (out["core_idx"] == 0xFFFF).sum() == out["counts"].sum()
        assert out["status"] == 0


def test_dense_decoder_full_sampled_rows():
    """All 224 dense-decoder matrices in three batched launches; rows sampled
    from the first, middle and last matrix of every launch checked exactly;
    counts checked against the escape slots of every matrix."""
    d = device()
    rng = np.random.default_rng(0)
    for b in workloads.dense_decoder(d):
        nb, rows, cols = b.w.shape
        gpr = cols // 8
        out = run_encode(b.w, b.scale, 16, b.signs, 128)
        core = out["core_idx"].reshape(nb, rows * gpr)
        assert ((core == 0xFFFF).sum(1) == out["counts"]).all()
        off = np.concatenate([[0], np.cumsum(out["counts"])])
        for m in (0, nb // 2, nb - 1):
            rsel = np.unique(np.concatenate([[0, 1, rows - 1], rng.integers(0, rows, 5)]))
            wm = wbits(b.w[m])[rsel]
            sm = b.scale[m * rows:(m + 1) * rows].cpu().numpy()[rsel]
            ref = oracle.encode_core_escape(wm, sm, b.signs.cpu().numpy(), 128, 16)
            got_core = core[m].reshape(rows, gpr)[rsel].reshape(-1)
            assert first_mismatch(got_core, ref["core_idx"]) is None
            seg = out["records"][off[m]:off[m + 1]]
            keep = np.isin(seg["group"] // gpr, rsel)
            seg = seg[keep]
            ref_rec = ref["records"].copy()
            ref_rec["group"] = rsel[ref_rec["group"] // gpr] * gpr + ref_rec["group"] % gpr
            assert np.array_equal(seg, ref_rec)
            assert (np.diff(out["records"][off[m]:off[m + 1]]["group"].astype(np.int64)) > 0).all()
        assert out["status"] == 0


def test_escape_capacity_overflow():
    d = device()
    w = workloads.normal((2, 64, 256), 42, d)
    s = workloads.rms_scale(w, 1.0)
    full = run_encode(w, s, 16)
    n = int(full["counts"].sum())
    assert n > 100
    for cap in (0, 1, n // 3, n - 1, n):
        out = run_encode(w, s, 16, cap=cap)
        ref = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), None, 0, 16, esc_capacity=cap)
        _compare(out, ref)


def test_two_z_output_and_invalid_rows():
    d = device()
    w = workloads.normal((1, 16, 128), 43, d, dtype=torch.float32)
    w[0, 3, 7] = float("nan")
    w[0, 5, :8] = 500.0
    s = workloads.rms_scale(w, 1.0)
    s[9] = 0.0
    out = run_encode(w, s, 16, two_z=True)
    ref = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), None, 0, 16, w_is_bf16=False,
                                    want_two_z=True)
    _compare(out, ref)
    assert np.array_equal(out["two_z_i8"].reshape(-1, 8), np.clip(ref["two_z"], -128, 127))


def test_deterministic_order_repeat():
    """Escape order must not depend on scheduling: run twice at alpha = 1
    (most groups escape) and compare everything bitwise."""
    d = device()
    b = workloads.moe_experts(d, "down", experts=16, alpha=1.0)
    a1 = run_encode(b.w, b.scale, 16, b.signs, 128)
    a2 = run_encode(b.w, b.scale, 16, b.signs, 128)
    assert np.array_equal(a1["records"], a2["records"])
    assert np.array_equal(a1["core_idx"], a2["core_idx"])
    assert a1["counts"].sum() > 0.5 * a1["core_idx"].size


@pytest.mark.parametrize("hb", [256, 1024, 4096])
@pytest.mark.parametrize("alpha", [1.0, 3.0])
def test_wide_blocks_encode(hb, alpha):
    """Encode with blocks wider than 128 columns: LDS stages in both passes
    (records are recomputed block-wide)."""
    d = device()
    w = workloads.normal((3, 7, 4096), 5000 + hb, d)
    s = workloads.rms_scale(w, alpha)
    sg = workloads.signs(4096, 6000 + hb, d)
    out = run_encode(w, s, 16, sg, hb)
    ref = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), hb, 16)
    _compare(out, ref)


def test_decoder_secondary_reading_encode():
    """Dense-decoder rows encoded with whole-row power-of-two blocks."""
    d = device()
    for rows, cols, hb in ((48, 4096, 4096), (20, 11008, 256)):
        w = workloads.normal((2, rows, cols), 7 * rows + cols, d)
        s = workloads.rms_scale(w, 3.0)
        sg = workloads.signs(cols, 4001 if cols == 4096 else 4002, d)
        out = run_encode(w, s, 16, sg, hb)
        ref = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), hb, 16)
        _compare(out, ref)


@pytest.mark.parametrize("bound", [16, 32, 40])
def test_tail_lanes_with_an_escaped_last_group(bound):
    """Lanes past the end of the input work on a copy of the last group; here
    that group's point is far outside the core, so they must not index the rank
    table (bounds 32 and 40 keep it in global memory)."""
    d = device()
    w = workloads.normal((1, 3, 136), 777 + bound, d, dtype=torch.float32)
    s = workloads.rms_scale(w, 1.0)
    w[0, 2, 128:136] = -25.0 * s[2]
    out = run_encode(w, s, bound)
    ref = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), None, 0, bound, w_is_bf16=False)
    assert ref["core_idx"][-1] == oracle.ESCAPE_SLOT
    _compare(out, ref)


@pytest.mark.parametrize("shape", [(5000, 1, 8), (1500, 3, 8), (900, 1, 72), (250, 37, 8)])
def test_many_small_batch_items(shape):
    """Batch items of 1 to 37 groups: tiles and 64-group slices span many
    items, so the per-item escape counts are split inside one tile."""
    d = device()
    w = workloads.normal(shape, 31 * shape[0] + shape[2], d)
    s = workloads.rms_scale(w, 1.0)
    for bound in (0, 16):
        out = run_encode(w, s, bound)
        ref = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), None, 0, bound)
        _compare(out, ref)
        assert out["counts"].sum() > shape[0] // 4


@pytest.mark.parametrize("cap", [None, 0, 10, 19, 20, 35])
def test_tile_escape_counts_around_the_staging_limit(cap):
    """Tiles of 4096 groups with 3, 16, 17, 0 and 1 escapes: tiles with at most
    16 escapes stage their records for a later placement, tiles with more place
    them directly; records in order, counts exact, truncation at the capacity."""
    d = device()
    w = torch.zeros((1, 320, 512), dtype=torch.float32)
    gen = np.random.default_rng(77)
    per_tile = [3, 16, 17, 0, 1]
    for k, n in enumerate(per_tile):
        for g in sorted(gen.choice(4096, n, replace=False)):
            gg = 4096 * k + int(g)
            w[0, gg // 64, (gg % 64) * 8:(gg % 64) * 8 + 8] = 3.0
    w = w.to(torch.bfloat16).to(d)
    s = torch.ones(320, dtype=torch.float32, device=d)
    out = run_encode(w, s, 16, cap=cap)
    ref = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), None, 0, 16,
                                    esc_capacity=(w.numel() // 8 if cap is None else cap))
    assert int(ref["counts"].sum()) == sum(per_tile)
    _compare(out, ref)


@pytest.mark.parametrize("rows,cols", [(13, 4096), (5, 8192), (3, 12288)])
@pytest.mark.parametrize("alpha", [1.0, 2.6])
def test_row_items(rows, cols, alpha):
    """Rows of 4096, 8192 and 12288 columns (one, two and three 512-group items
    of a tile per row), a batch of 2 whose group count leaves the last tile
    partly empty; 2.6 x RMS lists a few escapes per tile, 1 x RMS takes the
    second pass."""
    d = device()
    w = workloads.normal((2, rows, cols), 7000 + rows, d)
    s = workloads.rms_scale(w, alpha)
    sg = workloads.signs(cols, 7100 + rows, d)
    out = run_encode(w, s, 16, sg, 128)
    ref = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), 128, 16)
    _compare(out, ref)
