"""GPU parity of e8q_ptq_init against the oracle: chosen scales and
candidates (bit for bit: the choice is made on exact row errors), every
reported float64 row error within its stated bound of the exact one, the
finite-core points, core indices and status.  Rows built so that candidates
tie exactly or nearly make the kernel resolve its float64 screen exactly."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from bit_e8_lattice_amd import workloads
from gpu_util import device, first_mismatch, run_decode, run_ptq, wbits
from ptq_cases import tie_row

pytestmark = pytest.mark.gpu

ALPHAS = [0.75, 1.0, 1.5, 2.0, 2.5, 3.0]


def _check_err(err, exact, cols):
    """Every reported error within gamma_{cols+2} = n u / (1 - n u) of the
    exact one (n = cols + 2, u = 2^-53); +inf and NaN where the oracle has them."""
    n = cols + 2
    gamma = Fraction(n, 2 ** 53 - n)
    for r, row in enumerate(exact):
        for k, e in enumerate(row):
            got = float(err[r, k])
            if e is None:
                assert np.isnan(got), (r, k, got)
            elif e == float("inf"):
                assert got == float("inf"), (r, k, got)
            else:
                assert np.isfinite(got) and abs(Fraction(got) - e) <= gamma * e, (r, k, got, float(e))


def _cmp(out, ref, cols):
    assert first_mismatch(out["scale"].view(np.uint32), ref["scale"].view(np.uint32)) is None
    assert np.array_equal(out["k"], ref["k"]), (out["k"], ref["k"])
    _check_err(out["err"], ref["err_exact"], cols)
    assert first_mismatch(out["two_z_i8"].reshape(-1, 8), ref["two_z"]) is None
    assert first_mismatch(out["core_idx"], ref["core_idx"]) is None
    assert out["status"] == ref["status"], (out["status"], ref["status"])


@pytest.mark.parametrize("hb", [0, 128, 1024])
@pytest.mark.parametrize("bound", [8, 16, 24])
def test_ptq_init(hb, bound):
    d = device()
    w = workloads.student_t4((2, 23, 1024), 2100 + hb + bound, d)
    s0 = workloads.rms_scale(w, 1.0)
    sg = workloads.signs(1024, 2101, d) if hb else None
    out = run_ptq(w, s0, ALPHAS, bound, sg, hb)
    ref = oracle.ptq_init(wbits(w), s0.cpu().numpy(), ALPHAS, None if sg is None else sg.cpu().numpy(), hb, bound)
    _cmp(out, ref, 1024)


def test_ptq_invalid_rows_and_f32():
    d = device()
    w = workloads.normal((1, 9, 256), 2200, d, dtype=torch.float32)
    s0 = workloads.rms_scale(w, 1.0)
    w[0, 2, 17] = float("nan")
    w[0, 4, :8] = 1e6
    s0[6] = -1.0
    al = [0.0, 1.0, 2.0]
    out = run_ptq(w, s0, al, 16)
    ref = oracle.ptq_init(wbits(w), s0.cpu().numpy(), al, None, 0, 16, w_is_bf16=False)
    _cmp(out, ref, w.shape[-1])


def test_ptq_decoder_block_sampled_rows_and_decode():
    """One dense-decoder block (q, k, v, o, gate, up, down) in three launches;
    sampled rows exact against the oracle; the result decodes (zero escapes)
    to weights whose error is the reported row error."""
    d = device()
    rng = np.random.default_rng(7)
    for b in workloads.dense_decoder(d, blocks=1, alpha=1.0):
        nb, rows, cols = b.w.shape
        out = run_ptq(b.w, b.scale, ALPHAS, 16, b.signs, 128)
        assert out["status"] == 0
        for m in (0, nb - 1):
            rsel = np.unique(np.concatenate([[0, rows - 1], rng.integers(0, rows, 2)]))
            s0 = b.scale[m * rows:(m + 1) * rows].cpu().numpy()[rsel]
            ref = oracle.ptq_init(wbits(b.w[m])[rsel], s0, ALPHAS, b.signs.cpu().numpy(), 128, 16)
            r0 = m * rows + rsel
            sub = {"scale": out["scale"][r0], "k": out["k"][r0], "err": out["err"][r0],
                   "two_z_i8": out["two_z_i8"].reshape(nb, rows, cols)[m][rsel],
                   "core_idx": out["core_idx"].reshape(nb, rows, cols // 8)[m][rsel].reshape(-1),
                   "status": out["status"]}
            _cmp(sub, ref, cols)
        core, scale = out["dev"]
        cnt = torch.zeros(nb, dtype=torch.int64, device=d)
        dec = run_decode(core, None, cnt, (nb, rows, cols), 16, scale, b.signs, 128, two_z=True,
                         w_hat_dtype=torch.float32)
        assert dec["status"] == 0
        assert np.array_equal(dec["two_z_i8"], out["two_z_i8"])
        # the decoded weights' squared error is the chosen row error (float32 rounding aside)
        wf = b.w.float().cpu().numpy().reshape(nb * rows, cols).astype(np.float64)
        e = ((wf - dec["w_hat"].reshape(nb * rows, cols).astype(np.float64)) ** 2).sum(1)
        chosen = out["err"][np.arange(nb * rows), out["k"]]
        assert np.allclose(e, chosen, rtol=1e-4, atol=0)


def _search_groups(bound, n, seed):
    """Normalized groups (exact float32 values) that stress the core search:
    points on the bisector mu (t1 + t2) / 4 of two points of one shell (their
    keys are exactly equal), groups far outside the core, and ordinary ones."""
    rng = np.random.default_rng(seed)
    pts = oracle.core_points(bound).astype(np.int64)
    nrm = (pts * pts).sum(1)
    shells = [pts[nrm == s] for s in range(8, bound + 1, 8) if (nrm == s).any()]
    out = []
    while len(out) < n:
        kind = int(rng.integers(0, 3))
        if kind == 0 and shells:
            sh = shells[int(rng.integers(0, len(shells)))]
            t1, t2 = sh[rng.integers(0, len(sh), 2)]
            x = float(rng.choice([1.25, 1.5, 2.0, 3.0, 5.0])) * (t1 + t2) / 4.0
        elif kind == 1:
            x = np.round(rng.standard_normal(8) * float(rng.choice([4.0, 16.0, 64.0])) * 64) / 64
        else:
            x = np.round(rng.standard_normal(8) * 2 * 256) / 256
        out.append(x)
    return np.asarray(out, np.float32), pts, nrm


@pytest.mark.parametrize("bound", [0, 7, 16, 32, 40])
def test_ptq_search_ties_and_far_groups(bound):
    """The search against the oracle on groups chosen so that the best core
    point is often tied (equal float64 keys in different tiles and in one
    tile), including the one-point core and the largest core."""
    d = device()
    n = 128 if bound == 40 else 1024
    x, pts, nrm = _search_groups(bound, n, 2300 + bound)
    keys = x.astype(np.float64) @ pts.T.astype(np.float64) - nrm / 4.0
    outside = (oracle.nearest_e8_two_z(x) ** 2).sum(1) > bound
    ties = (keys == keys.max(1, keepdims=True)).sum(1) >= 2
    if bound >= 8:
        assert (outside & ties).sum() >= 10     # the tie cases are really searched
    assert outside.sum() >= n // 2
    w = torch.from_numpy(x.reshape(1, n // 32, 256)).to(d)
    s0 = torch.ones(n // 32, dtype=torch.float32, device=d)
    out = run_ptq(w, s0, [1.0], bound)
    ref = oracle.ptq_init(x.reshape(1, n // 32, 256), np.ones(n // 32, np.float32), [1.0], None, 0, bound,
                          w_is_bf16=False)
    _cmp(out, ref, w.shape[-1])


def _run_and_check(w, s0, alphas, bound, signs=None, hb=0, w_is_bf16=False):
    out = run_ptq(w, torch.as_tensor(s0).to(w.device), alphas, bound, signs, hb)
    ref = oracle.ptq_init(wbits(w) if w_is_bf16 else w.cpu().numpy(), np.asarray(s0, np.float32), alphas,
                          None if signs is None else signs.cpu().numpy(), hb, bound, w_is_bf16=w_is_bf16)
    _cmp(out, ref, w.shape[-1])
    return out, ref


@pytest.mark.parametrize("eta,k", [(0, 0), (1, 1)])
def test_ptq_constructed_tie_and_near_tie(eta, k):
    """Errors equal exactly (the smaller k wins) or differing by 2^-46 at
    E ~ 160 (the second wins): inside the float64 screen, decided exactly."""
    d = device()
    w, s0, al = tie_row(eta_units=eta)
    out, ref = _run_and_check(torch.from_numpy(w).to(d), s0, al, 16)
    assert out["k"][0] == k


def _least_squares_scale(wb, s, sgn, hb, iters=12):
    """Alternate the finite-core projection and the scale minimizing the
    row's error for those points, s = sum (kappa v) z / sum z^2."""
    rows, cols = wb.shape[-2:]
    v = oracle.fwht_blocks(oracle.bf16_to_f32(wb).reshape(rows, cols) * sgn.astype(np.float32), hb)
    kv = float(oracle.kappa(hb)) * v.astype(np.float64)
    s = np.asarray(s, np.float32)
    for _ in range(iters):
        z = 0.5 * oracle.ptq_init(wb.reshape(1, rows, cols), s, [1.0], sgn, hb, 16)["two_z"].reshape(rows, cols)
        num, den = (kv * z).sum(1), (z * z).sum(1)
        s = np.where(den > 0, num / np.maximum(den, 1e-300), 1.0).astype(np.float32)
    return s


def test_ptq_exact_resolution_on_rotated_rows():
    """bf16 rows with a 128-wide rotation, base scale at the least-squares
    scale of the row's own projection, candidates one or two float32 ulps
    apart (errors within ~1e-12 of each other) and a repeated candidate (an
    exact tie); plus an all-zero row (every error 0)."""
    d = device()
    rows, cols, hb = 12, 2048, 128
    w = workloads.student_t4((1, rows, cols), 2400, d)
    w[0, 5].zero_()
    sg = workloads.signs(cols, 2401, d)
    wb, sgn = wbits(w), sg.cpu().numpy()
    s_rms = workloads.rms_scale(w, 1.0).cpu().numpy()
    s_rms[5] = 1.0
    s_star = _least_squares_scale(wb, s_rms, sgn, hb)
    # worst first, so that exact comparisons both take and keep candidates
    al = np.array([1.0 + 2.0 ** -22, 1.0 + 2.0 ** -23, 1.0, 1.0, 1.0 - 2.0 ** -23], np.float32)
    out, ref = _run_and_check(w, s_star, al, 16, sg, hb, w_is_bf16=True)
    e = ref["err_exact"]
    close = [r for r in range(rows) if r != 5 and all(abs(x - e[r][2]) < Fraction(1, 2 ** 32) * e[r][2] for x in e[r])]
    assert len(close) >= rows - 3                # the screen leaves these rows to the exact comparison
    assert out["k"][5] == 0 and all(x == 0 for x in e[5])
    assert all(out["k"][r] != 3 for r in range(rows))   # the repeated candidate never beats its twin


def test_ptq_single_point_core_all_tied():
    """B = 0 (the core is the origin): every candidate's error is
    sum (kappa v)^2, an exact tie resolved to k = 0, with a 64-wide rotation."""
    d = device()
    w = workloads.normal((1, 6, 512), 2500, d, dtype=torch.float32)
    sg = workloads.signs(512, 2501, d)
    s0 = workloads.rms_scale(w, 1.0).cpu().numpy()
    out, ref = _run_and_check(w, s0, [0.5, 1.0, 2.0], 0, sg, 64)
    assert (out["k"] == 0).all()
