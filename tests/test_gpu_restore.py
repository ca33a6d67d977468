"""GPU parity of the inverse rotation: e8q_project_hadamard_restore (the
projection back in the original basis) and e8q_ste_backward_hadamard (the
rotated-basis gradient with the fused SGD step), bit for bit against the CPU
oracle."""

import numpy as np
import pytest
import torch

import oracle
from bit_e8_lattice_amd import workloads
import bit_e8_lattice_amd as e8q
from gpu_util import device, first_mismatch, run_restore, same_bits_or_nan, u16, wbits

pytestmark = pytest.mark.gpu

HBS = [8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096]


def _check(out, ref, bf16=True):
    m = first_mismatch(out["two_z_i8"].reshape(-1, 8), ref["two_z_i8"].reshape(-1, 8))
    assert m is None, f"2z: {m}"
    if bf16:
        m = first_mismatch(out["w_hat"].reshape(-1), ref["w_hat_bf16"].reshape(-1))
    else:
        m = first_mismatch(out["w_hat"].reshape(-1).view(np.uint32), ref["w_hat_f32"].reshape(-1).view(np.uint32))
    assert m is None, f"w_hat: {m}"
    assert out["status"] == ref["status"], (out["status"], ref["status"])


@pytest.mark.parametrize("hb", HBS)
@pytest.mark.parametrize("alpha", [1.0, 3.0])
def test_restore_every_block(hb, alpha):
    """Ragged batch and row counts, bf16 in and out, every block size."""
    d = device()
    cols = max(hb, 256)
    w = workloads.normal((3, 37, cols), 700 + hb, d)
    s = workloads.rms_scale(w, alpha)
    sg = workloads.signs(cols, 800 + hb, d)
    out = run_restore(w, s, sg, hb, core_bound=16)
    ref = oracle.project_restore(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), hb, core_bound=16)
    _check(out, ref)
    assert out["esc_count"].tolist() == ref["esc_count"].tolist()


@pytest.mark.parametrize("hb", [8, 128, 1024])
def test_restore_f32_in_and_out(hb):
    d = device()
    w = workloads.normal((2, 19, 2048), 900 + hb, d, dtype=torch.float32)
    s = workloads.rms_scale(w, 1.0)
    sg = workloads.signs(2048, 901, d)
    ref = oracle.project_restore(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), hb, w_is_bf16=False)
    _check(run_restore(w, s, sg, hb, out_dtype=torch.float32), ref, bf16=False)
    _check(run_restore(w, s, sg, hb, out_dtype=torch.bfloat16), ref, bf16=True)


@pytest.mark.parametrize("hb", [128, 4096])
def test_restore_mixes_fast_and_exact_groups(hb):
    """Small scales push many groups off the fast path (|x| >= 30), so blocks mix
    both paths; one row has huge coordinates, where the float32 butterflies of
    the inverse round."""
    d = device()
    w = workloads.normal((2, 24, 4096), 950 + hb, d)
    s = workloads.rms_scale(w, 0.04)
    s[5] = s[5] * 0.02          # |x| in the thousands on this row
    s[7] = 0.0                  # bad scale
    s[8] = float("inf")
    w[1, 3, 64:72] = float("nan")
    sg = workloads.signs(4096, 951, d)
    # row 9: rotated coordinates all large and positive, so that the sums of
    # the inverse transform exceed 2^24 for wide blocks and round
    rng = np.random.default_rng(952)
    s9 = float(s[9])
    y = (rng.uniform(3000.0, 7000.0, size=(1, 4096)) * s9).astype(np.float32)
    row9 = oracle.rotate_grad(y, sg.cpu().numpy(), hb, is_bf16=False)
    w[0, 9] = torch.from_numpy(row9[0]).to(d).to(torch.bfloat16)
    out = run_restore(w, s, sg, hb, core_bound=16)
    ref = oracle.project_restore(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), hb, core_bound=16)
    _check(out, ref)
    assert out["esc_count"].tolist() == ref["esc_count"].tolist()


def test_restore_qat_shape_sampled_rows():
    """4096 x 14336 bf16 (the QAT-loop matrix) in one launch; sampled rows exact."""
    d = device()
    b = workloads.qat_loop(d)
    out = run_restore(b.w, b.scale, b.signs, 128, core_bound=16)
    _, rows, cols = b.w.shape
    rsel = np.array([0, 1, 777, 2048, rows - 1])
    wr = wbits(b.w)[0][rsel]
    ref = oracle.project_restore(wr, b.scale.cpu().numpy()[rsel], b.signs.cpu().numpy(), 128)
    got = out["w_hat"].reshape(rows, cols)[rsel]
    assert first_mismatch(got, ref["w_hat_bf16"][0]) is None
    assert out["status"] == 0


@pytest.mark.parametrize("hb", HBS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ste_backward_hadamard(hb, dtype):
    d = device()
    rows, cols = 29, max(hb, 512)
    gen = torch.Generator(device=d).manual_seed(1000 + hb)
    g = (torch.randn(rows, cols, generator=gen, device=d) * 1e-3).to(dtype)
    wl = (torch.randn(rows, cols, generator=gen, device=d) * 0.02).to(dtype)
    g[3, 5] = float("nan")
    sg = workloads.signs(cols, 1100 + hb, d)
    is_bf16 = dtype == torch.bfloat16
    gb = wbits(g)
    wb = wbits(wl)
    gw = torch.empty_like(g)
    wl2 = wl.clone()
    e8q.e8q_ste_backward_hadamard(g, sg, hb, grad_w=gw, w_latent=wl2, lr=0.5)
    torch.cuda.synchronize()
    ref_g, ref_w = oracle.ste_backward_hadamard(gb, sg.cpu().numpy(), hb, is_bf16, wb, 0.5)
    if is_bf16:
        assert first_mismatch(u16(gw), ref_g) is None
        assert first_mismatch(u16(wl2), ref_w) is None
    else:
        assert same_bits_or_nan(gw.cpu().numpy(), ref_g) is None
        assert same_bits_or_nan(wl2.cpu().numpy(), ref_w) is None
    # in place, gradient only
    e8q.e8q_ste_backward_hadamard(g, sg, hb, grad_w=g)
    torch.cuda.synchronize()
    if is_bf16:
        assert first_mismatch(u16(g), ref_g) is None
    else:
        assert same_bits_or_nan(g.cpu().numpy(), ref_g) is None


def test_ste_backward_hadamard_is_adjoint_on_device():
    """<R w, g> = <w, R^T g> with both rotations from the library."""
    d = device()
    rows, cols, hb = 64, 4096, 128
    gen = torch.Generator(device=d).manual_seed(77)
    w = torch.randn(rows, cols, generator=gen, device=d)
    g = torch.randn(rows, cols, generator=gen, device=d)
    sg = workloads.signs(cols, 78, d)
    st = torch.zeros(1, dtype=torch.int32, device=d)
    u = torch.empty_like(w)
    e8q.e8q_project_hadamard(w, torch.ones(rows, device=d), sg, hb, st, rotated_out=u)
    rt = torch.empty_like(g)
    e8q.e8q_ste_backward_hadamard(g, sg, hb, grad_w=rt)
    lhs = (u.double() * g.double()).sum().item()
    rhs = (w.double() * rt.double()).sum().item()
    assert abs(lhs - rhs) <= 1e-5 * w.double().norm().item() * g.double().norm().item()
