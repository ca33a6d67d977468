"""GPU parity of e8q_sgd_project_hadamard, the QAT step's latent update fused
with the next forward projection: bit for bit the same latents, q, 2z, escape
counts and status as e8q_ste_backward followed by e8q_project_hadamard (or
e8q_project), and against the oracle's SGD rule and projection."""

import numpy as np
import pytest
import torch

import bit_e8_lattice_amd as e8q
import oracle
from bit_e8_lattice_amd import workloads
from gpu_util import device, first_mismatch, u16, wbits

pytestmark = pytest.mark.gpu


def _outputs(w, q_dtype, with_tz):
    d = w.device
    return {"q": torch.empty(w.shape, dtype=q_dtype, device=d),
            "tz": torch.empty(w.shape, dtype=torch.int8, device=d) if with_tz else None,
            "esc": torch.zeros(w.shape[0] if w.dim() == 3 else 1, dtype=torch.int64, device=d),
            "st": torch.zeros(1, dtype=torch.int32, device=d)}


def _unfused(w, g, lr, s, signs, hb, o, bound):
    e8q.e8q_ste_backward(g, w_latent=w, lr=lr)
    if signs is None:
        e8q.e8q_project(w, s, o["st"], q_out=o["q"], two_z_out=o["tz"], core_bound=bound, esc_count_out=o["esc"])
    else:
        e8q.e8q_project_hadamard(w, s, signs, hb, o["st"], q_out=o["q"], two_z_out=o["tz"], core_bound=bound,
                                 esc_count_out=o["esc"])


def _fused(w, g, lr, s, signs, hb, o, bound):
    e8q.e8q_sgd_project_hadamard(w, g, lr, s, o["st"], signs=signs, had_block=hb, q_out=o["q"], two_z_out=o["tz"],
                                 core_bound=bound, esc_count_out=o["esc"])


def _same(a, b):
    for k in a:
        if a[k] is None:
            continue
        x, y = a[k], b[k]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        elif x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), k


@pytest.mark.parametrize("shape,hb,q_dtype,tz", [
    ((1, 64, 1024), 128, torch.bfloat16, True),
    ((3, 17, 512), 64, torch.float32, False),
    ((2, 9, 136), 8, torch.bfloat16, True),
    ((1, 33, 264), 0, torch.bfloat16, True),
    ((1, 8, 4096), 4096, torch.bfloat16, False),
])
def test_fused_matches_unfused(shape, hb, q_dtype, tz):
    d = device()
    w = workloads.normal(shape, 700 + shape[2], d)
    s = workloads.rms_scale(w, 1.5)
    sg = workloads.signs(shape[2], 701, d) if hb else None
    w1, w2 = w.clone(), w.clone()
    o1, o2 = _outputs(w, q_dtype, tz), _outputs(w, q_dtype, tz)
    for k in range(3):
        g = workloads.normal(shape, 710 + k, d, std=0.05)
        _unfused(w1, g, 0.5, s, sg, hb, o1, 16)
        _fused(w2, g, 0.5, s, sg, hb, o2, 16)
        torch.cuda.synchronize()
        assert torch.equal(w1.view(torch.int16), w2.view(torch.int16)), f"latents, step {k}"
        _same(o1, o2)


def test_fused_against_oracle_with_special_values():
    """NaN, inf, subnormal and zero latents and gradients: the oracle's SGD
    rule (NaN -> 0x7FC0), then the oracle's projection of the new latents."""
    d = device()
    rows, cols = 6, 256
    w = workloads.normal((1, rows, cols), 720, d)
    g = workloads.normal((1, rows, cols), 721, d, std=0.02)
    special = torch.tensor([float("nan"), float("inf"), -float("inf"), 1e-40, -1e-39, 0.0, -0.0, 3e38],
                           dtype=torch.float32)
    w[0, 1, :8] = special.to(torch.bfloat16).to(d)
    g[0, 2, :8] = special.to(torch.bfloat16).to(d)
    w[0, 3, :8] = 1e-39
    g[0, 3, :8] = -1e-39
    s = workloads.rms_scale(torch.nan_to_num(w.float(), nan=0.0, posinf=0.0, neginf=0.0).to(torch.bfloat16), 1.0)
    sg = workloads.signs(cols, 722, d)
    w0, g0 = wbits(w), wbits(g)
    o = _outputs(w, torch.bfloat16, True)
    _fused(w, g, 1.0, s, sg, 128, o, 16)
    torch.cuda.synchronize()
    want_w = oracle.sgd_update(w0.reshape(-1), g0.reshape(-1), 1.0).reshape(w0.shape)
    assert first_mismatch(u16(w).reshape(-1), want_w.reshape(-1)) is None
    ref = oracle.project(want_w, s.cpu().numpy(), sg.cpu().numpy(), 128, core_bound=16)
    assert first_mismatch(u16(o["q"]).reshape(-1), ref["q_bf16"].reshape(-1)) is None
    assert np.array_equal(o["tz"].cpu().numpy().reshape(-1), ref["two_z_i8"].reshape(-1))
    assert int(o["esc"][0]) == int(ref["esc_count"][0])
    assert (int(o["st"].item()) & 0xFFFFFFFF) == ref["status"]


def test_fused_qat_loop_matches_unfused():
    """The 4096x14336 QAT loop, 12 steps: latents, q and escape counts of every
    step bit-identical between the fused and the unfused sequence."""
    d = device()
    b = workloads.qat_loop(d)
    w1, w2 = b.w[0].clone(), b.w[0].clone()
    o1, o2 = _outputs(w1[None], torch.bfloat16, False), _outputs(w2[None], torch.bfloat16, False)
    esc1, esc2 = [], []
    for k in range(12):
        g = workloads.qat_grad(k, w1.shape, d)
        _unfused(w1, g, 1.0, b.scale, b.signs, 128, o1, 16)
        _fused(w2, g, 1.0, b.scale, b.signs, 128, o2, 16)
        esc1.append(o1["esc"].clone())
        esc2.append(o2["esc"].clone())
    torch.cuda.synchronize()
    assert torch.equal(w1.view(torch.int16), w2.view(torch.int16))
    _same(o1, o2)
    assert all(torch.equal(x, y) for x, y in zip(esc1, esc2))


@pytest.mark.parametrize("hb,wh_dtype", [(128, torch.bfloat16), (64, torch.float32), (4096, torch.bfloat16)])
def test_fused_restore_matches_unfused(hb, wh_dtype):
    """The restored-basis variant: latents, w_hat, 2z, escape counts and status
    bit for bit as e8q_ste_backward + e8q_project_hadamard_restore."""
    d = device()
    shape = (2, 24, 4096) if hb == 4096 else (2, 24, 1024)
    w = workloads.normal(shape, 730 + hb, d)
    s = workloads.rms_scale(w, 1.5)
    sg = workloads.signs(shape[2], 731, d)
    w1, w2 = w.clone(), w.clone()
    o1 = {"wh": torch.empty(shape, dtype=wh_dtype, device=d), "tz": torch.empty(shape, dtype=torch.int8, device=d),
          "esc": torch.zeros(shape[0], dtype=torch.int64, device=d), "st": torch.zeros(1, dtype=torch.int32, device=d)}
    o2 = {k: v.clone() for k, v in o1.items()}
    for k in range(3):
        g = workloads.normal(shape, 740 + k, d, std=0.05)
        e8q.e8q_ste_backward(g, w_latent=w1, lr=0.5)
        e8q.e8q_project_hadamard_restore(w1, s, sg, hb, o1["wh"], o1["st"], two_z_out=o1["tz"], core_bound=16,
                                         esc_count_out=o1["esc"])
        e8q.e8q_sgd_project_hadamard_restore(w2, g, 0.5, s, sg, hb, o2["wh"], o2["st"], two_z_out=o2["tz"],
                                             core_bound=16, esc_count_out=o2["esc"])
        torch.cuda.synchronize()
        assert torch.equal(w1.view(torch.int16), w2.view(torch.int16)), f"latents, step {k}"
        _same({"q": o1["wh"], "tz": o1["tz"], "esc": o1["esc"], "st": o1["st"]},
              {"q": o2["wh"], "tz": o2["tz"], "esc": o2["esc"], "st": o2["st"]})


@pytest.mark.parametrize("hb,shape,q_dtype,tz", [(128, (2, 24, 1024), torch.bfloat16, True),
                                               (16, (1, 12, 272), torch.bfloat16, True),
                                               (1024, (1, 16, 2048), torch.bfloat16, True),
                                               (8, (3, 5, 136), torch.float32, False)])
def test_fused_rotated_grad_matches_unfused(hb, shape, q_dtype, tz):
    """The gradient taken back through the rotation: latents, q, escape counts
    and status bit for bit as e8q_ste_backward_hadamard +
    e8q_project_hadamard, also with non-finite gradient values."""
    d = device()
    w = workloads.normal(shape, 750 + hb, d)
    s = workloads.rms_scale(w, 1.5)
    sg = workloads.signs(shape[2], 751, d)
    w1, w2 = w.clone(), w.clone()
    o1, o2 = _outputs(w, q_dtype, tz), _outputs(w, q_dtype, tz)
    for k in range(3):
        g = workloads.normal(shape, 760 + k, d, std=0.05)
        if k == 2:
            g[0, 1, 3] = float("nan")
            g[0, 2 % shape[1], 5] = float("inf")
        e8q.e8q_ste_backward_hadamard(g, sg, hb, w_latent=w1, lr=0.5)
        e8q.e8q_project_hadamard(w1, s, sg, hb, o1["st"], q_out=o1["q"], two_z_out=o1["tz"], core_bound=16,
                                 esc_count_out=o1["esc"])
        e8q.e8q_sgd_rotated_project_hadamard(w2, g, 0.5, s, sg, hb, o2["st"], q_out=o2["q"], two_z_out=o2["tz"],
                                             core_bound=16, esc_count_out=o2["esc"])
        torch.cuda.synchronize()
        assert torch.equal(w1.view(torch.int16), w2.view(torch.int16)), f"latents, step {k}"
        _same(o1, o2)
