"""GPU parity of e8q_ste_backward (identity STE, fused SGD) and of the
simulated QAT loop (forward projection + STE + SGD on one latent matrix)."""

import numpy as np
import pytest
import torch

import bit_e8_lattice_amd as e8q
import oracle
from bit_e8_lattice_amd import workloads
from gpu_util import device, first_mismatch, run_project, u16, wbits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [1, 7, 8, 4096, 4096 * 3 + 5])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ste_identity_and_sgd(n, dtype):
    d = device()
    g = workloads.normal((n,), 11 + n, d, std=1e-4, dtype=dtype)
    w = workloads.normal((n,), 12 + n, d, dtype=dtype)
    gw = torch.empty_like(g)
    w0 = w.clone()
    e8q.e8q_ste_backward(g, grad_w=gw, w_latent=w, lr=0.75)
    torch.cuda.synchronize()
    if dtype == torch.bfloat16:
        assert np.array_equal(u16(gw), u16(g))
        want = oracle.sgd_update(u16(w0), u16(g), 0.75)
        assert first_mismatch(u16(w), want) is None
    else:
        assert np.array_equal(gw.cpu().numpy().view(np.uint32), g.cpu().numpy().view(np.uint32))
        want = oracle.sgd_update(w0.cpu().numpy(), g.cpu().numpy(), 0.75, is_bf16=False)
        assert first_mismatch(w.cpu().numpy().view(np.uint32), want.view(np.uint32)) is None


def test_ste_unaligned_views():
    d = device()
    base_g = workloads.normal((1000,), 3, d, std=1e-4)
    base_w = workloads.normal((1000,), 4, d)
    g = base_g[3:]                 # 6-byte offset: not 16-byte aligned
    w_view = base_w[1:998]         # 2-byte offset
    w0 = u16(w_view)
    e8q.e8q_ste_backward(g, w_latent=w_view, lr=1.0)
    torch.cuda.synchronize()
    assert first_mismatch(u16(w_view), oracle.sgd_update(w0, u16(g), 1.0)) is None


def test_ste_nan_canonical():
    d = device()
    g = torch.tensor([float("nan"), 1.0, float("inf"), 0.0] * 4, dtype=torch.bfloat16, device=d)
    w = torch.tensor([1.0, float("nan"), float("inf"), 2.0] * 4, dtype=torch.bfloat16, device=d)
    w0 = u16(w)
    e8q.e8q_ste_backward(g, w_latent=w, lr=1.0)
    torch.cuda.synchronize()
    assert first_mismatch(u16(w), oracle.sgd_update(w0, u16(g), 1.0)) is None


def _oracle_rows_loop(w_rows, s_rows, signs, grads, steps):
    """Oracle QAT loop restricted to a set of rows (rows evolve independently)."""
    hist = []
    w = w_rows.copy()
    for k in range(steps):
        p = oracle.project(w, s_rows, signs, 128, core_bound=16)
        hist.append((p["q_bf16"].reshape(w.shape), p["two_z_i8"].reshape(w.shape)))
        w = oracle.sgd_update(w, grads[k], 1.0)
    return w, hist


def test_qat_loop_full_size_sampled_rows():
    """4096x14336 latents, 100 steps of project(+escape count) then STE/SGD;
    six sampled rows followed step by step through the oracle; every tenth
    step's escape count checked against the GPU's own 2z; step 0 checked in
    full."""
    d = device()
    b = workloads.qat_loop(d)
    rows, cols = b.w.shape[1], b.w.shape[2]
    w = b.w[0].clone()
    s = b.scale
    rsel = np.array([0, 1, 777, 2048, 4000, rows - 1])
    w_rows0 = wbits(w)[rsel]
    grads_rows = []
    steps = 100
    q = torch.empty_like(w)
    tz = torch.empty(w.shape, dtype=torch.int8, device=d)
    esc = torch.empty(1, dtype=torch.int64, device=d)
    st = torch.zeros(1, dtype=torch.int32, device=d)
    for k in range(steps):
        if k == 0:
            w_full = wbits(w)
        e8q.e8q_project_hadamard(w, s, b.signs, 128, st, q_out=q, two_z_out=tz, core_bound=16,
                                 esc_count_out=esc)
        g = workloads.qat_grad(k, w.shape, d)
        grads_rows.append(wbits(g)[rsel])
        if k % 10 == 0 or k == steps - 1:
            tz_np = tz.cpu().numpy().astype(np.int64).reshape(-1, 8)
            assert int(esc.item()) == int(((tz_np * tz_np).sum(1) > 16).sum())
        if k == 0:
            ref = oracle.project(w_full, s.cpu().numpy(), b.signs.cpu().numpy(), 128, core_bound=16)
            assert first_mismatch(u16(q).reshape(-1), ref["q_bf16"].reshape(-1)) is None
            assert int(esc.item()) == int(ref["esc_count"][0])
        if k == 0:
            q_rows0 = u16(q)[rsel]
        if k == steps - 1:
            q_rows_last = u16(q)[rsel]
        e8q.e8q_ste_backward(g, w_latent=w, lr=1.0)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    w_end, hist = _oracle_rows_loop(w_rows0, s.cpu().numpy()[rsel], b.signs.cpu().numpy(),
                                    grads_rows, steps)
    assert np.array_equal(hist[0][0], q_rows0)
    assert np.array_equal(hist[-1][0], q_rows_last)
    assert first_mismatch(wbits(w)[rsel], w_end) is None
