"""Edge cases on the GPU: the smallest input (one group) through every entry
point, the widest rows the LDS sign table allows, and an encode whose group
count passes 2^31 (32-bit index arithmetic), each against the oracle."""

import numpy as np
import pytest
import torch

import bit_e8_lattice_amd as e8q
import oracle
from bit_e8_lattice_amd import workloads
from gpu_util import (device, first_mismatch, run_decode, run_encode, run_project, run_restore, u16,
                      upload_export, wbits)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_single_group_everywhere(dtype):
    d = device()
    w = workloads.normal((1, 1, 8), 3100, d, dtype=dtype)
    w[0, 0, 3] = w[0, 0, 3] * 40          # one coordinate well outside: an escape at alpha 0.5
    s = workloads.rms_scale(w, 0.5)
    sg = workloads.signs(8, 3101, d)
    is_bf16 = dtype == torch.bfloat16
    wb, sn, gn = wbits(w), s.cpu().numpy(), sg.cpu().numpy()
    # projection without and with rotation, restore
    ref = oracle.project(wb, sn, w_is_bf16=is_bf16, core_bound=16)
    out = run_project(w, s, q_dtype=torch.float32, core_bound=16)
    assert np.array_equal(out["q"].view(np.uint32), ref["q_f32"].view(np.uint32))
    assert np.array_equal(out["two_z_i8"], ref["two_z_i8"]) and out["esc_count"].tolist() == ref["esc_count"].tolist()
    ref_r = oracle.project_restore(wb, sn, gn, 8, w_is_bf16=is_bf16)
    out_r = run_restore(w, s, sg, 8, out_dtype=torch.float32)
    assert np.array_equal(out_r["w_hat"].view(np.uint32), ref_r["w_hat_f32"].view(np.uint32))
    # encode and decode
    enc = oracle.encode_core_escape(wb, sn, gn, 8, 16, w_is_bf16=is_bf16)
    assert len(enc["records"]) == 1
    got = run_encode(w, s, 16, sg, 8)
    assert np.array_equal(got["core_idx"], enc["core_idx"]) and np.array_equal(got["records"], enc["records"])
    core, esc, cnt = upload_export(enc, d)
    dec = run_decode(core, esc, cnt, (1, 1, 8), 16, s, sg, 8, q_dtype=torch.float32, w_hat_dtype=torch.float32)
    ref_d = oracle.decode_outputs(enc["core_idx"], enc["records"], enc["counts"], 16, (1, 1, 8), sn, gn, 8)
    assert np.array_equal(dec["w_hat"].view(np.uint32), ref_d["w_hat_f32"].view(np.uint32))
    assert np.array_equal(dec["q"].view(np.uint32), ref_d["q_f32"].view(np.uint32))
    # rotated STE on one group
    g = workloads.normal((1, 8), 3102, d, dtype=dtype)
    gw = torch.empty_like(g)
    e8q.e8q_ste_backward_hadamard(g, sg, 8, grad_w=gw)
    torch.cuda.synchronize()
    ref_g, _ = oracle.ste_backward_hadamard(wbits(g), gn, 8, is_bf16)
    got_g = u16(gw) if is_bf16 else gw.cpu().numpy().view(np.uint32)
    assert np.array_equal(got_g, ref_g if is_bf16 else ref_g.view(np.uint32))


@pytest.mark.parametrize("cols,hb", [(30720, 128), (22528, 2048)])
def test_widest_rows(cols, hb):
    """The widest rows the LDS sign table allows (with the wide-block buffer for
    blocks over 128 columns)."""
    d = device()
    w = workloads.normal((1, 6, cols), 3200 + hb, d)
    s = workloads.rms_scale(w, 2.0)
    sg = workloads.signs(cols, 3201, d)
    out = run_project(w, s, sg, hb, core_bound=16)
    ref = oracle.project(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), hb, core_bound=16)
    assert np.array_equal(out["q"], ref["q_bf16"]) and np.array_equal(out["two_z_i8"], ref["two_z_i8"])
    got = run_encode(w, s, 16, sg, hb)
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), hb, 16)
    assert np.array_equal(got["core_idx"], enc["core_idx"]) and np.array_equal(got["records"], enc["records"])


def test_encode_past_2_31_groups():
    """2^31 + 2^17 groups in one launch (34 GB of bf16 weights): counts against
    the escape slots everywhere, rows at the start, around 2^30 and 2^31 groups
    and at the end exact against the oracle."""
    d = device()
    rows, cols = (1 << 21) + 128, 8192
    gpr = cols // 8
    w = torch.empty((1, rows, cols), dtype=torch.bfloat16, device=d)
    step = 1 << 15
    for i, lo in enumerate(range(0, rows, step)):
        n = min(step, rows - lo)
        w[0, lo:lo + n] = workloads.normal((n, cols), 3300 + i, d)
    s = workloads.rms_scale(w, 3.0)
    groups = rows * gpr
    assert groups > (1 << 31)
    out = run_encode(w, s, 16, cap=groups // 256, keep_device=True)
    core, esc, cnt = out["dev"]
    n_esc = int(cnt.item())
    assert int((core == -1).sum().item()) == n_esc and out["status"] == 0
    rsel = np.array([0, 1, (1 << 20) - 1, 1 << 20, (1 << 21) - 1, 1 << 21, rows - 2, rows - 1])
    ref = oracle.encode_core_escape(wbits(w[0, torch.from_numpy(rsel).to(d)]), s[torch.from_numpy(rsel).to(d)].cpu().numpy(),
                                    None, 0, 16)
    got_core = out["core_idx"].reshape(rows, gpr)[rsel].reshape(-1)
    assert first_mismatch(got_core, ref["core_idx"]) is None
    rec = out["records"]
    keep = np.isin(rec["group"].astype(np.int64) // gpr, rsel)
    want = ref["records"].copy()
    want["group"] = (rsel[want["group"].astype(np.int64) // gpr] * gpr + want["group"] % gpr).astype(np.uint32)
    assert np.array_equal(rec[keep], want)
    assert (np.diff(rec["group"].astype(np.int64)) > 0).all()
