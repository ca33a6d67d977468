"""The allocation-free encode entry point against the allocating one: the same
inputs give bit-identical outputs, on two calls in a row whose second input is
smaller (the shared scratch keeps the first call's contents), and a shape
whose workspace exceeds the fixed scratch is refused before anything runs."""

import numpy as np
import pytest
import torch

import bit_e8_lattice_amd as e8q
from bit_e8_lattice_amd import workloads
from gpu_util import device, u16

pytestmark = pytest.mark.gpu


def _outputs(w, s, sg, hb, bound, noalloc, two_z):
    d = w.device
    batch, rows, cols = w.shape
    groups = batch * rows * cols // 8
    core = torch.full((groups,), -7, dtype=torch.int16, device=d)
    esc = torch.zeros(groups * e8q.ESCAPE_RECORD_BYTES, dtype=torch.uint8, device=d)
    cnt = torch.full((batch,), -1, dtype=torch.int64, device=d)
    st = torch.zeros(1, dtype=torch.int32, device=d)
    tz = torch.zeros(w.shape, dtype=torch.int8, device=d) if two_z else None
    if noalloc:
        e8q.e8q_encode_core_escape_noalloc(w, s, bound, core, esc, cnt, st, signs=sg, had_block=hb, two_z_out=tz)
    else:
        ws = torch.empty(e8q.e8q_encode_workspace_size(batch, rows, cols), dtype=torch.uint8, device=d)
        e8q.e8q_encode_core_escape(w, s, bound, core, esc, cnt, ws, st, signs=sg, had_block=hb, two_z_out=tz)
    torch.cuda.synchronize()
    n = int(cnt.sum().item())
    out = {"core": u16(core), "cnt": cnt.cpu().numpy(), "rec": esc[: n * 20].cpu().numpy(),
           "status": int(st.item())}
    if two_z:
        out["two_z"] = tz.cpu().numpy()
    return out


def _same(a, b):
    assert a.keys() == b.keys()
    for k in a:
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k


@pytest.mark.parametrize("two_z", [False, True])
def test_noalloc_matches_workspace_entry_point(two_z):
    d = device()
    # first call: 64 dense-decoder-shaped rows of 11008 columns in 3 batch items,
    # 256-wide blocks, alpha 1.2 (many escapes, tiles past the staging limit)
    w1 = workloads.normal((3, 64, 11008), 9101, d)
    s1 = workloads.rms_scale(w1, 1.2)
    g1 = workloads.signs(11008, 9102, d)
    # second call, smaller: 2 items of 40 x 4096, 128-wide blocks, alpha 3
    w2 = workloads.normal((2, 40, 4096), 9103, d)
    s2 = workloads.rms_scale(w2, 3.0)
    g2 = workloads.signs(4096, 9104, d)
    ref1 = _outputs(w1, s1, g1, 256, 16, False, two_z)
    ref2 = _outputs(w2, s2, g2, 128, 16, False, two_z)
    got1 = _outputs(w1, s1, g1, 256, 16, True, two_z)
    got2 = _outputs(w2, s2, g2, 128, 16, True, two_z)
    assert ref1["cnt"].sum() > 16 * 3 and ref1["status"] == 0
    _same(got1, ref1)
    _same(got2, ref2)


def test_noalloc_refuses_shapes_past_its_scratch():
    d = device()
    w = torch.zeros((1, 8, 8), dtype=torch.bfloat16, device=d)
    L = e8q.lib()
    # a shape whose workspace exceeds the scratch: refused by the host check
    # (the pointers are never touched)
    rows, cols = 1 << 20, 8192
    assert L.e8q_encode_workspace_size(1, rows, cols) > e8q.ENCODE_NOALLOC_SCRATCH_BYTES
    p = w.data_ptr()
    code = L.e8q_encode_core_escape_noalloc(p, 1, 1, rows, cols, p, None, 0, 16, p, None, 0, p, None, p, None)
    assert code == 5
    assert b"scratch" in L.e8q_status_string(code)
