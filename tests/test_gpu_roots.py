"""GPU parity of the root-packed escape records against the oracle: packed
records, the wide list and its count bit for bit, and the exact inverse."""

import numpy as np
import pytest
import torch

import bit_e8_lattice_amd as e8q
import oracle
from bit_e8_lattice_amd import workloads
from gpu_util import device, first_mismatch, run_encode, wbits

pytestmark = pytest.mark.gpu


def _pack(rec_np, bound, d, wide_cap=None):
    n = len(rec_np)
    esc = torch.from_numpy(rec_np.view(np.uint8).reshape(-1).copy()).to(d) if n else torch.empty(0, dtype=torch.uint8, device=d)
    packed = torch.empty(max(n, 1) * 8, dtype=torch.uint8, device=d)
    cap = n if wide_cap is None else wide_cap
    wide = torch.empty(max(cap, 1) * 20, dtype=torch.uint8, device=d)[: cap * 20] if cap else None
    cnt = torch.empty(1, dtype=torch.int64, device=d)
    ws = torch.empty(e8q.e8q_pack_workspace_size(n), dtype=torch.uint8, device=d)
    st = torch.zeros(1, dtype=torch.int32, device=d)
    e8q.e8q_pack_escapes(esc if n else None, n, bound, packed if n else None, wide, cnt, ws, st)
    torch.cuda.synchronize()
    nw = int(cnt.item())
    p = packed[: n * 8].cpu().numpy().view(oracle.PACKED_RECORD_DTYPE) if n else np.zeros(0, oracle.PACKED_RECORD_DTYPE)
    kept = min(nw, cap)
    w = wide[: kept * 20].cpu().numpy().view(oracle.ESCAPE_RECORD_DTYPE) if kept else np.zeros(0, oracle.ESCAPE_RECORD_DTYPE)
    return p, w, nw, int(st.item()), (packed, wide)


def _unpack(packed_dev, n, wide_dev, nw, bound, d):
    out = torch.empty(max(n, 1) * 20, dtype=torch.uint8, device=d)
    ws = torch.empty(e8q.e8q_pack_workspace_size(n), dtype=torch.uint8, device=d)
    st = torch.zeros(1, dtype=torch.int32, device=d)
    e8q.e8q_unpack_escapes(packed_dev, n, wide_dev if nw else None, nw, bound, out, ws, st)
    torch.cuda.synchronize()
    return out[: n * 20].cpu().numpy().view(oracle.ESCAPE_RECORD_DTYPE), int(st.item())


@pytest.mark.parametrize("bound", [8, 16, 24, 40])
@pytest.mark.parametrize("alpha", [1.0, 2.0])
def test_pack_unpack_oracle_records(bound, alpha):
    d = device()
    w = workloads.normal((2, 40, 2048), 2000 + bound, d)
    s = workloads.rms_scale(w, alpha)
    sg = workloads.signs(2048, 2001, d)
    enc = oracle.encode_core_escape(wbits(w), s.cpu().numpy(), sg.cpu().numpy(), 128, bound)
    rec = enc["records"]
    ref_p, ref_w = oracle.pack_escapes(rec, bound)
    p, wl, nw, st, dev = _pack(rec, bound, d)
    assert st == 0
    assert first_mismatch(p.view(np.uint64), ref_p.view(np.uint64)) is None
    assert nw == len(ref_w)
    assert np.array_equal(wl, ref_w)
    back, st2 = _unpack(dev[0], len(rec), dev[1], nw, bound, d)
    assert st2 == 0
    assert np.array_equal(back, rec)


def test_pack_device_encode_records_and_limits():
    """Records from the device encode (4 MoE down experts, alpha 1: about
    half a million records over many blocks); wide-list overflow; malformed
    packed records."""
    d = device()
    b = workloads.moe_experts(d, "down", experts=4, alpha=1.0)
    out = run_encode(b.w, b.scale, 16, b.signs, 128)
    rec = out["records"]
    assert 100000 < len(rec) < 2000000
    ref_p, ref_w = oracle.pack_escapes(rec, 16)
    p, wl, nw, st, dev = _pack(rec, 16, d)
    assert st == 0 and nw == len(ref_w)
    assert first_mismatch(p.view(np.uint64), ref_p.view(np.uint64)) is None
    assert np.array_equal(wl, ref_w)
    back, st2 = _unpack(dev[0], len(rec), dev[1], nw, 16, d)
    assert st2 == 0 and np.array_equal(back, rec)
    # wide list cut short
    small = rec[:5000]
    ref_p, ref_w = oracle.pack_escapes(small, 16)
    assert len(ref_w) > 10
    p, wl, nw, st, dev = _pack(small, 16, d, wide_cap=len(ref_w) - 3)
    assert st == oracle.STATUS_ESC_OVERFLOW and nw == len(ref_w)
    assert np.array_equal(wl, ref_w[:-3])
    back, st2 = _unpack(dev[0], len(small), dev[1], nw - 3, 16, d)
    assert st2 == oracle.STATUS_ESC_MISSING
    missing = np.nonzero(ref_p["root"] == oracle.ROOT_NONE)[0][-3:]
    assert (back["two_z"][missing] == 0).all()
    keep = np.setdiff1d(np.arange(len(small)), missing)
    assert np.array_equal(back[keep], small[keep])
    # a malformed packed record (root 250) decodes to zero
    bad = ref_p.copy()
    k = int(np.nonzero(bad["root"] != oracle.ROOT_NONE)[0][0])
    bad["root"][k] = 250
    pd = torch.from_numpy(bad.view(np.uint8).reshape(-1).copy()).to(d)
    wd = torch.from_numpy(ref_w.view(np.uint8).reshape(-1).copy()).to(d)
    back, st3 = _unpack(pd, len(small), wd, len(ref_w), 16, d)
    assert st3 == oracle.STATUS_BAD_INDEX and (back["two_z"][k] == 0).all()


def test_pack_empty():
    d = device()
    p, wl, nw, st, _ = _pack(np.zeros(0, oracle.ESCAPE_RECORD_DTYPE), 16, d)
    assert nw == 0 and st == 0
