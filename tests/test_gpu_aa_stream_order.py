"""Calls are stream-ordered: the library's read-only tables are part of its
device code object (generated when the library is built), so no call
allocates, uploads or waits on the host.

The check: with a long kernel still running on the stream, calls for every
core-bound table set return before that kernel finishes, and their results
(taken after it) equal the oracle's.  This file is named to run first among the
GPU tests, so that these are the library's first calls in the process (the one
time a device's table and scratch addresses are looked up)."""

import time

import numpy as np
import pytest
import torch

import bit_e8_lattice_amd as e8q
import oracle
from bit_e8_lattice_amd import workloads
from gpu_util import device, u16, wbits

pytestmark = pytest.mark.gpu


def _sleep_cycles_for(seconds):
    """torch.cuda._sleep cycle count that keeps the GPU busy about ``seconds``
    (measured once, the clock it counts is the device's)."""
    n = 10_000_000
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    torch.cuda._sleep(n)
    torch.cuda.synchronize()
    dt = max(time.perf_counter() - t0, 1e-4)
    return int(n * seconds / dt)


def test_calls_do_not_wait_for_the_stream():
    d = device()
    w = workloads.normal((2, 32, 1024), 4711, d)
    s = workloads.rms_scale(w, 1.5)
    sg = workloads.signs(1024, 4712, d)
    batch, rows, cols = w.shape
    groups = batch * rows * cols // 8
    bounds = [0, 8, 16, 24, 32, 40]
    outs = []
    for _ in bounds:
        outs.append({"core": torch.empty(groups, dtype=torch.int16, device=d),
                     "esc": torch.empty(groups * e8q.ESCAPE_RECORD_BYTES, dtype=torch.uint8, device=d),
                     "cnt": torch.empty(batch, dtype=torch.int64, device=d),
                     "ws": torch.empty(e8q.e8q_encode_workspace_size(batch, rows, cols), dtype=torch.uint8,
                                       device=d),
                     "st": torch.zeros(1, dtype=torch.int32, device=d)})
    q = torch.empty_like(w)
    st = torch.zeros(1, dtype=torch.int32, device=d)
    cycles = _sleep_cycles_for(1.0)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    torch.cuda._sleep(cycles)              # about one second of GPU time on this stream
    for b, o in zip(bounds, outs):
        e8q.e8q_encode_core_escape(w, s, b, o["core"], o["esc"], o["cnt"], o["ws"], o["st"], signs=sg,
                                   had_block=128)
    e8q.e8q_project_hadamard(w, s, sg, 128, st, q_out=q)
    busy = not stream.query()
    host_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    assert busy, f"a call waited for the stream ({host_s:.3f} s on the host)"

    wb, sn, gn = wbits(w), s.cpu().numpy(), sg.cpu().numpy()
    for b, o in zip(bounds, outs):
        ref = oracle.encode_core_escape(wb, sn, gn, 128, b)
        assert np.array_equal(u16(o["core"]), ref["core_idx"]), f"core indices, bound {b}"
        assert o["cnt"].cpu().numpy().tolist() == ref["counts"].tolist(), f"counts, bound {b}"
        n = len(ref["records"])
        rec = o["esc"][: n * 20].cpu().numpy().view(oracle.ESCAPE_RECORD_DTYPE)
        assert np.array_equal(rec, ref["records"]), f"records, bound {b}"
        assert int(o["st"].item()) == 0
    refp = oracle.project(wb, sn, gn, 128)
    assert np.array_equal(u16(q), refp["q_bf16"])
