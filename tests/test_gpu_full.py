"""Full-size parity and determinism of the workloads the benchmark times.

Every output of the full-size launches is compared with the CPU oracle (run in
the forked workers of oracle_pool, matrix by matrix): all 384 MoE expert
matrices at 3 x and 1 x row RMS, all 224 dense-decoder matrices, and the
4096x14336 QAT loop's escape count at every one of its 100 steps (with q and
2z in full at steps 0, 1 and 99).  Determinism: every workload run twice gives
bit-identical outputs."""

import numpy as np
import pytest
import torch

import bit_e8_lattice_amd as e8q
import oracle
import oracle_pool
from bit_e8_lattice_amd import workloads
from gpu_util import device, first_mismatch, u16, wbits

pytestmark = [pytest.mark.gpu, pytest.mark.oracle_pool]


def _encode(b, bound=16, cap=None):
    """GPU encode of one batched launch; device tensors."""
    d = b.w.device
    nb, rows, cols = b.w.shape
    groups = nb * rows * cols // 8
    cap = groups if cap is None else cap
    o = {"core": torch.empty(groups, dtype=torch.int16, device=d),
         "esc": torch.empty(cap * e8q.ESCAPE_RECORD_BYTES, dtype=torch.uint8, device=d),
         "cnt": torch.empty(nb, dtype=torch.int64, device=d),
         "st": torch.zeros(1, dtype=torch.int32, device=d)}
    ws = torch.empty(e8q.e8q_encode_workspace_size(nb, rows, cols), dtype=torch.uint8, device=d)
    e8q.e8q_encode_core_escape(b.w, b.scale, bound, o["core"], o["esc"], o["cnt"], ws, o["st"], signs=b.signs,
                               had_block=b.had_block)
    torch.cuda.synchronize()
    return o


def _check_launch_against_oracle(b, o, bound=16, ahead=3):
    """Every matrix of the launch: core indices, records (order included),
    count; the launch's status word equals the OR of the oracle's."""
    nb, rows, cols = b.w.shape
    gpm = rows * cols // 8
    counts = o["cnt"].cpu().numpy()
    off = np.concatenate([[0], np.cumsum(counts)])
    n = int(off[-1])
    recs = o["esc"][: n * 20].cpu().numpy().view(oracle.ESCAPE_RECORD_DTYPE)
    core = u16(o["core"]).reshape(nb, gpm)
    signs = b.signs.cpu().numpy()
    scale = b.scale.cpu().numpy()
    status = 0
    pending = []

    def check(m, h):
        nonlocal status
        ref_core, ref_rec, ref_cnt, st = oracle_pool.encode_result(h)
        status |= st
        assert first_mismatch(core[m], ref_core) is None, f"matrix {m}: core index {first_mismatch(core[m], ref_core)}"
        assert counts[m] == ref_cnt, f"matrix {m}: count {counts[m]} != {ref_cnt}"
        seg = recs[off[m]:off[m + 1]]
        assert np.array_equal(seg, ref_rec), f"matrix {m}: escape records differ"

    for m in range(nb):
        pending.append((m, oracle_pool.encode_matrix_async(wbits(b.w[m]), scale[m * rows:(m + 1) * rows], signs,
                                                           b.had_block, bound)))
        if len(pending) > ahead:
            check(*pending.pop(0))
    while pending:
        check(*pending.pop(0))
    assert int(o["st"].item()) == status


@pytest.mark.parametrize("alpha", [3.0, 1.0])
def test_moe_experts_full(alpha):
    """All 128 experts x {gate, up, down}: Student-t weights, 128-wide
    rotation, core ||2z||^2 <= 16; alpha 3 (sparse escapes) and 1 (most groups
    escape, every record compared)."""
    d = device()
    for kind in ("gate", "up", "down"):
        b = workloads.moe_experts(d, kind, alpha=alpha)
        o = _encode(b)
        _check_launch_against_oracle(b, o)
        del b, o
        torch.cuda.empty_cache()


def test_dense_decoder_full():
    """All 224 matrices of the 32-block dense decoder in the benchmark's three
    launches, every matrix compared with the oracle."""
    d = device()
    for b in workloads.dense_decoder(d):
        o = _encode(b, cap=b.w.numel() // 8 // 16)
        _check_launch_against_oracle(b, o)
        del b, o
        torch.cuda.empty_cache()


def test_qat_loop_full():
    """4096x14336 latents, 100 steps of rotated projection (+ escape count)
    then identity STE fused with SGD (lr 1): the oracle's escape count of the
    GPU's latents at every step; q and 2z in full at steps 0, 1 and 99; the
    SGD update in full at steps 0, 1 and 98."""
    d = device()
    b = workloads.qat_loop(d)
    w = b.w[0].clone()
    s = b.scale
    sn, gn = s.cpu().numpy(), b.signs.cpu().numpy()
    q = torch.empty_like(w)
    tz = torch.empty(w.shape, dtype=torch.int8, device=d)
    esc = torch.zeros(100, dtype=torch.int64, device=d)
    st = torch.zeros(1, dtype=torch.int32, device=d)
    pending = []
    for k in range(100):
        w_host = wbits(w)
        e8q.e8q_project_hadamard(w, s, b.signs, 128, st, q_out=q, two_z_out=tz, core_bound=16,
                                 esc_count_out=esc[k:k + 1])
        g = workloads.qat_grad(k, w.shape, d)
        if k in (0, 1, 99):
            rq, rtz, rcnt, rst = oracle_pool.project_matrix(w_host, sn, gn, 128, 16)
            assert first_mismatch(u16(q).reshape(-1), rq.reshape(-1)) is None, f"step {k}: q"
            assert np.array_equal(tz.cpu().numpy(), rtz), f"step {k}: 2z"
            assert int(esc[k].item()) == rcnt and rst == 0
        else:
            pending.append((k, oracle_pool.escape_count_async(w_host, sn, gn, 128, 16)))
        g_host = wbits(g) if k in (0, 1, 98) else None
        e8q.e8q_ste_backward(g, w_latent=w, lr=1.0)
        if g_host is not None:
            ref_w = oracle.sgd_update(w_host, g_host, 1.0)
            assert first_mismatch(wbits(w).reshape(-1), ref_w.reshape(-1)) is None, f"step {k}: SGD"
        while len(pending) > 4:
            kk, h = pending.pop(0)
            assert int(esc[kk].item()) == sum(h.get()), f"step {kk}: escape count"
    for kk, h in pending:
        assert int(esc[kk].item()) == sum(h.get()), f"step {kk}: escape count"
    assert int(st.item()) == 0


def test_determinism_every_workload():
    """Each workload run twice on the GPU: bit-identical outputs (escape order
    and counts included; scheduling must not change any bit)."""
    d = device()
    # 256x256 float32 and 4096x4096 bf16 projections
    for b in (workloads.small_f32(d), workloads.linear_4096(d)):
        outs = []
        for _ in range(2):
            q = torch.empty_like(b.w)
            tz = torch.empty(b.w.shape, dtype=torch.int8, device=d)
            st = torch.zeros(1, dtype=torch.int32, device=d)
            if b.signs is None:
                e8q.e8q_project(b.w, b.scale, st, q_out=q, two_z_out=tz)
            else:
                e8q.e8q_project_hadamard(b.w, b.scale, b.signs, b.had_block, st, q_out=q, two_z_out=tz)
            outs.append((q, tz, st))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0].view(torch.int16) if b.w.dtype == torch.bfloat16 else outs[0][0].view(torch.int32),
                           outs[1][0].view(torch.int16) if b.w.dtype == torch.bfloat16 else outs[1][0].view(torch.int32))
        assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][2], outs[1][2])
    # MoE stacks (alpha 3 and 1) and the dense decoder: encode twice
    launches = [workloads.moe_experts(d, k, alpha=a) for a in (3.0, 1.0) for k in ("gate", "up", "down")]
    for b in launches + workloads.dense_decoder(d):
        cap = b.w.numel() // 8 // (16 if b.w.shape[0] <= 128 and b.w.shape[1] * b.w.shape[2] > 8_000_000 else 1)
        o1, o2 = _encode(b, cap=cap), _encode(b, cap=cap)
        n = int(o1["cnt"].sum().item())
        assert torch.equal(o1["core"], o2["core"]) and torch.equal(o1["cnt"], o2["cnt"])
        assert torch.equal(o1["esc"][: n * 20], o2["esc"][: n * 20]) and torch.equal(o1["st"], o2["st"])
        del o1, o2
    del launches
    torch.cuda.empty_cache()
    # the 100-step QAT loop twice: escape series and final latents
    b = workloads.qat_loop(d)
    runs = []
    for _ in range(2):
        w = b.w[0].clone()
        q = torch.empty_like(w)
        esc = torch.zeros(100, dtype=torch.int64, device=d)
        st = torch.zeros(1, dtype=torch.int32, device=d)
        for k in range(100):
            e8q.e8q_project_hadamard(w, b.scale, b.signs, 128, st, q_out=q, core_bound=16, esc_count_out=esc[k:k + 1])
            e8q.e8q_ste_backward(workloads.qat_grad(k, w.shape, d), w_latent=w, lr=1.0)
        runs.append((w, q, esc, st))
    torch.cuda.synchronize()
    for x, y in zip(runs[0], runs[1]):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x, y.view(torch.int16) if y.dtype == torch.bfloat16 else y)
