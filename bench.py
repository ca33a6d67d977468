#!/usr/bin/env python3
"""Benchmark: E8 projection + 2-bit core/escape encoding of a dense decoder's weights.

One step = one encode pass (nearest E8 point after a 128-wide randomized
Walsh-Hadamard rotation, 16-bit core index, compacted escape records) over
every linear weight of a 32-block dense decoder: per block q, k, v, o
4096x4096, gate and up 11008x4096, down 4096x11008 (6,476,005,376 bf16
weights, N(0, 0.02^2), scale 3 x row RMS, core ||2z||^2 <= 16), issued as
three launches batched by shape.  Inputs are generated on the GPU and resident
in HBM before timing starts.

Prints one JSON line.  ``roofline`` is the encode launches' algorithmic HBM
bytes per launch over their mean duration (HIP events on the launching stream)
against the 8 TB/s HBM peak.  ``cpu_baseline`` is the CPU oracle timed on the
same input bits (block 0 of the decoder), with the oracle's rate on every other
workload and on one core in ``detail.cpu_oracle``; the oracle's workers are
forked before the GPU is touched.

``--config`` picks another workload for manual runs (the default is the one
above): ``decoder_alpha1`` (scale 1 x RMS, most groups escape),
``decoder_wide`` (whole-row 4096 / 256-column rotation blocks), ``linear``
(4096x4096 rotated projection), ``moe`` / ``moe_alpha1`` (128-expert stacks),
``qat`` (STE/SGD fused with the next forward projection on 4096x14336, one
kernel per step, escape count of every step in ``detail``), ``qat_unfused``,
``qat_restore``, ``qat_restore_unfused``, ``qat_rotated_grad``, ``qat_rotated_grad_unfused``,
``decode``, ``decode_q``, ``gemv``, ``pack``, ``ptq``.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "encode_dense_decoder_traffic.json")
# the encode kernel, its rank table and its launch configuration
KERNEL_SOURCES = ["e8q_device.hpp", "e8q_point.hpp", "e8q_encode.hip", "e8q_core_table.cpp", "e8q_core_table.hpp",
                  "e8q_host.hpp"]


def kernel_hash():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_e8_lattice_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# --------------------------------------------------------------- CPU baseline
#
# The oracle runs in single-threaded workers forked before the GPU is touched
# (a process that has initialised HIP must not fork).  The parent draws the
# inputs on the GPU, copies their bits into an anonymous shared mapping that
# the workers inherited, and hands out row chunks by offset, so the oracle
# sees exactly the bits the GPU encoded and the timing covers compute only.

_SHM = None                    # anonymous shared mapping, created before the fork
SHM_BYTES = 448 << 20          # largest sample: one decoder block (405 MB of bf16) + scales + signs


def _oracle_job(job):
    """One chunk: ``job`` = (kind, (w_off, w_shape, w_dtype), (s_off, n_s), (sg_off, n_sg) or None,
    had_block, core_bound).  Returns (weights, seconds of compute)."""
    import numpy as np
    import oracle
    kind, (w_off, w_shape, w_dt), (s_off, n_s), sg, hb, bound = job
    n = int(np.prod(w_shape))
    w = np.frombuffer(_SHM, dtype=w_dt, count=n, offset=w_off).reshape(w_shape)
    s = np.frombuffer(_SHM, dtype=np.float32, count=n_s, offset=s_off)
    signs = None if sg is None else np.frombuffer(_SHM, dtype=np.int8, count=sg[1], offset=sg[0])
    t0 = time.perf_counter()
    if kind == "encode":
        oracle.encode_core_escape(w, s, signs, hb, bound)
    else:                       # projection with dequantization (and escape count when bound >= 0)
        oracle.project(w, s, signs, hb, w_is_bf16=(w_dt == np.uint16), core_bound=bound)
    return n, time.perf_counter() - t0


class OraclePool:
    """Forked oracle workers (one per core, at most 16) and the shared input
    mapping; must be created before any GPU call."""

    def __init__(self):
        import multiprocessing as mp
        import mmap
        global _SHM
        _SHM = mmap.mmap(-1, SHM_BYTES)
        self.cores = min(16, len(os.sched_getaffinity(0)))
        self.pool = mp.get_context("fork").Pool(self.cores)
        self.single = mp.get_context("fork").Pool(1)

    def close(self):
        self.pool.terminate()
        self.single.terminate()

    def stage(self, tensors):
        """Copy host numpy arrays into the shared mapping; returns their offsets."""
        import numpy as np
        offs, pos = [], 0
        for a in tensors:
            a = np.ascontiguousarray(a)
            if pos + a.nbytes > SHM_BYTES:
                raise RuntimeError("oracle sample larger than the shared mapping")
            _SHM[pos:pos + a.nbytes] = a.tobytes()
            offs.append(pos)
            pos = (pos + a.nbytes + 255) & ~255
        return offs

    def run(self, kind, w, s, sg, hb, bound, chunk_rows, single=False):
        """Time the oracle on ``w`` [batch, rows, cols] (uint16 bf16 bits or float32),
        chunks of ``chunk_rows`` rows; returns (weights, wall s, cpu s, workers)."""
        import numpy as np
        batch, rows, cols = w.shape
        arrays = [w, s] + ([] if sg is None else [sg])
        offs = self.stage(arrays)
        sgd = None if sg is None else (offs[2], int(sg.size))
        jobs = []
        for b in range(batch):
            for lo in range(0, rows, chunk_rows):
                nr = min(chunk_rows, rows - lo)
                w_off = offs[0] + (b * rows + lo) * cols * w.dtype.itemsize
                s_off = offs[1] + (b * rows + lo) * 4
                jobs.append((kind, (w_off, (1, nr, cols), w.dtype), (s_off, nr), sgd, hb, bound))
        pool = self.single if single else self.pool
        t0 = time.perf_counter()
        res = pool.map(_oracle_job, jobs, chunksize=1)
        wall = time.perf_counter() - t0
        return sum(r[0] for r in res), wall, sum(r[1] for r in res), 1 if single else min(self.cores, len(jobs))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _host(t):
    """Device tensor -> host numpy array of the same bits (bf16 as uint16)."""
    import numpy as np
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def cpu_oracle_rates(pool, torch, workloads, decoder_batches):
    """The oracle's rate on every workload, on bounded samples of GPU-drawn
    inputs: the dense decoder's block 0 (all seven matrices; the headline
    sample), the 256x256 float32 matrix, the 4096x4096 projection (all cores
    and one core), 8 experts of each MoE kind and the 4096x14336 QAT forward.
    Returns (headline dict for ``cpu_baseline``, per-workload detail)."""
    dev = torch.device("cuda:0")
    per = {}

    def rec(name, r, what):
        n, wall, cpu_s, workers = r
        per[name] = {"gweights_per_s": round(n / wall / 1e9, 5), "weights": n, "workers": workers,
                     "wall_s": round(wall, 2), "cpu_s": round(cpu_s, 2), "sample": what}
        return r

    # dense decoder block 0: batch index 0-3 of 4096x4096 (q, k, v, o), 0-1 of
    # 11008x4096 (gate, up), 0 of 4096x11008 (down)
    firsts = {(4096, 4096): 4, (11008, 4096): 2, (4096, 11008): 1}
    tot = [0, 0.0, 0.0, 0]
    for b in decoder_batches:
        nb, rows, cols = b.w.shape
        k = firsts[(rows, cols)]
        r = pool.run("encode", _host(b.w[:k]), _host(b.scale[: k * rows]), _host(b.signs), 128, 16, 512)
        tot = [tot[0] + r[0], tot[1] + r[1], tot[2] + r[2], max(tot[3], r[3])]
    rec("dense_decoder", tuple(tot), "decoder block 0: all 7 matrices (q,k,v,o 4096x4096; gate,up 11008x4096; "
        "down 4096x11008), 128-wide rotation, 3x row RMS, core ||2z||^2<=16 encode")

    w = workloads.small_f32(dev)
    rec("small_f32", pool.run("project", _host(w.w), _host(w.scale), None, 0, -1, 64),
        "256x256 float32, no rotation, row RMS: projection + dequantization (whole matrix)")
    w = workloads.linear_4096(dev)
    hw, hs, hsg = _host(w.w), _host(w.scale), _host(w.signs)
    rec("linear_4096", pool.run("project", hw, hs, hsg, 128, -1, 256),
        "4096x4096 bf16, 128-wide rotation, row RMS: projection + dequantization (whole matrix)")
    rec("linear_4096_1core", pool.run("project", hw[:, :1024], hs[:1024], hsg, 128, -1, 256, single=True),
        "first 1024 rows of the 4096x4096 projection, one worker")
    del w
    tot = [0, 0.0, 0.0, 0]
    for kind in ("gate", "up", "down"):
        m = workloads.moe_experts(dev, kind, experts=8)
        r = pool.run("encode", _host(m.w), _host(m.scale), _host(m.signs), 128, 16, 256)
        tot = [tot[0] + r[0], tot[1] + r[1], tot[2] + r[2], max(tot[3], r[3])]
    rec("moe_experts", tuple(tot), "experts 0-7 of each kind (gate, up 768x2048; down 2048x768), Student-t, "
        "128-wide rotation, 3x row RMS, core ||2z||^2<=16 encode")
    q = workloads.qat_loop(dev)
    rec("qat_forward", pool.run("project", _host(q.w), _host(q.scale), _host(q.signs), 128, 16, 256),
        "4096x14336 bf16 latents, 128-wide rotation, 3x row RMS: projection + dequantization + escape count "
        "(one QAT forward, whole matrix)")
    del q
    d = per["dense_decoder"]
    head = {
        "value": d["gweights_per_s"],
        "unit": "Gweights/s",
        "cores": d["workers"],
        "kind": "oracle",
        "sample": (f"{d['weights']} weights: all 7 matrices of decoder block 0, the GPU's own input bits "
                   f"(same seeds, scales, signs), {d['cpu_s']:.1f} s of CPU time over {d['wall_s']:.1f} s wall, "
                   f"single-threaded numpy workers on {_cpu_model()}"),
    }
    return head, {"cpu_model": _cpu_model(), "per_workload": per}


# --------------------------------------------------------------------- GPU

def encode_bytes(batch, escapes):
    """Algorithmic HBM bytes of one encode launch: read weights, scales and
    signs; write core indices, escape records and per-batch counts."""
    nb, rows, cols = batch.w.shape
    weights = nb * rows * cols
    return (2 * weights + 4 * nb * rows + cols + 2 * (weights // 8) + 20 * escapes + 8 * nb)


def run_dense_decoder(args, torch, e8q, workloads, alpha=3.0, wide=False):
    """All 224 matrices, three launches per step.  ``wide``: whole-row
    power-of-two rotation blocks (4096 columns on 4096-wide rows, 256 on the
    11008-wide rows) instead of 128."""
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    batches = workloads.dense_decoder(dev, alpha=alpha)
    if wide:
        for b in batches:
            b.had_block = 4096 if b.w.shape[2] == 4096 else 256
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    bufs = []
    for b in batches:
        nb, rows, cols = b.w.shape
        groups = nb * rows * cols // 8
        cap = groups // 16 if alpha >= 2.0 else groups
        bufs.append({
            "core": torch.empty(groups, dtype=torch.int16, device=dev),
            "esc": torch.empty(cap * e8q.ESCAPE_RECORD_BYTES, dtype=torch.uint8, device=dev),
            "cnt": torch.empty(nb, dtype=torch.int64, device=dev),
            "ws": torch.empty(e8q.e8q_encode_workspace_size(nb, rows, cols), dtype=torch.uint8, device=dev),
        })
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def step(evs=None):
        for i, (b, o) in enumerate(zip(batches, bufs)):
            if evs is not None:
                evs[i][0].record()
            e8q.e8q_encode_core_escape(b.w, b.scale, 16, o["core"], o["esc"], o["cnt"], o["ws"], status,
                                       signs=b.signs, had_block=b.had_block)
            if evs is not None:
                evs[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in batches] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [[evs[k][i][0].elapsed_time(evs[k][i][1]) for i in range(len(batches))]
                 for k in range(args.steps)]
    st = int(status.item())
    escapes = [int(o["cnt"].sum().item()) for o in bufs]
    weights = sum(b.w.numel() for b in batches)
    groups = weights // 8
    alg_bytes = [encode_bytes(b, e) for b, e in zip(batches, escapes)]
    kernel_ms = sum(sum(r) for r in launch_ms) / args.steps          # per step, all 3 launches
    achieved = sum(alg_bytes) / (kernel_ms * 1e-3) / 1e9
    rho = sum(escapes) / groups
    traffic = None   # measured HBM bytes: per launch (mean of the three) and per step
    if os.path.exists(TRAFFIC_FILE) and alpha == 3.0 and not wide:
        tf = json.load(open(TRAFFIC_FILE))
        if tf.get("kernel_hash") == kernel_hash():
            per = [x["read"] + x["write"] for x in tf["per_launch_bytes"]]
            traffic = {"per_launch": round(sum(per) / len(per)), "per_step": tf.get("bytes_per_step"),
                       "ratio_to_algorithmic": tf.get("ratio_to_algorithmic"),
                       "valu_per_group": tf.get("valu_per_group")}
    return {
        "batches": batches, "weights": weights, "wall": wall, "status": st, "escapes": escapes, "rho": rho,
        "alg_bytes": alg_bytes, "launch_ms": launch_ms, "kernel_ms": kernel_ms, "achieved": achieved,
        "traffic": traffic, "gen_s": t_gen,
        "launches": [f"{b.w.shape[0]}x{b.w.shape[1]}x{b.w.shape[2]}" for b in batches],
    }


def run_decode(args, torch, e8q, workloads, kind):
    """Decode of the whole dense decoder's exported form (encoded once,
    untimed; the weights are then freed): ``decode`` writes the restored bf16
    weights in the original basis, ``decode_q`` the bf16 q in the rotated basis.
    Three launches per step, one per matrix shape."""
    dev = torch.device("cuda:0")
    batches = workloads.dense_decoder(dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    enc = []
    for b in batches:
        nb, rows, cols = b.w.shape
        groups = nb * rows * cols // 8
        core = torch.empty(groups, dtype=torch.int16, device=dev)
        esc = torch.empty((groups // 16) * e8q.ESCAPE_RECORD_BYTES, dtype=torch.uint8, device=dev)
        cnt = torch.empty(nb, dtype=torch.int64, device=dev)
        ws = torch.empty(e8q.e8q_encode_workspace_size(nb, rows, cols), dtype=torch.uint8, device=dev)
        e8q.e8q_encode_core_escape(b.w, b.scale, 16, core, esc, cnt, ws, status, signs=b.signs, had_block=128)
        torch.cuda.synchronize()
        enc.append({"shape": (nb, rows, cols), "core": core, "esc": esc, "cnt": cnt, "scale": b.scale,
                    "signs": b.signs, "escapes": int(cnt.sum().item()),
                    "out": torch.empty((nb, rows, cols), dtype=torch.bfloat16, device=dev),
                    "ws": torch.empty(e8q.e8q_decode_workspace_size(nb), dtype=torch.uint8, device=dev)})
        b.w = None
        del ws
    torch.cuda.empty_cache()

    def part(e):
        def fn(k):
            if kind == "decode":
                e8q.e8q_decode_core_escape(e["core"], e["esc"], e["cnt"], e["shape"], 16, e["ws"], status,
                                           row_scale=e["scale"], signs=e["signs"], had_block=128,
                                           w_hat_out=e["out"])
            else:
                e8q.e8q_decode_core_escape(e["core"], e["esc"], e["cnt"], e["shape"], 16, e["ws"], status,
                                           row_scale=e["scale"], q_out=e["out"])
        return fn

    parts = []
    for e in enc:
        nb, rows, cols = e["shape"]
        n = nb * rows * cols
        # index 0.25 B/w, records, counts, scales, signs (restore) in; 2 B/w out
        bpw = (2 * (n // 8) + 20 * e["escapes"] + 8 * nb + 4 * nb * rows
               + (cols if kind == "decode" else 0) + 2 * n) / n
        parts.append((f"{nb}x{rows}x{cols}", part(e), bpw, n))
    n = sum(e["out"].numel() for e in enc)
    alg = sum(bpw * pw for (_, _, bpw, pw) in parts)
    what = ("restored bf16 weights in the original basis (inverse 128-wide Walsh-Hadamard, sign flip)"
            if kind == "decode" else "bf16 q = s z in the rotated basis")
    r = _time_launches(args, torch, parts, n, alg, status,
                       "dense decoder 32 blocks x (q,k,v,o 4096x4096; gate,up 11008x4096; down 4096x11008): "
                       f"core ||2z||^2<=16 indices + escape records decoded to {what}")
    r["escapes"] = sum(e["escapes"] for e in enc)
    return r


def run_gemv(args, torch, e8q, workloads):
    """Decode-step products of all 224 dense-decoder matrices with one bf16
    activation vector each (m = --gemv-m), straight from the exported form
    (encoded once, untimed); the same products in BF16 (torch.bmm of the
    decoded bf16 weights, hipBLASLt) are timed alongside as the reference
    representation."""
    dev = torch.device("cuda:0")
    batches = workloads.dense_decoder(dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    m = args.gemv_m
    enc = []
    for i, b in enumerate(batches):
        nb, rows, cols = b.w.shape
        groups = nb * rows * cols // 8
        core = torch.empty(groups, dtype=torch.int16, device=dev)
        esc = torch.empty((groups // 16) * e8q.ESCAPE_RECORD_BYTES, dtype=torch.uint8, device=dev)
        cnt = torch.empty(nb, dtype=torch.int64, device=dev)
        ws = torch.empty(e8q.e8q_encode_workspace_size(nb, rows, cols), dtype=torch.uint8, device=dev)
        e8q.e8q_encode_core_escape(b.w, b.scale, 16, core, esc, cnt, ws, status, signs=b.signs, had_block=128)
        wh = torch.empty_like(b.w)
        dws = torch.empty(e8q.e8q_decode_workspace_size(nb), dtype=torch.uint8, device=dev)
        e8q.e8q_decode_core_escape(core, esc, cnt, (nb, rows, cols), 16, dws, status, row_scale=b.scale,
                                   signs=b.signs, had_block=128, w_hat_out=wh)
        g = torch.Generator(device=dev).manual_seed(6000 + i)
        x = torch.randn((nb, m, cols), generator=g, device=dev).to(torch.bfloat16)
        enc.append({"shape": (nb, rows, cols), "core": core, "esc": esc, "cnt": cnt, "scale": b.scale,
                    "signs": b.signs, "x": x, "xt": x.transpose(1, 2).contiguous(), "w_hat": wh,
                    "y": torch.empty((nb, m, rows), dtype=torch.float32, device=dev),
                    "yb": torch.empty((nb, rows, m), dtype=torch.bfloat16, device=dev),
                    "ws": torch.empty(e8q.e8q_gemv_workspace_size(nb, m, rows, cols), dtype=torch.uint8, device=dev)})
        b.w = None
        del ws, dws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    def part(e):
        def fn(k):
            e8q.e8q_gemv_core_escape(e["core"], e["esc"], e["cnt"], e["shape"], 16, e["scale"], e["x"], e["y"],
                                     e["ws"], status, signs=e["signs"], had_block=128)
        return fn

    def part_bf16(e):
        def fn(k):
            torch.bmm(e["w_hat"], e["xt"], out=e["yb"])
        return fn

    parts, parts_bf16 = [], []
    for e in enc:
        nb, rows, cols = e["shape"]
        n = nb * rows * cols
        parts.append((f"{nb}x{rows}x{cols}", part(e), (2 * (n // 8) + 4 * nb * rows + 2 * nb * m * cols) / n, n))
        parts_bf16.append((f"bf16 {nb}x{rows}x{cols}", part_bf16(e), 2.0, n))
    n = sum(p[3] for p in parts)
    alg = sum(p[2] * p[3] for p in parts)
    r = _time_launches(args, torch, parts, n, alg, status,
                       f"2-bit GEMV, dense decoder 224 matrices (q,k,v,o 4096x4096; gate,up 11008x4096; "
                       f"down 4096x11008) x {m} bf16 activation vector(s) each, from core ||2z||^2<=16 indices "
                       "+ escape records, 128-wide rotation")
    rb = _time_launches(args, torch, parts_bf16, n, 2 * n, status, "bf16 torch.bmm of the decoded weights")
    r["parts"].update(rb["parts"])
    r["parts"]["bf16_ms_per_step"] = round(rb["kernel_ms"], 4)
    r["parts"]["speedup_vs_bf16"] = round(rb["kernel_ms"] / r["kernel_ms"], 3)
    return r


def run_pack(args, torch, e8q, workloads):
    """Root packing of every escape record of the dense decoder encoded at
    scale 2 x row RMS (about 30 M records; encoded once, untimed): pack and
    unpack timed per step, three launch shapes."""
    dev = torch.device("cuda:0")
    batches = workloads.dense_decoder(dev, alpha=2.0)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    sets = []
    for b in batches:
        nb, rows, cols = b.w.shape
        groups = nb * rows * cols // 8
        core = torch.empty(groups, dtype=torch.int16, device=dev)
        esc = torch.empty((groups // 8) * e8q.ESCAPE_RECORD_BYTES, dtype=torch.uint8, device=dev)
        cnt = torch.empty(nb, dtype=torch.int64, device=dev)
        ws = torch.empty(e8q.e8q_encode_workspace_size(nb, rows, cols), dtype=torch.uint8, device=dev)
        e8q.e8q_encode_core_escape(b.w, b.scale, 16, core, esc, cnt, ws, status, signs=b.signs, had_block=128)
        torch.cuda.synchronize()
        n = int(cnt.sum().item())
        b.w = None
        del core, ws
        sets.append({"n": n, "esc": esc[: n * 20], "packed": torch.empty(n * 8, dtype=torch.uint8, device=dev),
                     "wide": torch.empty(n * 20, dtype=torch.uint8, device=dev),
                     "wcnt": torch.empty(1, dtype=torch.int64, device=dev),
                     "out": torch.empty(n * 20, dtype=torch.uint8, device=dev),
                     "ws": torch.empty(e8q.e8q_pack_workspace_size(n), dtype=torch.uint8, device=dev),
                     "groups": groups})
    torch.cuda.empty_cache()

    def pack(e):
        return lambda k: e8q.e8q_pack_escapes(e["esc"], e["n"], 16, e["packed"], e["wide"], e["wcnt"], e["ws"], status)

    def unpack(e):
        return lambda k: e8q.e8q_unpack_escapes(e["packed"], e["n"], e["wide"], e["wcnt_host"], 16, e["out"],
                                                e["ws"], status)

    nrec = sum(e["n"] for e in sets)
    parts = [(f"pack {i}", pack(e), 28.0, e["n"]) for i, e in enumerate(sets)]
    r = _time_launches(args, torch, parts, nrec, 28 * nrec, status,
                       "root packing of the dense decoder's escape records (scale 2x row RMS, core ||2z||^2<=16)")
    for e in sets:
        e["wcnt_host"] = int(e["wcnt"].item())
    ru = _time_launches(args, torch, [(f"unpack {i}", unpack(e), 28.0, e["n"]) for i, e in enumerate(sets)],
                        nrec, 28 * nrec, status, "unpack")
    r["parts"].update(ru["parts"])
    wide = sum(e["wcnt_host"] for e in sets)
    groups = sum(e["groups"] for e in sets)
    rho = nrec / groups
    r["parts"]["records"] = nrec
    r["parts"]["wide_records"] = wide
    r["parts"]["payload_bits_20B"] = round(2 + 20 * rho, 6)
    r["parts"]["payload_bits_packed"] = round(2 + (8 * nrec + 20 * wide) * 8 / (8 * groups), 6)
    r["unit_override"] = "Grecords/s"
    return r


PTQ_ALPHAS = [0.75, 1.0, 1.5, 2.0, 2.5, 3.0]


def run_ptq(args, torch, e8q, workloads):
    """PTQ initialization of one dense-decoder block (q, k, v, o 4096x4096;
    gate, up 11008x4096; down 4096x11008; 202 M weights) onto C(16): scale
    search over 6 multipliers of the row RMS, then the finite-core projection;
    three launches per step."""
    dev = torch.device("cuda:0")
    batches = workloads.dense_decoder(dev, blocks=1, alpha=1.0)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    al = torch.tensor(PTQ_ALPHAS, dtype=torch.float32, device=dev)
    sets = []
    for b in batches:
        nb, rows, cols = b.w.shape
        sets.append({"b": b, "scale": torch.empty(nb * rows, dtype=torch.float32, device=dev),
                     "choice": torch.empty(nb * rows, dtype=torch.int32, device=dev),
                     "core": torch.empty(nb * rows * cols // 8, dtype=torch.int16, device=dev),
                     "tz": torch.empty((nb, rows, cols), dtype=torch.int8, device=dev),
                     "ws": torch.empty(e8q.e8q_ptq_workspace_size(nb, rows, cols), dtype=torch.uint8, device=dev)})

    def part(e):
        b = e["b"]
        return lambda k: e8q.e8q_ptq_init(b.w, b.scale, al, 16, e["scale"], e["core"], e["tz"], e["ws"], status,
                                          signs=b.signs, had_block=128, choice_out=e["choice"])

    parts = []
    for e in sets:
        nb, rows, cols = e["b"].w.shape
        n = nb * rows * cols
        # weights in, transform written and read back per candidate, points out
        parts.append((f"{nb}x{rows}x{cols}", part(e), 2 + 4 + 4 * (len(PTQ_ALPHAS) + 1) + 1.25, n))
    n = sum(p[3] for p in parts)
    r = _time_launches(args, torch, parts, n, sum(p[2] * p[3] for p in parts), status,
                       "PTQ init of one dense-decoder block (q,k,v,o 4096x4096; gate,up 11008x4096; down "
                       "4096x11008) bf16 N(0,0.02^2) onto core ||2z||^2<=16: per-row scale search over "
                       f"{PTQ_ALPHAS} x row RMS, finite-core projection")
    ch = torch.cat([e["choice"] for e in sets]).cpu()
    r["parts"]["choice_histogram"] = [int((ch == k).sum()) for k in range(len(PTQ_ALPHAS))]
    return r


def run_linear(args, torch, e8q, workloads):
    """4096x4096 bf16 rotated projection (q in bf16), cycling over 8 copies of
    the matrix (537 MB) so that the 256 MB last-level cache cannot hold the input."""
    dev = torch.device("cuda:0")
    b = workloads.linear_4096(dev)
    copies = 8
    ws = [b.w.clone() for _ in range(copies)]
    qs = [torch.empty_like(b.w) for _ in range(copies)]
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def launch(k):
        e8q.e8q_project_hadamard(ws[k % copies], b.scale, b.signs, 128, status, q_out=qs[k % copies])

    n = b.w.numel()
    return _time_launches(args, torch, launch, n, 4 * n + 4 * b.w.shape[1] + b.w.shape[2], status,
                          "linear 4096x4096 bf16 N(0,0.02^2); 128-wide Walsh-Hadamard; scale = row RMS; "
                          "E8 projection + dequant to bf16")


def run_moe(args, torch, e8q, workloads, alpha=3.0):
    """128 experts x {gate, up, down} Student-t weights, 128-wide rotation,
    scale alpha x RMS (3 by default, 1 for the stress run), encode (three
    launches per step)."""
    dev = torch.device("cuda:0")
    batches = [workloads.moe_experts(dev, k, alpha=alpha) for k in ("gate", "up", "down")]
    bufs = []
    for bt in batches:
        nb, rows, cols = bt.w.shape
        groups = nb * rows * cols // 8
        cap = groups // 16 if alpha >= 2.0 else groups
        bufs.append((torch.empty(groups, dtype=torch.int16, device=dev),
                     torch.empty(cap * e8q.ESCAPE_RECORD_BYTES, dtype=torch.uint8, device=dev),
                     torch.empty(nb, dtype=torch.int64, device=dev),
                     torch.empty(e8q.e8q_encode_workspace_size(nb, rows, cols), dtype=torch.uint8, device=dev)))
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def launch(k):
        for bt, (core, esc, cnt, ws) in zip(batches, bufs):
            e8q.e8q_encode_core_escape(bt.w, bt.scale, 16, core, esc, cnt, ws, status, signs=bt.signs, had_block=128)

    n = sum(bt.w.numel() for bt in batches)
    r = _time_launches(args, torch, launch, n, None, status,
                       "moe 128 experts x (gate 768x2048, up 768x2048, down 2048x768) bf16 Student-t nu=4 std 0.02; "
                       f"128-wide Walsh-Hadamard; scale {alpha:g}x row RMS; core ||2z||^2<=16 encode, "
                       "per-expert escapes")
    esc = sum(int(b[2].sum().item()) for b in bufs)
    r["alg_bytes"] = sum(encode_bytes(bt, int(b[2].sum().item())) for bt, b in zip(batches, bufs))
    r["escapes"] = esc
    return r


def run_qat(args, torch, e8q, workloads, mode="qat"):
    """One step of the simulated QAT loop on 4096x14336 bf16 latents (lr 1,
    gradients N(0, 1e-4^2) drawn before timing, one per step):

    * ``qat``: one kernel per step: the identity STE with SGD on the latents
      (the previous step's gradient) fused with the projection in the rotated
      basis (q bf16 + escape count);
    * ``qat_unfused``: the same step as two kernels, projection then STE + SGD;
    * ``qat_restore``: one kernel per step: the identity STE (exact for the
      composite) with SGD fused with the projection restored to the original
      basis; ``qat_restore_unfused`` the same step as two kernels;
    * ``qat_rotated_grad``: one kernel per step: the gradient taken back through
      the rotation (R^T) with SGD fused with the rotated projection;
      ``qat_rotated_grad_unfused`` the same step as two kernels.
    """
    dev = torch.device("cuda:0")
    b = workloads.qat_loop(dev)
    w = b.w[0].clone()
    q = torch.empty_like(w)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    nsteps = args.steps + args.warmup
    esc = torch.zeros(nsteps, dtype=torch.int64, device=dev)    # escape count of every step
    grads = [workloads.qat_grad(k, w.shape, dev) for k in range(nsteps)]

    def fwd_rotated(k):
        e8q.e8q_project_hadamard(w, b.scale, b.signs, 128, status, q_out=q, core_bound=16,
                                 esc_count_out=esc[k:k + 1])

    def fwd_restore(k):
        e8q.e8q_project_hadamard_restore(w, b.scale, b.signs, 128, q, status, core_bound=16,
                                         esc_count_out=esc[k:k + 1])

    def bwd_identity(k):
        e8q.e8q_ste_backward(grads[k], w_latent=w, lr=1.0)

    def bwd_rotated(k):
        e8q.e8q_ste_backward_hadamard(grads[k], b.signs, 128, w_latent=w, lr=1.0)

    def sgd_fwd_restore(k):
        e8q.e8q_sgd_project_hadamard_restore(w, grads[k - 1] if k > 0 else grads[-1], 1.0, b.scale, b.signs, 128, q,
                                             status, core_bound=16, esc_count_out=esc[k:k + 1])

    def sgd_fwd_rotated(k):
        e8q.e8q_sgd_rotated_project_hadamard(w, grads[k - 1] if k > 0 else grads[-1], 1.0, b.scale, b.signs, 128,
                                             status, q_out=q, core_bound=16, esc_count_out=esc[k:k + 1])

    def sgd_fwd(k):
        # the previous step's gradient applied to the latents, then this step's projection
        e8q.e8q_sgd_project_hadamard(w, grads[k - 1] if k > 0 else grads[-1], 1.0, b.scale, status, signs=b.signs,
                                     had_block=128, q_out=q, core_bound=16, esc_count_out=esc[k:k + 1])

    parts, desc = {
        "qat": ([("sgd_project_hadamard", sgd_fwd, 8)],
                "identity STE with SGD on the latents fused with the next 128-wide rotated projection + escape "
                "count (one kernel per step)"),
        "qat_unfused": ([("project_hadamard", fwd_rotated, 4), ("ste_backward", bwd_identity, 6)],
                        "128-wide rotated projection + escape count, then identity STE fused with SGD (two "
                        "kernels per step)"),
        "qat_restore": ([("sgd_project_hadamard_restore", sgd_fwd_restore, 8)],
                        "identity STE with SGD on the latents fused with the next 128-wide projection restored to "
                        "the original basis + escape count (one kernel per step)"),
        "qat_restore_unfused": ([("project_hadamard_restore", fwd_restore, 4), ("ste_backward", bwd_identity, 6)],
                                "128-wide projection restored to the original basis + escape count, then "
                                "identity STE fused with SGD (two kernels per step)"),
        "qat_rotated_grad": ([("sgd_rotated_project_hadamard", sgd_fwd_rotated, 8)],
                             "gradient through R^T with SGD on the latents fused with the next 128-wide rotated "
                             "projection + escape count (one kernel per step)"),
        "qat_rotated_grad_unfused": ([("project_hadamard", fwd_rotated, 4), ("ste_backward_hadamard", bwd_rotated, 6)],
                             "128-wide rotated projection + escape count, gradient through R^T "
                             "fused with SGD"),
    }[mode]
    n = w.numel()
    r = _time_launches(args, torch, parts, n, sum(p[2] for p in parts) * n, status,
                       f"qat step 4096x14336 bf16 latents: {desc} (lr 1, grad N(0,1e-4^2))",
                       steps_offset=True)
    series = esc.cpu().tolist()
    r["parts"]["escapes_per_step"] = series          # warmup steps first, then the timed steps
    r["parts"]["escapes_first_last"] = [series[0], series[-1]]
    r["parts"]["escapes_min_mean_max"] = [min(series), sum(series) / len(series), max(series)]
    r["escapes"] = series[-1]
    return r


def _time_launches(args, torch, parts, weights, bytes_per_step, status, workload, steps_offset=False):
    """``parts``: [(name, launch(k), algorithmic bytes per weight)], run in order
    each step; events around each part give per-part kernel time."""
    if callable(parts):
        parts = [("step", parts, None if bytes_per_step is None else bytes_per_step / weights)]
    parts = [p if len(p) == 4 else (p[0], p[1], p[2], weights) for p in parts]
    for k in range(args.warmup):
        for _, fn, _, _ in parts:
            fn(k)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        evs[k][0].record()
        for i, (_, fn, _, _) in enumerate(parts):
            fn(k + args.warmup if steps_offset else k)
            evs[k][i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    part_ms = [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps for i in range(len(parts))]
    detail = {name: {"ms": round(m, 4), "alg_bytes_per_weight": None if bpw is None else round(bpw, 4),
                     "hbm_gbs": None if bpw is None else round(bpw * pw / (m * 1e-3) / 1e9, 1)}
              for (name, _, bpw, pw), m in zip(parts, part_ms)}
    return {"weights": weights, "wall": wall, "kernel_ms": sum(part_ms), "alg_bytes": bytes_per_step,
            "status": int(status.item()), "workload": workload, "parts": detail}


DECODER_CONFIGS = {"decoder": (3.0, False), "decoder_alpha1": (1.0, False), "decoder_wide": (3.0, True)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="decoder",
                    choices=list(DECODER_CONFIGS) + ["linear", "moe", "moe_alpha1", "qat", "qat_unfused", "qat_restore",
                                                     "qat_restore_unfused", "qat_rotated_grad",
                                                     "qat_rotated_grad_unfused", "decode", "decode_q", "gemv", "pack",
                                                     "ptq"])
    ap.add_argument("--gemv-m", type=int, default=1, choices=[1, 2])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 4 GiB device copy (known bytes) for counter scaling")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the encode shards by whole matrices with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)

    # the oracle's workers are forked before anything touches the GPU
    pool = OraclePool() if (not args.no_cpu_baseline and args.config == "decoder") else None

    import torch
    import bit_e8_lattice_amd as e8q
    from bit_e8_lattice_amd import workloads
    e8q.lib()
    if args.copy_calibration:
        n = 1 << 30                       # 4 GiB of float32 read, 4 GiB written
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.config not in DECODER_CONFIGS:
        if args.config.startswith("qat"):
            r = run_qat(args, torch, e8q, workloads, args.config)
        elif args.config == "gemv":
            r = run_gemv(args, torch, e8q, workloads)
        elif args.config == "pack":
            r = run_pack(args, torch, e8q, workloads)
        elif args.config == "ptq":
            r = run_ptq(args, torch, e8q, workloads)
        elif args.config.startswith("decode"):
            r = run_decode(args, torch, e8q, workloads, args.config)
        elif args.config.startswith("moe"):
            r = run_moe(args, torch, e8q, workloads, alpha=1.0 if args.config == "moe_alpha1" else 3.0)
        else:
            r = run_linear(args, torch, e8q, workloads)
        gbs = r["alg_bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
        out = {
            "metric": f"{args.config}: {r.get('unit_override', 'Gweights/s')} and % of HBM peak BW, 1xMI355X",
            "value": round(r["weights"] * args.steps / r["wall"] / 1e9, 3),
            "unit": r.get("unit_override", "Gweights/s"), "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(r["wall"] * 1e3 / args.steps, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": r["workload"], "weights": r["weights"]},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
            "cpu_baseline": None,
            "detail": {"kernel_ms_per_step": round(r["kernel_ms"], 4), "alg_bytes_per_step": r["alg_bytes"],
                       "escapes": r.get("escapes"), "status": r["status"], "parts": r.get("parts")},
        }
        print(json.dumps(out), flush=True)
        return

    alpha, wide = DECODER_CONFIGS[args.config]
    r = run_dense_decoder(args, torch, e8q, workloads, alpha=alpha, wide=wide)
    if r["status"] != 0:
        print(f"warning: device status bits {r['status']:#x}", file=sys.stderr)
    cpu, cpu_detail = None, None
    if pool is not None:
        try:
            cpu, cpu_detail = cpu_oracle_rates(pool, torch, workloads, r["batches"])
        finally:
            pool.close()

    ms_per_step = r["wall"] * 1e3 / args.steps
    value = r["weights"] * args.steps / r["wall"] / 1e9
    # roofline of the encode launches: algorithmic bytes per launch over the
    # launch's mean duration (HIP events on the launching stream, timed steps only)
    nl = len(r["launches"])
    launch_mean_ms = [sum(x[i] for x in r["launch_ms"]) / args.steps for i in range(nl)]
    bytes_per_launch = sum(r["alg_bytes"]) / nl
    ms_per_launch = sum(launch_mean_ms) / nl
    achieved = bytes_per_launch / (ms_per_launch * 1e-3) / 1e9
    blocks = "4096 (4096-column rows) / 256 (11008-column rows)" if wide else "128"
    out = {
        "metric": "Gweights/s projected+encoded and % of HBM peak BW, 1xMI355X vs CPU oracle",
        "value": round(value, 3),
        "unit": "Gweights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": ("dense decoder 32 blocks x (q,k,v,o 4096x4096; gate,up 11008x4096; down 4096x11008) "
                         f"bf16 N(0,0.02^2); sign flip + {blocks}-column Walsh-Hadamard blocks; "
                         f"scale {alpha:g}x row RMS; E8 projection + core ||2z||^2<=16 index + escape records"),
            "weights": r["weights"],
            "launches": r["launches"],
            "core_bound": 16,
            "had_block": 0 if wide else 128,
            "alpha": alpha,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": r["traffic"]["per_launch"] if r["traffic"] else None,
        },
        "cpu_baseline": cpu,
        "detail": {
            "target_frac": 0.70,
            "kernel_ms_per_step": round(r["kernel_ms"], 4),
            "launch_ms_mean": [round(x, 4) for x in launch_mean_ms],
            "alg_bytes_per_step": sum(r["alg_bytes"]),
            "alg_bytes_per_launch": round(bytes_per_launch),
            "hbm_traffic_bytes_per_step": r["traffic"]["per_step"] if r["traffic"] else None,
            "hbm_traffic_ratio_to_algorithmic": r["traffic"]["ratio_to_algorithmic"] if r["traffic"] else None,
            "valu_per_group": r["traffic"].get("valu_per_group") if r["traffic"] else None,
            "escapes": sum(r["escapes"]),
            "rho": r["rho"],
            "payload_bits_per_weight": 2 + 20 * r["rho"],
            "status": r["status"],
            "input_gen_s": round(r["gen_s"], 1),
            "kernel_hash": kernel_hash(),
            "cpu_oracle": cpu_detail,
        },
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
