"""Seeded synthetic inputs for the E8 projection path.

This module only draws random tensors and computes the per-row scales that the
library takes as an input; it holds none of the projection arithmetic.  Tests,
the benchmark and the smoke check use it to feed the HIP library and the CPU
oracle the same bits (tensors are drawn on one device and copied to the other).

Workloads (weights are stand-ins for LLM linear / expert-FFN weights; no real
checkpoint is involved):

* ``small_f32``      one 256x256 float32 matrix, N(0, 0.02^2), scale = row RMS,
                     no rotation;
* ``linear_4096``    one 4096x4096 bf16 matrix, N(0, 0.02^2), random signs and
                     128-wide Walsh-Hadamard blocks, scale = row RMS;
* ``moe_experts``    128 experts x {gate 768x2048, up 768x2048, down 2048x768},
                     bf16, Student-t (nu = 4) scaled to std 0.02, 128-wide
                     rotation, scale = 3 x row RMS (1 x in the stress run);
* ``dense_decoder``  32 blocks x {q, k, v, o 4096x4096; gate, up 11008x4096;
                     down 4096x11008}, bf16 N(0, 0.02^2), 128-wide rotation,
                     scale = 3 x row RMS; batched by shape (three tensors);
* ``qat_loop``       one 4096x14336 bf16 latent matrix, N(0, 0.02^2), 128-wide
                     rotation, scale = 3 x row RMS, and per-step gradients
                     N(0, 1e-4^2) in bf16.

Seeds are fixed per tensor so any matrix can be regenerated alone.
"""

from dataclasses import dataclass, field
from typing import List, Tuple

import torch

STD = 0.02


@dataclass
class Batch:
    """One batched launch: ``w`` [batch, rows, cols], per-row ``scale``
    [batch*rows] float32, per-column ``signs`` int8 (or None), block size."""
    name: str
    w: torch.Tensor
    scale: torch.Tensor
    signs: torch.Tensor = None
    had_block: int = 0
    seeds: List[int] = field(default_factory=list)


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, seed, device, std=STD, dtype=torch.bfloat16):
    """N(0, std^2) drawn in float32, rounded once to ``dtype``."""
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return (x * std).to(dtype)


def student_t4(shape, seed, device, std=STD, dtype=torch.bfloat16):
    """Student-t with 4 degrees of freedom scaled to standard deviation ``std``:
    t = Z0 / sqrt((Z1^2 + ... + Z4^2) / 4), w = std * t / sqrt(2) (Var t4 = 2)."""
    g = _gen(seed, device)
    z = torch.randn((5,) + tuple(shape), generator=g, device=device, dtype=torch.float32)
    chi = (z[1:] * z[1:]).sum(0) / 4.0
    t = z[0] / torch.sqrt(chi)
    return (t * (std / 2.0 ** 0.5)).to(dtype)


def signs(cols, seed, device):
    """Random +-1 column signs (int8)."""
    g = _gen(seed, device)
    b = torch.randint(0, 2, (cols,), generator=g, device=device, dtype=torch.int8)
    return (b * 2 - 1).to(torch.int8)


def rms_scale(w, alpha=1.0):
    """Per-row ``fl32(alpha * sqrt(mean(w^2)))``, accumulated in float64.
    ``w`` [..., cols] -> float32 [prod(leading dims)]."""
    cols = w.shape[-1]
    flat = w.reshape(-1, cols)
    out = torch.empty(flat.shape[0], dtype=torch.float32, device=w.device)
    step = max(1, (1 << 24) // cols)
    for lo in range(0, flat.shape[0], step):
        part = flat[lo:lo + step].to(torch.float64)
        out[lo:lo + step] = (alpha * torch.sqrt((part * part).mean(dim=1))).to(torch.float32)
    return out


# ------------------------------------------------------------------ workloads

def small_f32(device="cpu"):
    w = normal((1, 256, 256), 11, device, dtype=torch.float32)
    return Batch("small_f32 256x256 f32", w, rms_scale(w, 1.0), None, 0, [11])


def linear_4096(device="cpu", rows=4096, cols=4096, had_block=128):
    w = normal((1, rows, cols), 21, device)
    return Batch(f"linear {rows}x{cols} bf16", w, rms_scale(w, 1.0),
                 signs(cols, 22, device), had_block, [21])


MOE_KINDS = {"gate": (768, 2048, 0), "up": (768, 2048, 1), "down": (2048, 768, 2)}


def moe_experts(device="cpu", kind="gate", experts=128, alpha=3.0, had_block=128):
    rows, cols, k = MOE_KINDS[kind]
    w = torch.empty((experts, rows, cols), dtype=torch.bfloat16, device=device)
    seeds = []
    for e in range(experts):
        sd = 30000 + e * 3 + k
        w[e] = student_t4((rows, cols), sd, device)
        seeds.append(sd)
    sg = signs(cols, 3001 if cols == 2048 else 3002, device)
    return Batch(f"moe {experts}x{kind} {rows}x{cols} bf16 t4", w, rms_scale(w, alpha),
                 sg, had_block, seeds)


DECODER_MATS = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]


def dense_decoder_shapes(blocks=32) -> List[Tuple[str, int, int, List[int]]]:
    """The three batched launches of the dense decoder: (name, rows, cols, seeds).
    Seeds are 4100 + matrix index, layer-major in q, k, v, o, gate, up, down order."""
    groups = {}
    for blk in range(blocks):
        for j, (nm, r, c) in enumerate(DECODER_MATS):
            groups.setdefault((r, c), []).append(4100 + blk * len(DECODER_MATS) + j)
    out = []
    for (r, c), sds in groups.items():
        out.append((f"decoder {len(sds)}x {r}x{c} bf16", r, c, sds))
    return out


def dense_decoder(device="cpu", blocks=32, alpha=3.0, had_block=128, rows_limit=None):
    """Returns three ``Batch`` objects (4096x4096, 11008x4096, 4096x11008).
    ``rows_limit`` keeps only the first rows of every matrix (for small tests)."""
    out = []
    for name, r, c, sds in dense_decoder_shapes(blocks):
        rr = r if rows_limit is None else min(r, rows_limit)
        w = torch.empty((len(sds), rr, c), dtype=torch.bfloat16, device=device)
        for i, sd in enumerate(sds):
            w[i] = normal((r, c), sd, device)[:rr]
        sg = signs(c, 4001 if c == 4096 else 4002, device)
        out.append(Batch(name, w, rms_scale(w, alpha), sg, had_block, sds))
    return out


def qat_loop(device="cpu", rows=4096, cols=14336, alpha=3.0, had_block=128):
    w = normal((1, rows, cols), 51, device)
    return Batch(f"qat latent {rows}x{cols} bf16", w, rms_scale(w, alpha),
                 signs(cols, 52, device), had_block, [51])


def qat_grad(step, shape, device="cpu"):
    """Gradient passed through the identity STE at ``step``: N(0, 1e-4^2), bf16."""
    return normal(shape, 5300 + step, device, std=1e-4)
