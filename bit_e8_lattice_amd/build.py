"""Build the gfx950 shared library ``libe8q.so`` in-tree with hipcc.

Every source is compiled to an object in parallel (the kernels of one file
call nothing on the device in another), then the objects are linked.

Usage: ``python -m bit_e8_lattice_amd.build`` (or ``__graft_entry__.build()``).
"""

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libe8q.so")

SOURCES = ["e8q_common.hip", "e8q_project.hip", "e8q_encode.hip", "e8q_ste.hip", "e8q_decode.hip",
           "e8q_roots.hip", "e8q_ptq.hip", "e8q_core_table.cpp"]

# -ffp-contract=off: every float32 step is one IEEE operation (no fused
# multiply-add), which the bit-exact contract in include/e8q.h relies on.
# Packed FP32 instructions are disabled for the device code.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Per-source additions.  The PTQ search and the GEMV keep their MFMA
# accumulators in ordinary VGPRs (no copies out of the accumulation registers).
SOURCE_FLAGS = {"e8q_ptq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "e8q_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _filtered(res):
    return "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())


def build(verbose=False, jobs=None):
    jobs = jobs or min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with tempfile.TemporaryDirectory(prefix="e8q_build_") as tmpdir:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            cmd = [hipcc()] + FLAGS + SOURCE_FLAGS.get(src, []) + ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            objs.append(obj)
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
            while sum(p.poll() is None for p in procs) >= jobs:
                procs[[p.poll() is None for p in procs].index(True)].wait()
        failed = []
        for src, p in zip(SOURCES, procs):
            out, err = p.communicate()
            res = subprocess.CompletedProcess(p.args, p.returncode, out, err)
            if p.returncode != 0:
                failed.append(f"{src}:\n{_filtered(res)}")
            elif verbose and _filtered(res):
                print(_filtered(res), file=sys.stderr)
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
        tmp = LIB + ".tmp"
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{_filtered(res)}")
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
