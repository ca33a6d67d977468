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

SOURCES = ["e8q_common.hip", "e8q_tables.hip", "e8q_project.hip", "e8q_encode.hip", "e8q_ste.hip",
           "e8q_decode.hip", "e8q_roots.hip", "e8q_ptq.hip"]
# host program run before the library is compiled: writes the device table
# blob and its layout header (embedded by e8q_tables.hip)
TABLEGEN_SOURCES = ["e8q_tablegen.cpp", "e8q_tables_build.cpp", "e8q_core_table.cpp"]

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


def gen_tables(tmpdir, verbose=False):
    """Compile and run the table generator; the blob and header land in tmpdir."""
    exe = os.path.join(tmpdir, "e8q_tablegen")
    cxx = shutil.which("g++") or shutil.which("c++")
    if not cxx:
        raise RuntimeError("no host C++ compiler for the table generator")
    cmd = [cxx, "-O2", "-std=c++17", "-I", CSRC, "-o", exe] + [os.path.join(CSRC, s) for s in TABLEGEN_SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"table generator build failed:\n{res.stdout}{res.stderr}")
    res = subprocess.run([exe, tmpdir], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"table generator failed ({res.returncode}):\n{res.stdout}{res.stderr}")


# Host-only sanitizers for the CPU checks of the C ABI: the host code gets
# AddressSanitizer and UndefinedBehaviorSanitizer (every report fatal); the
# device code is built as usual (at -O1, since it never runs there).
SANITIZE_HOST = ["-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined"]
SANITIZE_LINK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]


def _compile_and_link(tmpdir, out, flags, link_flags, verbose, jobs):
    gen_tables(tmpdir, verbose)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(tmpdir, src + ".o")
        cmd = [hipcc()] + flags + SOURCE_FLAGS.get(src, []) + ["-I", INCLUDE, "-I", CSRC, "-I", tmpdir,
                                                               f"--embed-dir={tmpdir}", "-c",
                                                               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        objs.append(obj)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
        while sum(p.poll() is None for p in procs) >= jobs:
            procs[[p.poll() is None for p in procs].index(True)].wait()
    failed = []
    for src, p in zip(SOURCES, procs):
        o, e = p.communicate()
        res = subprocess.CompletedProcess(p.args, p.returncode, o, e)
        if p.returncode != 0:
            failed.append(f"{src}:\n{_filtered(res)}")
        elif verbose and _filtered(res):
            print(_filtered(res), file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + link_flags + ["-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{_filtered(res)}")
    os.replace(tmp, out)
    return out


def _jobs(jobs):
    return jobs or min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))


def build(verbose=False, jobs=None):
    with tempfile.TemporaryDirectory(prefix="e8q_build_") as tmpdir:
        return _compile_and_link(tmpdir, LIB, FLAGS, [], verbose, _jobs(jobs))


def build_host_sanitized(out_dir, verbose=False, jobs=None):
    """``out_dir/libe8q_sanitized.so``: the library with its host code under
    ASan + UBSan (load it with the ASan runtime preloaded; see
    ``asan_runtime``)."""
    flags = ["-O1" if f == "-O3" else f for f in FLAGS] + SANITIZE_HOST
    with tempfile.TemporaryDirectory(prefix="e8q_build_san_") as tmpdir:
        return _compile_and_link(tmpdir, os.path.join(out_dir, "libe8q_sanitized.so"), flags, SANITIZE_LINK,
                                 verbose, _jobs(jobs))


def asan_runtime():
    """Path of the compiler's shared ASan runtime."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip().splitlines()[-1] if res.returncode == 0 and res.stdout.strip() else ""
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("ASan runtime not found")
    return path


if __name__ == "__main__":
    print(build(verbose=True))
