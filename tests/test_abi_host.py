"""CPU-side checks of the C ABI: the library loads, exports every declared
symbol, host-only helpers agree with the oracle, and argument validation
rejects bad calls before anything is launched (no GPU needed)."""

import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# A build of the library whose host code is compiled with the address and
# undefined-behaviour sanitizers runs these checks when
# test_host_sanitizers.py names it here (its device code is not the product's).
HOST_ONLY_LIBRARY = os.environ.get("E8Q_TEST_HOST_ONLY_LIBRARY")
needs_device_code = pytest.mark.skipif(HOST_ONLY_LIBRARY is not None, reason="sanitized build: device code differs")


@pytest.fixture(scope="module")
def L():
    import bit_e8_lattice_amd as e8q
    if HOST_ONLY_LIBRARY:
        e8q.library_path = HOST_ONLY_LIBRARY
    elif not os.path.exists(e8q.library_path):
        from bit_e8_lattice_amd.build import build
        build()
    return e8q.lib()


def _declared():
    txt = open(os.path.join(ROOT, "include", "e8q.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(e8q_[a-z_0-9]+)\s*\(", txt)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert {"e8q_project", "e8q_project_hadamard", "e8q_encode_core_escape", "e8q_ste_backward"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_core_size_matches_oracle(L):
    for b in range(0, 41):
        assert L.e8q_core_size(b) == oracle.core_size(b)
    assert L.e8q_core_size(-1) == -1 and L.e8q_core_size(41) == -1


def test_strings(L):
    assert L.e8q_status_string(0) == b"ok"
    assert b"invalid" in L.e8q_status_string(1)
    assert b"gfx950" in L.e8q_version()


def test_workspace_size(L):
    assert L.e8q_encode_workspace_size(1, 1, 12) == 0
    assert L.e8q_encode_workspace_size(0, 4, 8) == 0
    groups = 128 * 4096 * 4096 // 8
    tiles = (groups + 4095) // 4096
    a256 = lambda v: (v + 255) // 256 * 256
    # counter, tile status words, row coefficients, per-tile counts, 16 staged records per tile
    assert L.e8q_encode_workspace_size(128, 4096, 4096) == (256 + a256(8 * tiles) + a256(4 * 128 * 4096)
                                                          + a256(4 * tiles) + a256(20 * 16 * tiles))


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first


@pytest.mark.parametrize("args", [
    # (w, dtype, batch, rows, cols, scale, q, qdt, two_z, bound, esc, status)
    (None, 1, 1, 4, 16, FAKE, FAKE, 1, None, -1, None, FAKE),
    (FAKE, 1, 1, 4, 12, FAKE, FAKE, 1, None, -1, None, FAKE),       # cols % 8
    (FAKE, 1, 0, 4, 16, FAKE, FAKE, 1, None, -1, None, FAKE),       # batch
    (FAKE, 7, 1, 4, 16, FAKE, FAKE, 1, None, -1, None, FAKE),       # dtype
    (FAKE, 1, 1, 4, 16, None, FAKE, 1, None, -1, None, FAKE),       # scale
    (FAKE, 1, 1, 4, 16, FAKE, FAKE, 1, None, -1, None, None),       # status
    (FAKE, 1, 1, 4, 16, FAKE, None, 1, None, -1, None, FAKE),       # no output
    (FAKE, 1, 1, 4, 16, FAKE, None, 1, None, -1, FAKE, FAKE),       # esc without bound
])
def test_project_rejects(L, args):
    assert L.e8q_project(*args, None) == 1


@pytest.mark.parametrize("signs,block,cols", [(None, 128, 256), (FAKE, 96, 384), (FAKE, 4, 16),
                                              (FAKE, 8192, 8192), (FAKE, 256, 384)])
def test_project_hadamard_rejects_blocks(L, signs, block, cols):
    assert L.e8q_project_hadamard(FAKE, 1, 1, 4, cols, FAKE, signs, block, FAKE, 1, None, None,
                                  -1, None, FAKE, None) == 1


def test_project_rejects_huge(L):
    # 2^32 groups or more is unsupported (32-bit group indices on the device)
    assert L.e8q_project(FAKE, 1, 1 << 16, 1 << 16, 8, FAKE, FAKE, 1, None, -1, None, FAKE, None) == 2


def test_encode_rejects(L):
    ws = L.e8q_encode_workspace_size(1, 4, 16)
    base = [FAKE, 1, 1, 4, 16, FAKE, None, 0, 16, FAKE, FAKE, 10, FAKE, None, FAKE, ws, FAKE, None]
    bad = []
    b = list(base); b[8] = 41; bad.append(b)                      # core bound
    b = list(base); b[8] = -1; bad.append(b)
    b = list(base); b[9] = None; bad.append(b)                    # core index output
    b = list(base); b[12] = None; bad.append(b)                   # counts
    b = list(base); b[14] = None; bad.append(b)                   # workspace
    b = list(base); b[15] = ws - 1; bad.append(b)                 # too small
    b = list(base); b[14] = ctypes.c_void_p(0x10010); bad.append(b)   # misaligned
    b = list(base); b[10] = None; bad.append(b)                   # capacity without records
    b = list(base); b[6] = FAKE; b[7] = 24; bad.append(b)         # bad block
    for args in bad:
        assert L.e8q_encode_core_escape(*args) == 1, args


def test_ste_rejects(L):
    assert L.e8q_ste_backward(None, FAKE, None, 1.0, 1, 10, None) == 1
    assert L.e8q_ste_backward(FAKE, None, None, 1.0, 1, 10, None) == 1
    assert L.e8q_ste_backward(FAKE, FAKE, None, 1.0, 1, 0, None) == 1
    assert L.e8q_ste_backward(FAKE, FAKE, None, 1.0, 5, 10, None) == 1
    assert L.e8q_ste_backward(FAKE, FAKE, None, 1.0, 1, 10, None) == 1     # grad_w aliases grad_q


def test_restore_rejects(L):
    # (w, dt, batch, rows, cols, scale, signs, block, w_hat, w_hat_dt, two_z, bound, esc, status, stream)
    base = [FAKE, 1, 1, 4, 256, FAKE, FAKE, 128, FAKE, 1, None, -1, None, FAKE, None]
    bad = []
    b = list(base); b[8] = None; bad.append(b)                    # w_hat required
    b = list(base); b[9] = 3; bad.append(b)                       # w_hat dtype
    b = list(base); b[6] = None; bad.append(b)                    # signs required
    b = list(base); b[7] = 0; bad.append(b)                       # a block is required
    b = list(base); b[7] = 96; bad.append(b)
    b = list(base); b[4] = 200; bad.append(b)                     # block does not divide cols
    b = list(base); b[12] = FAKE; bad.append(b)                   # counts without a bound
    for args in bad:
        assert L.e8q_project_hadamard_restore(*args) == 1, args


def test_ste_hadamard_rejects(L):
    # (grad_q, dt, rows, cols, signs, block, grad_w, w_latent, lr, stream)
    base = [FAKE, 1, 4, 256, FAKE, 128, FAKE, None, 1.0, None]
    bad = []
    b = list(base); b[0] = None; bad.append(b)
    b = list(base); b[6] = None; bad.append(b)                    # no output
    b = list(base); b[1] = 4; bad.append(b)                       # dtype
    b = list(base); b[2] = 0; bad.append(b)
    b = list(base); b[4] = None; bad.append(b)                    # signs
    b = list(base); b[5] = 24; bad.append(b)                      # block
    b = list(base); b[7] = FAKE; bad.append(b)                    # latent aliases grad_w
    for args in bad:
        assert L.e8q_ste_backward_hadamard(*args) == 1, args
    # rows wider than the LDS sign table
    assert L.e8q_ste_backward_hadamard(FAKE, 1, 4, 65536, FAKE, 128, FAKE, None, 1.0, None) == 2


def _device_code_objects(path):
    """The gfx950 code objects inside the library's fat binaries (one per
    source file): ELF images found in the .hip_fatbin section."""
    objcopy = "/opt/rocm/llvm/bin/llvm-objcopy"
    if not os.path.exists(objcopy):
        pytest.skip("llvm-objcopy not available")
    import subprocess
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "fatbin")
        subprocess.run([objcopy, "--dump-section=.hip_fatbin=" + out, path, os.path.join(d, "stripped")],
                       check=True, capture_output=True)
        data = open(out, "rb").read()
    objs, i = [], data.find(b"\x7fELF")
    while i >= 0:
        objs.append(data[i:])
        i = data.find(b"\x7fELF", i + 4)
    return objs


def _symbols(elf):
    """(name, size, section index) of every symbol of a 64-bit ELF image."""
    import struct
    shoff, = struct.unpack_from("<Q", elf, 0x28)
    shentsize, shnum = struct.unpack_from("<HH", elf, 0x3A)
    secs = [struct.unpack_from("<IIQQQQIIQQ", elf, shoff + k * shentsize) for k in range(shnum)]
    out = []
    for (_, typ, _, _, off, size, link, _, _, entsize) in secs:
        if typ != 2:                                  # SHT_SYMTAB
            continue
        stroff = secs[link][4]
        for k in range(size // entsize):
            name_off, _, _, shndx, _, sz = struct.unpack_from("<IBBHQQ", elf, off + k * entsize)
            end = elf.index(b"\0", stroff + name_off)
            out.append((elf[stroff + name_off:end].decode(), sz, shndx))
    return out


@needs_device_code
def test_device_tables_in_code_object(L):
    """The read-only tables live in the device code object (no call uploads
    them): a defined device symbol of the generated blob's size."""
    import bit_e8_lattice_amd as e8q
    found = [(n, sz, ndx) for elf in _device_code_objects(e8q.library_path) for (n, sz, ndx) in _symbols(elf)
             if "g_table_blob" in n]
    assert found, "table blob missing from the device code objects"
    assert all(ndx != 0 for (_, _, ndx) in found)
    assert max(sz for (_, sz, _) in found) > 10_000_000


def test_noalloc_scratch_in_code_object_and_size_check(L):
    """The allocation-free encode's scratch is a device array of the stated
    size in the code object, and a shape past it is refused by the host check
    (before any pointer is touched or anything is enqueued)."""
    import bit_e8_lattice_amd as e8q
    if not HOST_ONLY_LIBRARY:
        found = [sz for elf in _device_code_objects(e8q.library_path) for (n, sz, ndx) in _symbols(elf)
                 if n.endswith("scratch") or "7scratch" in n]
        assert e8q.ENCODE_NOALLOC_SCRATCH_BYTES in found
    rows, cols = 1 << 20, 8192
    assert L.e8q_encode_workspace_size(1, rows, cols) > e8q.ENCODE_NOALLOC_SCRATCH_BYTES
    fake = 1 << 20
    code = L.e8q_encode_core_escape_noalloc(fake, 1, 1, rows, cols, fake, None, 0, 16, fake, None, 0, fake, None,
                                            fake, None)
    assert code == 5 and b"scratch" in L.e8q_status_string(code)


def test_sgd_project_rejects(L):
    """Missing latents or gradient, or a bad rotation block, are refused on the
    host before anything is launched."""
    fake = 1 << 20
    assert L.e8q_sgd_project_hadamard(None, fake, 1.0, 1, 8, 64, fake, None, 0, fake, 1, None, 16, None, fake,
                                      None) == 1
    assert L.e8q_sgd_project_hadamard(fake, None, 1.0, 1, 8, 64, fake, None, 0, fake, 1, None, 16, None, fake,
                                      None) == 1
    assert L.e8q_sgd_project_hadamard(fake, fake, 1.0, 1, 8, 64, fake, fake, 48, fake, 1, None, 16, None, fake,
                                      None) == 1
    assert L.e8q_sgd_project_hadamard(fake, fake, 1.0, 1, 8, 60, fake, None, 0, fake, 1, None, 16, None, fake,
                                      None) == 1
    # the rotated-gradient step needs the rotation: signs and a valid block
    f = L.e8q_sgd_rotated_project_hadamard
    assert f(None, fake, 1.0, 1, 8, 128, fake, fake, 128, fake, 1, None, 16, None, fake, None) == 1
    assert f(fake, None, 1.0, 1, 8, 128, fake, fake, 128, fake, 1, None, 16, None, fake, None) == 1
    assert f(fake, fake, 1.0, 1, 8, 128, fake, None, 128, fake, 1, None, 16, None, fake, None) == 1
    assert f(fake, fake, 1.0, 1, 8, 128, fake, fake, 0, fake, 1, None, 16, None, fake, None) == 1
    assert f(fake, fake, 1.0, 1, 8, 136, fake, fake, 128, fake, 1, None, 16, None, fake, None) == 1
