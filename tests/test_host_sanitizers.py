"""The host layer of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: the library is rebuilt with its host
code sanitized (device code as usual) and ``test_abi_host.py`` runs against
it in a child process with the ASan runtime preloaded; any report is fatal."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_checks_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from bit_e8_lattice_amd import build as b
    try:
        runtime = b.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = b.build_host_sanitized(str(tmp_path))
    env = dict(os.environ)
    env.update({
        "E8Q_TEST_HOST_ONLY_LIBRARY": lib,
        "LD_PRELOAD": runtime,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "PYTHONDONTWRITEBYTECODE": "1",
    })
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q",
                          "-p", "no:cacheprovider"], cwd=str(tmp_path), env=env, capture_output=True, text=True,
                         timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-6000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert " passed" in out
