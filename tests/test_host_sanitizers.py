"""The library's host code under AddressSanitizer and ThreadSanitizer: a
host-instrumented build of libqlx (the device code is the ordinary one) runs
the CPU tests of the host logic -- the disk source's reader threads, their
bounce buffers and job queue, file layout and error paths, and the argument
validation of every entry point -- in a child python with the sanitizer
runtime preloaded. Any sanitizer report fails the test (halt_on_error)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_layer_file.py", "tests/test_abi.py"]


@pytest.mark.parametrize("san", ["address", "thread"])
def test_host_code_is_clean_under_sanitizer(san):
    from qlora_fine_tuning_dequant_amd.build import build, sanitizer_env
    lib = build(verbose=False, sanitize=san)
    env = sanitizer_env(san, lib)
    # the runtime is really there: its init symbol resolves in the child
    probe = f"import ctypes; ctypes.CDLL(None).__{'asan' if san == 'address' else 'tsan'}_init"
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", *HOST_TESTS,
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "Sanitizer" not in out, out[-4000:]
    assert " passed" in out and " skipped" not in out, out[-2000:]
