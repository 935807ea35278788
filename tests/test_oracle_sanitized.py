"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) runs the hand-worked cases, the exact rational brute
force, the finite-difference checks and the settings pins without a report:
no out-of-bounds access, use of freed memory, signed overflow or other
undefined behaviour on the paths the pins cover. The sanitized library is
loaded in a child Python process with the AddressSanitizer runtime
preloaded (it must come first in the process)."""

import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

SAN_FLAGS = ("-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g")

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle
import test_oracle_mutants as M
lib = {lib!r}
assert M._golden_ok(oracle, lib), "hand-worked cases"
assert M._exact_ok(oracle, lib), "exact rational brute force"
assert M._fd_ok(oracle, lib), "finite differences"
assert M._settings_ok(oracle, lib), "settings pins"
print("SANITIZED_ORACLE_OK", flush=True)
"""


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_under_address_and_undefined_sanitizers(oracle_mod, tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle_mod.build(out_path=str(tmp_path / "liboracle_san.so"), extra_flags=SAN_FLAGS)
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    code = CHILD.format(root=ROOT, tests=HERE, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and "SANITIZED_ORACLE_OK" in r.stdout, out[-4000:]
