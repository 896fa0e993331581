"""The oracle's pins again, on an AddressSanitizer + UndefinedBehaviorSanitizer build of the
oracle (gcc, host code only): every out-of-bounds access, use after free, signed overflow,
misaligned access or other undefined behaviour met by the pins aborts the run. A canary run
first shows that the sanitizer is live in this set-up (an out-of-bounds write planted in a
call of the oracle must be caught)."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_numerics.py", "tests/test_oracle_attention.py", "tests/test_oracle_extra.py"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def san_env(tmp_path_factory):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle.build(out=str(tmp_path_factory.mktemp("san") / "liboracle_san.so"), sanitize=True)
    return dict(os.environ, SA_ORACLE_LIB=lib, LD_PRELOAD=asan,
                ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def test_sanitizer_catches_a_planted_overflow(san_env):
    code = ("import numpy as np, oracle, ctypes as C\n"
            "x = np.zeros(16, np.uint16); y = np.zeros(15, np.float32)\n"
            "oracle.lib().orc_bf16_to_f32_array(x.ctypes.data_as(C.c_void_p), y.ctypes.data_as(C.c_void_p), 16)\n"
            "print('not caught')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=san_env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stdout + r.stderr[-2000:]


def test_oracle_pins_pass_under_sanitizers(san_env):
    pins = [p for p in PINS if os.path.exists(os.path.join(ROOT, p))]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *pins], cwd=ROOT, env=san_env, capture_output=True,
                       text=True, timeout=1800)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout
