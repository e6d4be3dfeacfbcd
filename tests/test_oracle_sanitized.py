"""The C oracle (oracle/ref.c) built with AddressSanitizer and
UndefinedBehaviorSanitizer, run through the same pins as the normal build
(tests/pins.py: forward, block mask and backward), so that an out-of-bounds
access or undefined behaviour in any of its paths fails the CPU tier.  The
pins run in a child process with the sanitizer runtime preloaded (the Python
interpreter itself is not instrumented)."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(os.path.dirname(oracle.__file__), "ref.c")

CHILD = r"""
import functools, sys
sys.path.insert(0, {root!r})
import oracle
from tests import pins
lib = oracle._open({so!r})
att = functools.partial(oracle.attention, _lib_override=lib)
bwd = functools.partial(oracle.attention_bwd, _lib_override=lib)
for pin in pins.ALL_PINS:
    pin(att)
    print("pin", pin.__name__, "ok", flush=True)
for pin in pins.BWD_PINS:
    pin(att, bwd)
    print("pin", pin.__name__, "ok", flush=True)
# several thread counts over the same rows: the row threading under the sanitizers
q, k, v = pins.rand((2, 97, 4, 16), 1), pins.rand((2, 97, 2, 16), 2), pins.rand((2, 97, 2, 16), 3)
ref = att(q, k, v, 0.3, True, threads=1)
for t in (2, 5, 13):
    o, l = att(q, k, v, 0.3, True, threads=t)
    assert (o == ref[0]).all() and (l == ref[1]).all()
print("SANITIZED-OK", flush=True)
"""


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(600)
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    so = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", so, SRC, "-lm", "-lpthread"],
                   check=True)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, so=so)], capture_output=True, text=True,
                       env=env, timeout=580)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and "SANITIZED-OK" in r.stdout, out[-4000:]


@pytest.mark.timeout(600)
def test_a_planted_overflow_is_caught(tmp_path):
    """The same harness on a copy of ref.c whose score buffer is one element
    short must stop with an AddressSanitizer report."""
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = open(SRC).read()
    old = "double *s = (double *)malloc(sizeof(double) * (size_t)J->Nk);"
    assert src.count(old) == 1
    bad = tmp_path / "ref_short.c"
    bad.write_text(src.replace(old, "double *s = (double *)malloc(sizeof(double) * (size_t)(J->Nk - 1));"))
    so = str(tmp_path / "liboracle_short.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", so, str(bad), "-lm",
                    "-lpthread"], check=True)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, so=so)], capture_output=True, text=True,
                       env=env, timeout=580)
    assert r.returncode != 0 and "AddressSanitizer: heap-buffer-overflow" in r.stderr
