"""The C ABI's host code (argument validation, size arithmetic, the error
paths) built with AddressSanitizer and UndefinedBehaviorSanitizer, and the
CPU ABI tests (tests/test_abi.py) run against it.  Only the host side is
instrumented (each -fsanitize= sits behind -Xarch_host); no test here
reaches a launch.  The tests run in a child process with clang's sanitizer
runtime preloaded (the Python interpreter itself is not instrumented)."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_93_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
# the size limit of the dense forward's validation, and the same computed in
# 32-bit arithmetic (the planted mistake)
LIMIT = "if (((int64_t)Nq + 256) * Hq * d >= ((int64_t)1 << 29)) return FA_ERR_SHAPE;"
LIMIT_32 = "if ((Nq + 256) * Hq * d >= (1 << 29)) return FA_ERR_SHAPE;"

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import pytest
import exact_attention_93_amd as fa
fa._lib = fa.load_library({so!r})      # every call below goes to the sanitised build
rc = pytest.main(["-x", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu", {tests!r}])
print("SANITIZED-RC", int(rc), flush=True)
sys.exit(int(rc))
"""


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm*/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _compile_all(jobs):
    """Compile (source, object) pairs in parallel; raise with the first error."""
    procs = [(src, subprocess.Popen([HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src,
                                     "-o", obj], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
             for src, obj in jobs]
    for src, p in procs:
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, f"{src}: {err[-3000:]}"


def _link(objs, so):
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-shared-libsan", *objs, "-o", so],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return so


@pytest.fixture(scope="module")
def san(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    d = tmp_path_factory.mktemp("abi_san")
    src = open(os.path.join(CSRC, "fa_api.cpp")).read()
    assert LIMIT in src
    bad = d / "fa_api_bad.cpp"
    bad.write_text(src.replace(LIMIT, LIMIT_32, 1))
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = [(s, str(d / (os.path.basename(s) + ".o"))) for s in sources] + [(str(bad), str(d / "fa_api_bad.o"))]
    _compile_all(jobs)
    objs = {os.path.basename(s): o for s, o in jobs}
    good = [o for name, o in objs.items() if name != "fa_api_bad.cpp"]
    planted = [o for name, o in objs.items() if name not in ("fa_api.cpp",)]
    return asan, _link(good, str(d / "libfa_san.so")), _link(planted, str(d / "libfa_planted.so"))


def _run(so, asan, tests):
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, so=so, tests=tests)], capture_output=True,
                       text=True, env=env, timeout=560, cwd=ROOT)
    return r, r.stdout + r.stderr


@pytest.mark.timeout(1200)
def test_abi_validation_under_asan_and_ubsan(san):
    asan, good, _ = san
    r, out = _run(good, asan, os.path.join(ROOT, "tests", "test_abi.py"))
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and "SANITIZED-RC 0" in out, out[-4000:]


@pytest.mark.timeout(1200)
def test_a_planted_overflow_in_validation_is_caught(san):
    """The same harness on a copy of the API layer whose size limit is
    computed in 32-bit arithmetic: the N = 2^20, Hq = 32, d = 128 case of
    test_invalid_arguments overflows it, and UndefinedBehaviorSanitizer must
    stop the run."""
    asan, _, planted = san
    r, out = _run(planted, asan, os.path.join(ROOT, "tests", "test_abi.py") + "::test_invalid_arguments")
    assert "runtime error" in out and "signed integer overflow" in out, out[-4000:]
    assert r.returncode != 0
