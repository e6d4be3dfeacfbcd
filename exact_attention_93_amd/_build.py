"""Compile the HIP sources into the in-tree shared libraries (gfx950):

libfa.so               the library;
libfa_single_stage.so  the same library with its forward and backward kernels
                       built with one LDS stage per streamed tile
                       (FA_SINGLE_STAGE=1), a debug build whose outputs must
                       equal libfa.so's bit for bit.

Every source is compiled to an object in a temporary directory (in
parallel), and each library is linked from those objects."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libfa.so")
SINGLE_STAGE_LIB_PATH = os.path.join(PKG, "libfa_single_stage.so")
SINGLE_STAGE_SOURCES = ("fa_fwd_bf16.hip", "fa_fwd_fp8.hip", "fa_fwd_f32.hip", "fa_bwd_bf16.hip")   # read FA_SINGLE_STAGE
ARCH = "gfx950"

# Packed fp32 VALU instructions are switched off for all device code.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Each library resolves its own symbols to itself, so that both can be
# loaded into one process and neither calls into the other.
LINK_FLAGS = ["-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,-Bsymbolic"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.stderr and verbose:
        print(r.stderr, end="", flush=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stderr[-4000:]}")


def _link(hipcc, objs, out, verbose):
    tmp = out + ".tmp"
    _run([hipcc, *LINK_FLAGS, *objs, "-o", tmp], verbose)
    # A kernel whose host-side stub went missing would only fail at load time.
    und = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True, check=True).stdout
    bad = [ln.split()[-1] for ln in und.splitlines() if "device_stub" in ln or "_ZN2fa" in ln]
    if bad:
        os.remove(tmp)
        raise RuntimeError(f"{os.path.basename(out)} has undefined library symbols: {bad}")
    os.replace(tmp, out)


def build(verbose: bool = False, extra_flags=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    tmpdir = tempfile.mkdtemp(prefix="fa_build_")
    try:
        jobs = []   # (command, object, library it goes into: "main", "single" or "both")
        for src in sources():
            base = os.path.basename(src)
            obj = os.path.join(tmpdir, base + ".o")
            cmd = [hipcc, *HIPCC_FLAGS, *extra_flags, *inc, "-c", src, "-o", obj]
            if base in SINGLE_STAGE_SOURCES:
                jobs.append((cmd, obj, "main"))
                obj1 = os.path.join(tmpdir, base + ".single_stage.o")
                jobs.append(([hipcc, *HIPCC_FLAGS, *extra_flags, "-DFA_SINGLE_STAGE=1", *inc, "-c", src,
                              "-o", obj1], obj1, "single"))
            else:
                jobs.append((cmd, obj, "both"))
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(_run, cmd, verbose) for cmd, _, _ in jobs]:
                f.result()
        _link(hipcc, [o for _, o, lib in jobs if lib != "single"], LIB_PATH, verbose)
        _link(hipcc, [o for _, o, lib in jobs if lib != "main"], SINGLE_STAGE_LIB_PATH, verbose)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
