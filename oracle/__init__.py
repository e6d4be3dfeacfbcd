"""CPU oracle for the exact attention forward.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
benchmark's CPU-baseline leg are the only users; the GPU library never
imports, links or runs anything here, and this package never touches the GPU
library.

* :func:`attention` -- the plain definition (3-pass safe softmax, fp64), in C
  (``ref.c``), threaded over query rows.  See the header of ``ref.c`` for the
  passages it follows.
* :mod:`oracle.recurrence` -- the pages' online-softmax / tiled recurrences,
  step by step, in numpy (for the worked-example pins and cross-checks).

Inputs are the exact host values the GPU receives: bf16 tensors are widened
to float32 (exact) before they reach the C code; the scale is the float32
value handed to the GPU, widened to double.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ref.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile ref.c into liboracle.so with gcc (plain C, -O2, pthreads)."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _open(path):
    lib = ctypes.CDLL(path)
    f = lib.oracle_attention
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 6 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = _open(LIB_PATH)
    return _lib


def host_threads() -> int:
    """Number of host cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _as_f32(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor on the host
        import torch
        x = x.detach()
        if x.dtype != torch.float32:
            x = x.to(torch.float32)  # bf16 -> fp32 is exact
        x = x.contiguous().numpy()
    x = np.ascontiguousarray(x)
    if x.dtype != np.float32:
        raise TypeError("oracle inputs must be float32 (or bf16 tensors)")
    return x


def attention(q, k, v, scale, causal=False, rows=None, threads=None, _lib_override=None):
    """Exact attention forward, fp64, for selected query rows.

    q: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d] (float32 arrays or bf16/fp32
    host tensors).  scale: a float (rounded to float32 first, as the GPU sees
    it).  causal: key j visible to query i iff j <= i + Nk - Nq (bottom-right
    alignment); a row that sees no key gives O = 0, lse = -inf.
    rows: int array [R, 3] of (b, h, i); None means every row, in (b, h, i)
    order.  Returns (o [R, d] float64, lse [R] float64).
    ``_lib_override`` lets the mutation tests run a deliberately broken copy.
    """
    lib = _lib_override if _lib_override is not None else _load()
    q, k, v = _as_f32(q), _as_f32(k), _as_f32(v)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, Nk, Hkv, d) or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k and v")
    if rows is None:
        bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(Nq), indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    R = rows.shape[0]
    o = np.empty((R, d), dtype=np.float64)
    lse = np.empty(R, dtype=np.float64)
    sc = float(np.float32(scale))
    nt = threads or host_threads()
    rc = lib.oracle_attention(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                              B, Hq, Hkv, Nq, Nk, d, sc, int(bool(causal)),
                              rows.ctypes.data, R, o.ctypes.data, lse.ctypes.data, nt)
    if rc != 0:
        raise RuntimeError(f"oracle_attention failed with code {rc}")
    return o, lse
