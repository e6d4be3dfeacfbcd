"""CPU oracle for the exact attention forward and its gradients.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
benchmark's CPU-baseline leg are the only users; the GPU library never
imports, links or runs anything here, and this package never touches the GPU
library.

* :func:`attention` -- the plain definition (3-pass safe softmax, fp64), in C
  (``ref.c``), threaded over query rows.  See the header of ``ref.c`` for the
  passages it follows.
* :func:`attention_bwd` -- dq, dk, dv: the derivative of that definition for
  an upstream gradient dO, fp64, in C (``ref.c``), per key/value head group.
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
    f = lib.oracle_attention_masked
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 6 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    f = lib.oracle_attention_bwd
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 6 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
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


def attention(q, k, v, scale, causal=False, rows=None, threads=None, _lib_override=None,
              block_mask=None, block=(128, 64)):
    """Exact attention forward, fp64, for selected query rows.

    q: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d] (float32 arrays or bf16/fp32
    host tensors).  scale: a float (rounded to float32 first, as the GPU sees
    it).  causal: key j visible to query i iff j <= i + Nk - Nq (bottom-right
    alignment); a row that sees no key gives O = 0, lse = -inf.
    rows: int array [R, 3] of (b, h, i); None means every row, in (b, h, i)
    order.  block_mask: None, or a uint8 array [Hq, ceil(Nq/bq), ceil(Nk/bk)]
    with block = (bq, bk): key j is kept for query i of head h only where the
    mask entry of their blocks is nonzero.  Returns (o [R, d] float64,
    lse [R] float64).
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
    if block_mask is None:
        rc = lib.oracle_attention(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                  B, Hq, Hkv, Nq, Nk, d, sc, int(bool(causal)),
                                  rows.ctypes.data, R, o.ctypes.data, lse.ctypes.data, nt)
    else:
        bq, bk = int(block[0]), int(block[1])
        m = block_mask.detach().cpu().numpy() if hasattr(block_mask, "detach") else block_mask
        m = np.ascontiguousarray(np.asarray(m, dtype=np.uint8))
        if m.shape != (Hq, -(-Nq // bq), -(-Nk // bk)):
            raise ValueError(f"block mask shape {m.shape} does not match the blocks")
        rc = lib.oracle_attention_masked(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                         B, Hq, Hkv, Nq, Nk, d, sc, int(bool(causal)), m.ctypes.data, bq, bk,
                                         rows.ctypes.data, R, o.ctypes.data, lse.ctypes.data, nt)
    if rc != 0:
        raise RuntimeError(f"oracle_attention failed with code {rc}")
    return o, lse


def attention_bwd(q, k, v, dout, scale, causal=False, groups=None, threads=None, _lib_override=None):
    """Gradients of the exact attention forward, fp64, per key/value head group.

    q, dout: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d]; scale and causal as in
    :func:`attention`.  groups: int array [G, 2] of (b, hk); None means every
    group in (b, hk) order.  Returns (dq [G, Hq/Hkv, Nq, d], dk [G, Nk, d],
    dv [G, Nk, d]) as float64: dq for the query heads hk*g .. hk*g+g-1 of each
    group, dk and dv of the shared head summed over them.
    """
    lib = _lib_override if _lib_override is not None else _load()
    q, k, v, dout = _as_f32(q), _as_f32(k), _as_f32(v), _as_f32(dout)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, Nk, Hkv, d) or v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v and dout")
    if groups is None:
        bb, hh = np.meshgrid(np.arange(B), np.arange(Hkv), indexing="ij")
        groups = np.stack([bb.ravel(), hh.ravel()], axis=1)
    groups = np.ascontiguousarray(np.asarray(groups, dtype=np.int32).reshape(-1, 2))
    G, g = groups.shape[0], Hq // Hkv
    dq = np.empty((G, g, Nq, d), dtype=np.float64)
    dk = np.empty((G, Nk, d), dtype=np.float64)
    dv = np.empty((G, Nk, d), dtype=np.float64)
    nt = threads or host_threads()
    rc = lib.oracle_attention_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                  B, Hq, Hkv, Nq, Nk, d, float(np.float32(scale)), int(bool(causal)),
                                  groups.ctypes.data, G, dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, nt)
    if rc != 0:
        raise RuntimeError(f"oracle_attention_bwd failed with code {rc}")
    return dq, dk, dv
