"""Exact, IO-aware attention forward for MI355X (gfx950).

The computation runs entirely in the HIP kernels of the in-tree shared
library ``libfa.so`` (C ABI declared in ``include/fa.h``).  This module only
marshals arguments: it checks tensor shapes, allocates the outputs with
torch on the inputs' device and passes raw device pointers and the current
HIP stream through ctypes.  There is no CPU fallback: if ``libfa.so`` is
missing or the tensors are not on a GPU, the call raises.

    o, lse = fwd(q, k, v, causal=False, scale=None)

q: [B, N, Hq, d]; k, v: [B, N, Hkv, d]; bf16 (-> fa_fwd) or float32
(-> fa_fwd_f32), contiguous.  o has q's shape and dtype; lse is float32
[B, Hq, N], the natural log-sum-exp of each row's scaled, masked scores.
"""
from __future__ import annotations

import ctypes
import math
import os

from ._build import LIB_PATH

__all__ = ["fwd", "fa_fwd", "fa_fwd_f32", "fa_strerror", "fa_version", "load_library", "FAError",
           "STATUS", "EXPORTS"]

STATUS = {
    "FA_OK": 0, "FA_ERR_NULL": 1, "FA_ERR_SHAPE": 2, "FA_ERR_HEADS": 3, "FA_ERR_HEADDIM": 4,
    "FA_ERR_ALIGN": 5, "FA_ERR_SCALE": 6, "FA_ERR_ALIAS": 7, "FA_ERR_LAUNCH": 8,
}
EXPORTS = ("fa_fwd", "fa_fwd_f32", "fa_strerror", "fa_version")

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"fa status {status}: {msg}")
        self.status = status


def load_library(path: str = LIB_PATH):
    """Open libfa.so and declare the C signatures (raises if it is not built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with __graft_entry__.build() "
            "(or python -m exact_attention_93_amd._build)")
    lib = ctypes.CDLL(path)
    args = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    for name in ("fa_fwd", "fa_fwd_f32"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = args
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_strerror.argtypes = [ctypes.c_int]
    lib.fa_version.restype = ctypes.c_int
    lib.fa_version.argtypes = []
    if path == LIB_PATH:
        _lib = lib
    return lib


def fa_strerror(status: int) -> str:
    return load_library().fa_strerror(int(status)).decode()


def fa_version() -> int:
    return load_library().fa_version()


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, stream) -> int:
    """Direct call of the C entry point with integer device addresses."""
    return load_library().fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, float(scale), int(causal), stream)


def fa_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, stream) -> int:
    return load_library().fa_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, N, d, float(scale), int(causal), stream)


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None, stream=None):
    """Attention forward through libfa.so.  Returns (o, lse)."""
    import torch

    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("fwd: q, k and v must be GPU tensors (there is no CPU path)")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("fwd: expected 4-D tensors [B, N, H, d]")
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, N, Hkv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"fwd: shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("fwd: q, k, v must all be bfloat16 or all float32")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("fwd: q, k, v must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    entry = fa_fwd if q.dtype == torch.bfloat16 else fa_fwd_f32
    st = entry(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
               B, Hq, Hkv, N, d, scale, causal, stream.cuda_stream)
    if st != 0:
        raise FAError(st, fa_strerror(st))
    return out, lse
