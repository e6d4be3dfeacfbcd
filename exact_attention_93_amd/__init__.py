"""Exact, IO-aware attention forward for MI355X (gfx950).

The computation runs entirely in the HIP kernels of the in-tree shared
library ``libfa.so`` (C ABI declared in ``include/fa.h``).  This module only
marshals arguments: it checks tensor shapes, allocates the outputs with
torch on the inputs' device and passes raw device pointers and the current
HIP stream through ctypes.  There is no CPU fallback: if ``libfa.so`` is
missing or the tensors are not on a GPU, the call raises.

    o, lse = fwd(q, k, v, causal=False, scale=None, num_splits=1)

q: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d]; bf16 or float32, contiguous.  o
has q's shape and dtype; lse is float32 [B, Hq, Nq], the natural
log-sum-exp of each row's scaled, masked scores.  Equal lengths and one key
range go to fa_fwd / fa_fwd_f32; unequal lengths (bottom-right causal
alignment) or a split key sequence go to fa_fwd_splitkv(_f32), with the
workspace allocated here by torch.

    dq, dk, dv = bwd(q, k, v, o, lse, dout, causal=False, scale=None)

Gradients through fa_bwd (bf16): o and lse are the forward's outputs for
the same q, k, v, causal and scale; dout has o's shape.
"""
from __future__ import annotations

import ctypes
import math
import os

from ._build import LIB_PATH, SINGLE_STAGE_LIB_PATH

__all__ = ["fwd", "fa_fwd_splitkv_static", "fwd_blocksparse", "fa_fwd_blocksparse", "fwd_fp8", "fa_fwd_fp8", "fwd_fp8_block",
           "fa_fwd_fp8_block", "quantize_fp8", "fa_quantize_fp8", "bwd", "fa_bwd", "fa_bwd_workspace_size", "fa_fwd", "fa_fwd_f32", "fa_fwd_splitkv", "fa_fwd_splitkv_f32", "fa_splitkv_num_splits",
           "fa_splitkv_workspace_size", "fa_strerror", "fa_version", "fa_lds_stages", "load_library", "FAError",
           "STATUS", "EXPORTS"]

STATUS = {
    "FA_OK": 0, "FA_ERR_NULL": 1, "FA_ERR_SHAPE": 2, "FA_ERR_HEADS": 3, "FA_ERR_HEADDIM": 4,
    "FA_ERR_ALIGN": 5, "FA_ERR_SCALE": 6, "FA_ERR_ALIAS": 7, "FA_ERR_LAUNCH": 8,
    "FA_ERR_SPLITS": 9, "FA_ERR_WORKSPACE": 10, "FA_ERR_SCRATCH": 11,
}
STATIC_SCRATCH_BYTES = 32 << 20   # FA_STATIC_SCRATCH_BYTES
EXPORTS = ("fa_fwd", "fa_fwd_f32", "fa_fwd_splitkv", "fa_fwd_splitkv_f32", "fa_fwd_splitkv_static",
           "fa_splitkv_num_splits",
           "fa_splitkv_workspace_size", "fa_fwd_blocksparse", "fa_fwd_fp8", "fa_fwd_fp8_block", "fa_quantize_fp8",
           "fa_bwd", "fa_bwd_workspace_size", "fa_strerror", "fa_version", "fa_lds_stages")

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
    sargs = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [ctypes.c_float, ctypes.c_int, ctypes.c_int,
             ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p])
    for name in ("fa_fwd_splitkv", "fa_fwd_splitkv_f32"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = sargs
    lib.fa_fwd_splitkv_static.restype = ctypes.c_int
    lib.fa_fwd_splitkv_static.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 +
                                          [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p])
    lib.fa_splitkv_num_splits.restype = ctypes.c_int
    lib.fa_splitkv_num_splits.argtypes = [ctypes.c_int] * 7
    lib.fa_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.fa_splitkv_workspace_size.argtypes = [ctypes.c_int] * 7
    lib.fa_fwd_blocksparse.restype = ctypes.c_int
    lib.fa_fwd_blocksparse.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p])
    lib.fa_fwd_fp8.restype = ctypes.c_int
    lib.fa_fwd_fp8.argtypes = ([ctypes.c_void_p] * 8 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int,
                               ctypes.c_void_p])
    lib.fa_fwd_fp8_block.restype = ctypes.c_int
    lib.fa_fwd_fp8_block.argtypes = ([ctypes.c_void_p] * 8 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int,
                                     ctypes.c_void_p])
    lib.fa_quantize_fp8.restype = ctypes.c_int
    lib.fa_quantize_fp8.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 4 + [ctypes.c_void_p] * 2
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd.argtypes = ([ctypes.c_void_p] * 9 + [ctypes.c_int] * 6 + [ctypes.c_float, ctypes.c_int,
                           ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p])
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd_workspace_size.argtypes = [ctypes.c_int] * 3
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_strerror.argtypes = [ctypes.c_int]
    lib.fa_version.restype = ctypes.c_int
    lib.fa_version.argtypes = []
    lib.fa_lds_stages.restype = ctypes.c_int
    lib.fa_lds_stages.argtypes = []
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check_buffer(name, t, shape, dtype, device):
    """A caller-supplied output: on q's GPU, contiguous, of the shape and
    dtype the kernels write (they write every element of it, so a smaller
    or strided buffer would be written out of bounds)."""
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a tensor on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(name, t, need, device):
    """A caller-supplied workspace: contiguous bytes on q's GPU, at least `need` of them."""
    if not t.is_cuda or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {device}")
    if t.numel() * t.element_size() < need:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, {need} needed")


def fa_strerror(status: int) -> str:
    return load_library().fa_strerror(int(status)).decode()


def fa_version() -> int:
    return load_library().fa_version()


def fa_lds_stages() -> int:
    return load_library().fa_lds_stages()


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, stream) -> int:
    """Direct call of the C entry point with integer device addresses."""
    return load_library().fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, float(scale), int(causal), stream)


def fa_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, stream) -> int:
    return load_library().fa_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, N, d, float(scale), int(causal), stream)


def fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, num_splits, ws, ws_bytes,
                   stream) -> int:
    return load_library().fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, float(scale), int(causal),
                                         int(num_splits), ws, ws_bytes, stream)


def fa_fwd_splitkv_f32(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, num_splits, ws, ws_bytes,
                       stream) -> int:
    return load_library().fa_fwd_splitkv_f32(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, float(scale), int(causal),
                                             int(num_splits), ws, ws_bytes, stream)


def fa_fwd_splitkv_static(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, num_splits, stream) -> int:
    """fa_fwd_splitkv with the library's static scratch array (allocates nothing)."""
    return load_library().fa_fwd_splitkv_static(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, float(scale), int(causal),
                                                int(num_splits), stream)


def fa_splitkv_num_splits(B, Hq, Hkv, Nq, Nk, d, num_splits) -> int:
    return load_library().fa_splitkv_num_splits(B, Hq, Hkv, Nq, Nk, d, num_splits)


def fa_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits) -> int:
    return load_library().fa_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits)


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None, stream=None,
        num_splits: int = 1, workspace=None):
    """Attention forward through libfa.so.  Returns (o, lse).

    num_splits: 1 = the whole key sequence per workgroup; n > 1 = at most n
    key ranges merged afterwards; 0 = the library's choice.  workspace: an
    optional preallocated uint8 GPU tensor for the split forward.
    """
    import torch

    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("fwd: q, k and v must be GPU tensors (there is no CPU path)")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("fwd: expected 4-D tensors [B, N, H, d]")
    B, N, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Nk, Hkv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"fwd: shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("fwd: q, k, v must all be bfloat16 or all float32")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("fwd: q, k, v must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_buffer("fwd: out", out, q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check_buffer("fwd: lse", lse, (B, Hq, N), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    bf16 = q.dtype == torch.bfloat16
    if Nk == N and num_splits == 1:
        entry = fa_fwd if bf16 else fa_fwd_f32
        st = entry(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                   B, Hq, Hkv, N, d, scale, causal, stream.cuda_stream)
    else:
        need = fa_splitkv_workspace_size(B, Hq, Hkv, N, Nk, d, num_splits)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if workspace is not None:
            _check_workspace("fwd: workspace", workspace, need, q.device)
        ws_ptr = workspace.data_ptr() if workspace is not None else 0
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        entry = fa_fwd_splitkv if bf16 else fa_fwd_splitkv_f32
        st = entry(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                   B, Hq, Hkv, N, Nk, d, scale, causal, num_splits, ws_ptr, ws_bytes, stream.cuda_stream)
    if st != 0:
        raise FAError(st, fa_strerror(st))
    return out, lse


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale, causal, ws, ws_bytes, stream) -> int:
    return load_library().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, float(scale),
                                 int(causal), ws, ws_bytes, stream)


def fa_bwd_workspace_size(B, Hq, Nq) -> int:
    return load_library().fa_bwd_workspace_size(B, Hq, Nq)


def bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None, dq=None, dk=None, dv=None,
        workspace=None, stream=None):
    """Attention backward through libfa.so (bf16).  Returns (dq, dk, dv)."""
    import torch

    ts = (q, k, v, o, dout)
    if not all(t.is_cuda for t in ts) or not lse.is_cuda:
        raise ValueError("bwd: every tensor must be on the GPU (there is no CPU path)")
    if any(t.dtype != torch.bfloat16 for t in ts) or lse.dtype != torch.float32:
        raise ValueError("bwd: q, k, v, o, dout must be bfloat16 and lse float32")
    if not all(t.is_contiguous() for t in ts) or not lse.is_contiguous():
        raise ValueError("bwd: tensors must be contiguous")
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if (tuple(k.shape) != (B, Nk, Hkv, d) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape
            or tuple(lse.shape) != (B, Hq, Nq)):
        raise ValueError("bwd: shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_buffer("bwd: dq", dq, q.shape, torch.bfloat16, q.device)
    _check_buffer("bwd: dk", dk, k.shape, torch.bfloat16, q.device)
    _check_buffer("bwd: dv", dv, v.shape, torch.bfloat16, q.device)
    need = fa_bwd_workspace_size(B, Hq, Nq)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check_workspace("bwd: workspace", workspace, need, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq, Nk, d, scale, causal,
                workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if st != 0:
        raise FAError(st, fa_strerror(st))
    return dq, dk, dv


def fa_fwd_fp8(q, k, v, qd, kd, vd, o, lse, B, Hq, Hkv, N, d, scale, causal, stream) -> int:
    return load_library().fa_fwd_fp8(q, k, v, qd, kd, vd, o, lse, B, Hq, Hkv, N, d, float(scale), int(causal),
                                     stream)


def fwd_fp8(q, k, v, q_descale, k_descale, v_descale, causal: bool = False, scale: float | None = None,
            out=None, lse=None, stream=None):
    """fp8 (e4m3) attention forward through libfa.so.  Returns (o bf16, lse).

    q: [B, N, Hq, d], k, v: [B, N, Hkv, d] as torch.float8_e4m3fn (or uint8
    codes); q_descale [B, Hq], k_descale and v_descale [B, Hkv] float32: the
    real inputs are code * descale."""
    import torch

    ts = (q, k, v, q_descale, k_descale, v_descale)
    if not all(t.is_cuda for t in ts):
        raise ValueError("fwd_fp8: every tensor must be on the GPU (there is no CPU path)")
    if any(t.element_size() != 1 for t in (q, k, v)):
        raise ValueError("fwd_fp8: q, k, v must hold one-byte e4m3 codes")
    if any(t.dtype != torch.float32 for t in ts[3:]):
        raise ValueError("fwd_fp8: descale factors must be float32")
    if not all(t.is_contiguous() for t in ts):
        raise ValueError("fwd_fp8: tensors must be contiguous")
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    if (tuple(k.shape) != (B, N, Hkv, d) or v.shape != k.shape or tuple(q_descale.shape) != (B, Hq)
            or tuple(k_descale.shape) != (B, Hkv) or tuple(v_descale.shape) != (B, Hkv)):
        raise ValueError("fwd_fp8: shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, N, Hq, d), dtype=torch.bfloat16, device=q.device)
    _check_buffer("fwd_fp8: out", out, (B, N, Hq, d), torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check_buffer("fwd_fp8: lse", lse, (B, Hq, N), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), q_descale.data_ptr(), k_descale.data_ptr(),
                    v_descale.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d, scale, causal,
                    stream.cuda_stream)
    if st != 0:
        raise FAError(st, fa_strerror(st))
    return out, lse


QUANT_BLOCK = 64         # rows per block of the block-scaled fp8 format


def fa_quantize_fp8(x, codes, exps, B, N, H, d, signs, stream) -> int:
    return load_library().fa_quantize_fp8(x, codes, exps, B, N, H, d, signs, stream)


def quantize_fp8(x, signs=None, codes=None, exps=None, stream=None):
    """Block-scaled e4m3 quantisation through libfa.so.  Returns (codes, exps).

    x: bf16 GPU tensor [B, N, H, 128].  signs: None, or an int8 GPU tensor of
    128 values +-1, which rotates every row first, y = (x * signs) H (H the
    Sylvester-Hadamard matrix; rotating both q and k multiplies the scores by
    128, see fwd_fp8_block).  codes: uint8 [B, N, H, 128] (e4m3 codes);
    exps: int8 [B, H, ceil(N / 64)]; the real block values are code * 2^exp."""
    import torch

    if not x.is_cuda or x.dtype != torch.bfloat16 or x.dim() != 4 or not x.is_contiguous():
        raise ValueError("quantize_fp8: x must be a contiguous bfloat16 GPU tensor [B, N, H, d]")
    B, N, H, d = x.shape
    nb = -(-N // QUANT_BLOCK)
    if signs is not None:
        if not signs.is_cuda or signs.dtype != torch.int8 or tuple(signs.shape) != (d,) or not signs.is_contiguous():
            raise ValueError(f"quantize_fp8: signs must be a contiguous int8 GPU tensor of {d} values")
    codes = torch.empty((B, N, H, d), dtype=torch.uint8, device=x.device) if codes is None else codes
    exps = torch.empty((B, H, nb), dtype=torch.int8, device=x.device) if exps is None else exps
    _check_buffer("quantize_fp8: codes", codes, (B, N, H, d), torch.uint8, x.device)
    _check_buffer("quantize_fp8: exps", exps, (B, H, nb), torch.int8, x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    st = fa_quantize_fp8(x.data_ptr(), codes.data_ptr(), exps.data_ptr(), B, N, H, d,
                         signs.data_ptr() if signs is not None else 0, stream.cuda_stream)
    if st != 0:
        raise FAError(st, fa_strerror(st))
    return codes, exps


def fa_fwd_fp8_block(q, k, v, qe, ke, ve, o, lse, B, Hq, Hkv, N, d, scale, causal, stream) -> int:
    return load_library().fa_fwd_fp8_block(q, k, v, qe, ke, ve, o, lse, B, Hq, Hkv, N, d, float(scale),
                                           int(causal), stream)


def fwd_fp8_block(q, k, v, q_exp, k_exp, v_exp, causal: bool = False, scale: float | None = None, out=None,
                  lse=None, stream=None):
    """fp8 attention forward with per-block scales through libfa.so.
    Returns (o bf16, lse).

    q: [B, N, Hq, 128], k, v: [B, N, Hkv, 128] e4m3 codes (uint8 or
    torch.float8_e4m3fn); q_exp [B, Hq, ceil(N/64)], k_exp and v_exp
    [B, Hkv, ceil(N/64)] int8: the real inputs are code * 2^exp of their
    64-row block (quantize_fp8's output).  When q and k were both rotated by
    quantize_fp8 with the same signs, pass scale / 128 (the rotation
    multiplies every score by 128)."""
    import torch

    ts = (q, k, v, q_exp, k_exp, v_exp)
    if not all(t.is_cuda for t in ts):
        raise ValueError("fwd_fp8_block: every tensor must be on the GPU (there is no CPU path)")
    if any(t.element_size() != 1 for t in ts):
        raise ValueError("fwd_fp8_block: codes and exponents are one byte each")
    if not all(t.is_contiguous() for t in ts):
        raise ValueError("fwd_fp8_block: tensors must be contiguous")
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    nb = -(-N // QUANT_BLOCK)
    if (tuple(k.shape) != (B, N, Hkv, d) or v.shape != k.shape or tuple(q_exp.shape) != (B, Hq, nb)
            or tuple(k_exp.shape) != (B, Hkv, nb) or tuple(v_exp.shape) != (B, Hkv, nb)):
        raise ValueError("fwd_fp8_block: shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, N, Hq, d), dtype=torch.bfloat16, device=q.device)
    _check_buffer("fwd_fp8_block: out", out, (B, N, Hq, d), torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check_buffer("fwd_fp8_block: lse", lse, (B, Hq, N), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_fwd_fp8_block(q.data_ptr(), k.data_ptr(), v.data_ptr(), q_exp.data_ptr(), k_exp.data_ptr(),
                          v_exp.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d, scale, causal,
                          stream.cuda_stream)
    if st != 0:
        raise FAError(st, fa_strerror(st))
    return out, lse


MASK_BLOCK = (128, 64)   # query rows x keys per block-mask entry


def fa_fwd_blocksparse(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, mask, stream) -> int:
    return load_library().fa_fwd_blocksparse(q, k, v, o, lse, B, Hq, Hkv, N, d, float(scale), int(causal),
                                             mask, stream)


def fwd_blocksparse(q, k, v, block_mask, causal: bool = False, scale: float | None = None, out=None, lse=None,
                    stream=None):
    """Block-sparse bf16 forward.  block_mask: uint8 GPU tensor
    [Hq, ceil(N/128), ceil(N/64)], nonzero = the block is computed."""
    import torch

    if not all(t.is_cuda for t in (q, k, v, block_mask)):
        raise ValueError("fwd_blocksparse: every tensor must be on the GPU (there is no CPU path)")
    if any(t.dtype != torch.bfloat16 for t in (q, k, v)) or block_mask.dtype != torch.uint8:
        raise ValueError("fwd_blocksparse: q, k, v bfloat16 and block_mask uint8")
    if not all(t.is_contiguous() for t in (q, k, v, block_mask)):
        raise ValueError("fwd_blocksparse: tensors must be contiguous")
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    want = (Hq, -(-N // MASK_BLOCK[0]), -(-N // MASK_BLOCK[1]))
    if tuple(k.shape) != (B, N, Hkv, d) or v.shape != k.shape or tuple(block_mask.shape) != want:
        raise ValueError(f"fwd_blocksparse: shape mismatch (mask must be {want})")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    _check_buffer("fwd_blocksparse: out", out, q.shape, torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check_buffer("fwd_blocksparse: lse", lse, (B, Hq, N), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            B, Hq, Hkv, N, d, scale, causal, block_mask.data_ptr(), stream.cuda_stream)
    if st != 0:
        raise FAError(st, fa_strerror(st))
    return out, lse
