"""The fp8 forward against the fp64 oracle on the dequantised inputs.

Bound per output element (o_ix for query row i, coordinate x), from the
arithmetic: the scores are exact products of the e4m3 codes summed in fp32;
the kernel forms P'_j = 2^(s_j c - m + 7) against a running maximum m that
ends within one base-2 unit of the row's maximum, so the largest P' lies in
[2^7, 2^8] and S = sum_j P'_j >= 2^7; each P'_j is rounded to e4m3, with
error e_j <= max(2^-4 P'_j, 2^-10) (relative 2^-4 for normal values, half
the subnormal step 2^-9 below 2^-6); and O is normalised by the sum S~ of
the rounded values.  Exactly, o_i - O_i = sum_j (P~'_j - P'_j)(v_j - O_i) / S~,
so with w_j = P'_j / S and S~ >= S (1 - 2^-4) - n 2^-10:
    |o_ix - O_ix| <= sum_j max(2^-4 w_j, 2^-17) (|v_jx| + |O_ix|) / (1 - 2^-4 - n 2^-17)
over the n visible keys; the bf16 output adds half an ulp (<= 2^-8 |O_ix|),
and 1e-5 covers fp32 accumulation.  The log-sum-exp uses the unrounded fp32
sum: |dlse| <= 1e-4 max(1, |lse|) as for bf16, plus the fp32 rounding of the
scores themselves, which the log-sum-exp passes on at most unchanged (it is
1-Lipschitz in the max norm): a sum of d products accumulated in fp32 in any
order is within gamma_d = d 2^-24 / (1 - d 2^-24) of sum_x |q_x k_x|, so
|dlse| gains scale * gamma_d * max_j sum_x |q_ix k_jx| over visible keys (a
term that matters only when the block scales make the products large).
"""
from __future__ import annotations

import numpy as np
import torch

import exact_attention_93_amd as fa
import oracle
from exact_attention_93_amd import workloads as W
from tests.gpu_util import say


def gpu_fp8(q8, k8, v8, qd, kd, vd, causal, scale):
    o, lse = fa.fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), qd.cuda(), kd.cuda(), vd.cuda(), causal=causal,
                        scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def compare_fp8(q8, k8, v8, qd, kd, vd, causal, scale, o, lse, rows=None, label=""):
    q, k, v = W.dequantize_fp8(q8, qd), W.dequantize_fp8(k8, kd), W.dequantize_fp8(v8, vd)
    return compare_fp8_real(q, k, v, causal, scale, o, lse, rows=rows, label=label)


def compare_fp8_real(q, k, v, causal, scale, o, lse, rows=None, label=""):
    """The bound above, for real inputs q, k, v (float32 tensors holding the
    dequantised values exactly)."""
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    ro, rl = oracle.attention(q, k, v, scale, causal, rows=rows)
    if rows is None:
        bb, hh, ii = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(N), indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
    rows = np.asarray(rows)
    go = o.float().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]].astype(np.float64)
    gl = lse.numpy()[rows[:, 0], rows[:, 1], rows[:, 2]].astype(np.float64)
    # sum_j w_ij |v_jx| for each checked row, w_ij = exp(s_ij - lse_i) (fp64)
    pv = np.zeros_like(ro)
    wsum = np.zeros((ro.shape[0], 1))
    sabs = np.zeros(ro.shape[0])
    sc = float(np.float32(scale))
    for b in range(B):
        for h in range(Hq):
            sel = np.nonzero((rows[:, 0] == b) & (rows[:, 1] == h))[0]
            if len(sel) == 0:
                continue
            qi = torch.from_numpy(q[b, rows[sel, 2], h].double().numpy())
            kk = k[b, :, h // g].double()
            s = (qi @ kk.t()) * sc
            if causal:
                s = s.masked_fill(torch.arange(N)[None, :] > torch.from_numpy(rows[sel, 2])[:, None], float("-inf"))
            w = torch.exp(s - torch.from_numpy(rl[sel])[:, None])
            vis = torch.isfinite(s)
            wt = torch.where(vis, torch.clamp(2.0 ** -4 * w, min=2.0 ** -17), torch.zeros_like(w))
            n = vis.sum(dim=1, keepdim=True).double()
            denom = 1.0 - 2.0 ** -4 - n * 2.0 ** -17
            pv[sel] = ((wt @ v[b, :, h // g].double().abs()) / denom).numpy()
            wsum[sel] = (wt.sum(dim=1, keepdim=True) / denom).numpy()
            absdot = qi.abs() @ kk.abs().t()
            absdot = torch.where(vis, absdot, torch.zeros_like(absdot))
            sabs[sel] = absdot.max(dim=1).values.numpy()
    bound = pv + wsum * np.abs(ro) + 2.0 ** -8 * np.abs(ro) + 1e-5
    err = np.abs(go - ro)
    ratio = err / bound
    gamma = d * 2.0 ** -24 / (1 - d * 2.0 ** -24)
    lerr = (np.abs(gl - rl) - abs(sc) * gamma * sabs) / np.maximum(1.0, np.abs(rl))
    say(f"[fp8] {label} rows={len(rl)} max|dO|={err.max():.3e} mean|dO|={err.mean():.3e} "
        f"max err/bound={ratio.max():.3f} mean bound={bound.mean():.3e} max rel dLSE={lerr.max():.3e}")
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl)), "non-finite output"
    assert ratio.max() <= 1.0, f"an element exceeds the e4m3 bound by x{ratio.max():.3f}"
    assert lerr.max() <= 1e-4, f"LSE error {lerr.max()}"
    return float(err.max()), float(ratio.max())


def fp8_inputs(B, N, Hq, Hkv, d, seed, q_std=1.0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, N, Hq, d), generator=g) * q_std
    k = torch.randn((B, N, Hkv, d), generator=g)
    v = torch.randn((B, N, Hkv, d), generator=g)
    (q8, qd), (k8, kd), (v8, vd) = W.quantize_fp8(q), W.quantize_fp8(k), W.quantize_fp8(v)
    return q8, k8, v8, qd, kd, vd


def dequantize_blocks_f32(codes, exps):
    """Block-scaled codes (uint8) and exponents (int8) as the float32 real
    values code * 2^exp (exact), through the oracle's e4m3 decoder."""
    from oracle import fp8 as F
    return torch.from_numpy(F.dequantize_blocks(codes.numpy(), exps.numpy()).astype(np.float32))
