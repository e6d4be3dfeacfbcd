"""Helpers for the backward GPU tests: the HIP path, the fp64 oracle on the
same host values, and the per-element bound the gradients are held to.

The bound is an interval for every gradient element, derived from the
arithmetic the backward performs (the recomputing backward of
"FlashAttention：IO 感知的精确注意力", section 6, and "[Attention优化] 从
Online-Softmax到FlashAttention V1/V2/V3", sections 0x04 and 0x05, with P
and dS as 16-bit matrix operands), written out in fp64 here:

  p  = exp(scale s - lse)            s = q.k; lse as the forward returned it
  t  = dp - delta                    dp = dO.v; delta = dO.o, o as returned
  ds = p t
  dq = scale sum_j bf16(ds) k,  dk = scale sum_i bf16(ds) q,  dv = sum_i bf16(p) dO

with fp32 in place of every exact operation.  Each fp32 intermediate is
within a proven distance of its exact value (standard bounds, u = 2^-24:
gamma_n = n u / (1 - n u) for an n-term sum in any order, u per rounding,
two units in the last place for the hardware exp2), so its bf16 rounding
lies between the bf16 roundings of the two ends of that range (rounding is
monotone).  Summed against the other operand, plus gamma_n times the sum of
magnitudes for the fp32 accumulation, times the fp32 scale, and rounded to
bf16 at both ends, this gives an interval that must hold the GPU's output
element.  The tests run the backward on o and lse computed by the oracle
(rounded to bf16 and fp32, as the forward stores them) for the heads they
check, so no expected value depends on the HIP path."""
from __future__ import annotations

import numpy as np
import torch

import exact_attention_93_amd as fa
import oracle
from tests.gpu_util import say

U = 2.0 ** -24
LOG2E = 1.4426950408889634


def gamma(n):
    n = np.asarray(n, dtype=np.float64)
    return n * U / (1.0 - n * U)


def bf16r(x):
    """x rounded to fp32 and then to bfloat16 (both to nearest even), as fp64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def _f64(t):
    return t.double().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, dtype=np.float64)


def forward_inputs(q, k, v, scale, causal, heads):
    """o (bf16) and lse (fp32) of the listed (b, h) query heads, from the fp64
    oracle, rounded as the forward stores them.  Returns {(b, h): (o [Nq, d]
    torch bf16, lse [Nq] torch fp32)}."""
    B, Nq, Hq, d = q.shape
    rows = np.array([(b, h, i) for b, h in heads for i in range(Nq)], dtype=np.int32)
    ro, rl = oracle.attention(q, k, v, scale, causal, rows=rows)
    out = {}
    for n, (b, h) in enumerate(heads):
        o = torch.from_numpy(ro[n * Nq:(n + 1) * Nq].astype(np.float32)).to(torch.bfloat16)
        lse = torch.from_numpy(rl[n * Nq:(n + 1) * Nq].astype(np.float32))
        out[(b, h)] = (o, lse)
    return out


def gpu_fwd_bwd(q, k, v, do, causal, scale, groups=None):
    """The backward through libfa.so on host tensors.  o and lse come from the
    GPU forward and, for the query heads of the listed (b, hk) groups (None:
    all), are replaced by the oracle's (forward_inputs), so that the checked
    gradients depend only on oracle-side values.  Returns host (dq, dk, dv,
    o, lse), o and lse as passed to the backward."""
    B, Nq, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    if groups is None:
        groups = [(b, hk) for b in range(B) for hk in range(Hkv)]
    heads = [(b, hk * g + j) for b, hk in groups for j in range(g)]
    ref = forward_inputs(q, k, v, scale, causal, heads)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for (b, h), (ro, rl) in ref.items():
        o[b, :, h] = ro
        lse[b, h] = rl
    dq, dk, dv = fa.bwd(qd, kd, vd, o.cuda(), lse.cuda(), dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu(), o, lse


def bwd_intervals(q, k, v, do, o, lse, scale, causal, b, hk, exact=False):
    """Per-element intervals [lo, hi] for the bf16 gradients of group (b, hk)
    (see the module docstring): dq [g, Nq, d], dk [Nk, d], dv [Nk, d], each
    as a (lo, hi) pair of fp64 arrays.  exact=True drops every rounding (lo
    = hi = the exact gradient of the same o and lse), which pins the
    formulas to the oracle."""
    rnd = (lambda x: np.asarray(x, dtype=np.float64)) if exact else bf16r
    gam = (lambda n: 0.0 * np.asarray(n, dtype=np.float64)) if exact else gamma
    u = 0.0 if exact else U
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    s32 = float(np.float32(scale))
    c = float(np.float32(abs(s32) * LOG2E)) if s32 != 0 else 0.0
    K, V = _f64(k[b, :, hk]), _f64(v[b, :, hk])
    aK, aV = np.abs(K), np.abs(V)
    if causal:
        vis = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)
    else:
        vis = np.ones((Nq, Nk), dtype=bool)
    gd = gam(d + 2)
    dk_c = np.zeros((Nk, d)); dk_w = np.zeros((Nk, d)); dk_a = np.zeros((Nk, d))
    dv_c = np.zeros((Nk, d)); dv_w = np.zeros((Nk, d)); dv_a = np.zeros((Nk, d))
    dq_iv = []
    for j in range(g):
        h = hk * g + j
        Q, dO, O = _f64(q[b, :, h]), _f64(do[b, :, h]), _f64(o[b, :, h])
        L = _f64(lse[b, h])
        S = Q @ K.T
        S1 = np.abs(Q) @ aK.T
        live = vis & np.isfinite(L)[:, None]
        Lf = np.where(np.isfinite(L), L, 0.0)
        P = np.where(live, np.exp(np.where(live, s32 * S - Lf[:, None], 0.0)), 0.0)
        # error of the exponent argument (base 2): scores, c and lse2 in fp32, the fma
        l2 = np.abs(Lf) * LOG2E
        darg = c * gd * S1 + 2 * u * c * np.abs(S) + 4 * u * l2[:, None] + u * (c * np.abs(S) + l2[:, None])
        dP_ = np.where(live, P * (np.expm1(np.log(2.0) * darg) + 4 * u) * (1 + 16 * u) + u * 2.0 ** -102, 0.0)
        dPm = dO @ V.T
        D1 = np.abs(dO) @ aV.T
        delta = (dO * O).sum(axis=1)
        E = np.abs(dO * O).sum(axis=1)
        T = dPm - delta[:, None]
        dT = gd * (D1 + E[:, None])
        dT = dT + u * (np.abs(T) + dT)
        DS = P * T
        dDS = np.where(live, (dP_ * (np.abs(T) + dT) + P * dT) * (1 + u) + u * np.abs(DS) + u * 2.0 ** -102, 0.0)
        ds_lo, ds_hi = rnd(DS - dDS), rnd(DS + dDS)
        p_lo, p_hi = rnd(P - dP_), rnd(P + dP_)
        ds_c, ds_w, ds_m = (ds_lo + ds_hi) / 2, (ds_hi - ds_lo) / 2, np.maximum(np.abs(ds_lo), np.abs(ds_hi))
        p_c, p_w, p_m = (p_lo + p_hi) / 2, (p_hi - p_lo) / 2, np.maximum(np.abs(p_lo), np.abs(p_hi))
        n_row = np.maximum(vis.sum(axis=1), 1)
        # dq = scale * sum_j bf16(ds) k: interval of the sum, fp32 accumulation, the scale, bf16
        acc_c = ds_c @ K
        acc_r = ds_w @ aK + gam(n_row)[:, None] * (ds_m @ aK)
        dq_iv.append(_scaled_bf16(acc_c, acc_r, s32, rnd, u))
        dk_c += ds_c.T @ Q; dk_w += ds_w.T @ np.abs(Q); dk_a += ds_m.T @ np.abs(Q)
        dv_c += p_c.T @ dO; dv_w += p_w.T @ np.abs(dO); dv_a += p_m.T @ np.abs(dO)
    n_col = np.maximum(g * vis.sum(axis=0), 1)[:, None]
    dk_iv = _scaled_bf16(dk_c, dk_w + gam(n_col) * dk_a, s32, rnd, u)
    dv_iv = _scaled_bf16(dv_c, dv_w + gam(n_col) * dv_a, 1.0, rnd, u)
    dq_lo = np.stack([x[0] for x in dq_iv]); dq_hi = np.stack([x[1] for x in dq_iv])
    return (dq_lo, dq_hi), dk_iv, dv_iv


def _scaled_bf16(center, radius, scale, rnd, u):
    """Roundings (rnd: to bf16) of the ends of scale * [center - radius,
    center + radius], the product in fp32 (one rounding of relative size u)."""
    a, b = scale * (center - radius), scale * (center + radius)
    lo, hi = np.minimum(a, b), np.maximum(a, b)
    lo = lo - u * np.abs(lo)
    hi = hi + u * np.abs(hi)
    return rnd(lo), rnd(hi)


def compare_bwd(q, k, v, do, causal, scale, dq, dk, dv, o, lse, groups=None, label=""):
    """dq, dk, dv from the GPU ([B, N, H, d] host tensors), computed from o and
    lse, against the fp64 oracle on the listed (b, hk) groups: every element
    must lie in its interval (bwd_intervals), which bounds its distance to
    the oracle's gradient."""
    B, Nq, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    if groups is None:
        groups = [(b, hk) for b in range(B) for hk in range(Hkv)]
    ref = oracle.attention_bwd(q, k, v, do, scale, causal, groups=groups)
    for n, (b, hk) in enumerate(groups):
        ivs = bwd_intervals(q, k, v, do, o, lse, scale, causal, b, hk)
        mine = (dq[b, :, hk * g:(hk + 1) * g].permute(1, 0, 2).double().numpy(),
                dk[b, :, hk].double().numpy(), dv[b, :, hk].double().numpy())
        for name, m, r, (lo, hi) in zip(("dq", "dk", "dv"), mine, (ref[0][n], ref[1][n], ref[2][n]), ivs):
            assert np.all(np.isfinite(m)), f"{name}: non-finite output"
            bad = (m < lo) | (m > hi)
            e = np.abs(m - r)
            tol = np.maximum(np.abs(lo - r), np.abs(hi - r))
            say(f"[bwd] {label} ({b},{hk}) {name}: max|err| {e.max():.3e} mean {e.mean():.3e} | implied bound "
                f"max {tol.max():.3e} mean {tol.mean():.3e} | max|ref| {np.abs(r).max():.3e}")
            if bad.any():
                i = np.argwhere(bad)[0]
                raise AssertionError(f"{label} ({b},{hk}) {name}: {int(bad.sum())} elements outside their interval, "
                                     f"first {tuple(i)}: {m[tuple(i)]!r} not in [{lo[tuple(i)]!r}, {hi[tuple(i)]!r}], "
                                     f"oracle {r[tuple(i)]!r}")
