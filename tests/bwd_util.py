"""Helpers for the backward GPU tests: the HIP path, the fp64 oracle on the
same host values, and a plain PyTorch bf16 evaluation for the tolerance."""
from __future__ import annotations

import numpy as np
import torch

import exact_attention_93_amd as fa
import oracle
from tests.gpu_util import say


def gpu_fwd_bwd(q, k, v, do, causal, scale):
    """Forward then backward through libfa.so on host tensors; host results."""
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def torch_bf16_grads(q, k, v, do, causal, scale, groups):
    """softmax(scale q k^T + mask) v and its gradients evaluated by PyTorch in
    bfloat16 on the CPU (autograd), for the listed (b, hk) groups:
    dq [G, g, Nq, d], dk and dv [G, Nk, d] as float64."""
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    outs = ([], [], [])
    keep = torch.ones(Nq, Nk, dtype=torch.bool).tril(Nk - Nq) if causal else None
    for b, hk in groups:
        tq = q[b, :, hk * g:(hk + 1) * g].permute(1, 0, 2).contiguous().requires_grad_()   # [g, Nq, d]
        tk = k[b, :, hk].contiguous().requires_grad_()                                     # [Nk, d]
        tv = v[b, :, hk].contiguous().requires_grad_()
        s = torch.matmul(tq, tk.t().contiguous()) * scale
        if keep is not None:
            s = s.masked_fill(~keep, float("-inf"))
        pm = torch.softmax(s, dim=-1)
        pm = torch.nan_to_num(pm, nan=0.0)
        o = torch.matmul(pm, tv)
        o.backward(do[b, :, hk * g:(hk + 1) * g].permute(1, 0, 2).contiguous())
        outs[0].append(tq.grad.double().numpy())
        outs[1].append(tk.grad.double().numpy())
        outs[2].append(tv.grad.double().numpy())
    return tuple(np.stack(x) for x in outs)


def compare_bwd(q, k, v, do, causal, scale, dq, dk, dv, groups=None, label="", factor=2.0):
    """dq, dk, dv from the GPU ([B, N, H, d] host tensors) against the fp64
    oracle on the listed (b, hk) groups.  Bound for each gradient: the largest
    error of the plain PyTorch bf16 evaluation times `factor`, and the mean
    error likewise."""
    B, Nq, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    if groups is None:
        groups = [(b, hk) for b in range(B) for hk in range(Hkv)]
    ref = oracle.attention_bwd(q, k, v, do, scale, causal, groups=groups)
    tb = torch_bf16_grads(q, k, v, do, causal, scale, groups)
    mine = (np.stack([dq[b, :, hk * g:(hk + 1) * g].permute(1, 0, 2).double().numpy() for b, hk in groups]),
            np.stack([dk[b, :, hk].double().numpy() for b, hk in groups]),
            np.stack([dv[b, :, hk].double().numpy() for b, hk in groups]))
    res = {}
    for name, m, r, t in zip(("dq", "dk", "dv"), mine, ref, tb):
        assert np.all(np.isfinite(m)), f"{name}: non-finite output"
        e, et = np.abs(m - r), np.abs(t - r)
        res[name] = (float(e.max()), float(e.mean()), float(et.max()), float(et.mean()), float(np.abs(r).max()))
        say(f"[bwd] {label} {name}: max|err| {e.max():.3e} mean {e.mean():.3e} | torch-bf16 max {et.max():.3e} "
            f"mean {et.mean():.3e} | max|ref| {np.abs(r).max():.3e}")
    # fp32 accumulation noise, relative to the largest gradient of the call:
    # where an exact gradient is zero (one key, zero scale) the bf16
    # evaluation can hit it exactly while fp32 sums in another order leave
    # cancellation residue of this size
    floor = 2.0 ** -16 * max(r[4] for r in res.values())
    for name, (mx, mn, tmx, tmn, rmax) in res.items():
        assert mx <= factor * tmx + floor, f"{name}: max error {mx:.3e} > {factor} x {tmx:.3e}"
        assert mn <= factor * tmn + floor, f"{name}: mean error {mn:.3e} > {factor} x {tmn:.3e}"
    return res
