"""The per-element bound of the backward tests (tests/bwd_util.py), pinned on
the CPU.

- With every rounding dropped, the interval collapses to the exact gradient
  of the same o and lse; on o and lse from the oracle's forward it must
  equal the C oracle's gradient (so a dropped term, a wrong sign or a
  transposed operand in the bound's own formulas fails here).
- An fp32 evaluation of the backward's arithmetic, written here
  independently (fp32 scores, exp2, dP and delta; dS and P rounded to bf16
  for the products; fp32 sums; bf16 output), must fall inside the intervals:
  the bound is not tighter than the arithmetic it describes.
- The same evaluation with a planted mistake must fall outside: the bound is
  tight enough to catch it."""
import numpy as np
import pytest
import torch

import oracle
from tests.bwd_util import LOG2E, bf16r, bwd_intervals, forward_inputs

CASES = [  # B, Nq, Nk, Hq, Hkv, d, causal, scale
    (1, 37, 37, 2, 2, 64, False, 0.125),
    (1, 70, 70, 4, 2, 64, True, 0.125),
    (2, 33, 90, 2, 1, 128, True, 0.0884),
    (1, 90, 33, 2, 1, 64, True, 0.125),
    (1, 50, 50, 2, 2, 64, True, -0.2),
    (1, 40, 40, 2, 1, 64, False, 0.0),
]


def inputs(B, Nq, Nk, Hq, Hkv, d, seed, q_std=1.0):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn((B, Nq, Hq, d), generator=g) * q_std).to(torch.bfloat16)
    k = torch.randn((B, Nk, Hkv, d), generator=g).to(torch.bfloat16)
    v = torch.randn((B, Nk, Hkv, d), generator=g).to(torch.bfloat16)
    do = torch.randn((B, Nq, Hq, d), generator=g).to(torch.bfloat16)
    return q, k, v, do


def rounded_forward(q, k, v, scale, causal):
    """o (bf16) and lse (fp32) for every head, from the oracle."""
    B, Nq, Hq, d = q.shape
    ref = forward_inputs(q, k, v, scale, causal, [(b, h) for b in range(B) for h in range(Hq)])
    o = torch.empty((B, Nq, Hq, d), dtype=torch.bfloat16)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32)
    for (b, h), (ro, rl) in ref.items():
        o[b, :, h] = ro
        lse[b, h] = rl
    return o, lse


def emulate(q, k, v, do, o, lse, scale, causal, b, hk, mistake=None):
    """The backward's arithmetic in fp32 (bf16 operands of the products) for
    group (b, hk): (dq [g, Nq, d], dk [Nk, d], dv [Nk, d]) as fp64."""
    f32, f64 = np.float32, np.float64
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    s32 = f32(scale)
    if s32 > 0:
        sign, c = 1.0, f32(f64(s32) * LOG2E)
    elif s32 < 0:
        sign, c = -1.0, f32(-f64(s32) * LOG2E)
    else:
        sign, c = 0.0, f32(1.0)
    K, V = k[b, :, hk].float().numpy(), v[b, :, hk].float().numpy()
    if causal:
        off = 0 if mistake == "top_left" else Nk - Nq
        vis = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + off
    else:
        vis = np.ones((Nq, Nk), dtype=bool)
    dk_acc = np.zeros((Nk, d), dtype=f32)
    dv_acc = np.zeros((Nk, d), dtype=f32)
    dqs = []
    for j in range(g):
        h = hk * g + j
        Q, dO, O = q[b, :, h].float().numpy(), do[b, :, h].float().numpy(), o[b, :, h].float().numpy()
        L = lse[b, h].numpy()
        S = (f32(sign) * Q) @ K.T
        with np.errstate(invalid="ignore"):
            l2 = L if mistake == "natural_log" else (L * f32(LOG2E)).astype(f32)
        l2 = np.where(np.isfinite(L), l2, np.inf).astype(f32)
        with np.errstate(invalid="ignore", over="ignore"):
            arg = (S.astype(f64) * f64(c) - l2.astype(f64)[:, None]).astype(f32)   # one rounding, as the fma
            p = np.exp2(arg).astype(f32)
        p = np.where(vis & np.isfinite(L)[:, None], p, f32(0))
        dp = dO @ V.T
        delta = np.zeros(Nq, dtype=f32) if mistake == "no_delta" else (dO * O).sum(axis=1, dtype=f32)
        t = (dp - delta[:, None]).astype(f32)
        ds = (p * t).astype(f32)
        dsb, pb = bf16r(ds).astype(f32), bf16r(p).astype(f32)
        acc = dsb @ K
        dqs.append(bf16r(acc if mistake == "dq_unscaled" else (acc * s32).astype(f32)))
        dk_acc += dsb.T @ Q
        dv_acc += (dsb if mistake == "dv_from_ds" else pb).T @ dO
    return np.stack(dqs), bf16r((dk_acc * s32).astype(f32)), bf16r(dv_acc)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}q{}k{}h{}/{}d{}{}s{}".format(*c))
def test_exact_intervals_are_the_oracle_gradient(case):
    B, Nq, Nk, Hq, Hkv, d, causal, scale = case
    q, k, v, do = inputs(B, Nq, Nk, Hq, Hkv, d, seed=Nq + Nk + d)
    rows = np.array([(b, h, i) for b in range(B) for h in range(Hq) for i in range(Nq)], dtype=np.int32)
    ro, rl = oracle.attention(q, k, v, scale, causal, rows=rows)
    o = ro.reshape(B, Hq, Nq, d).transpose(0, 2, 1, 3)            # exact, unrounded
    lse = rl.reshape(B, Hq, Nq)
    groups = [(b, hk) for b in range(B) for hk in range(Hkv)]
    ref = oracle.attention_bwd(q, k, v, do, scale, causal, groups=groups)
    for n, (b, hk) in enumerate(groups):
        ivs = bwd_intervals(q, k, v, do, o, lse, scale, causal, b, hk, exact=True)
        for name, (lo, hi), r in zip(("dq", "dk", "dv"), ivs, (ref[0][n], ref[1][n], ref[2][n])):
            assert np.array_equal(lo, hi), name
            err = np.abs(lo - r).max()
            assert err <= 1e-10 * max(1.0, np.abs(r).max()), f"{name} ({b},{hk}): {err:.3e}"


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}q{}k{}h{}/{}d{}{}s{}".format(*c))
def test_fp32_evaluation_lies_inside(case, seed):
    B, Nq, Nk, Hq, Hkv, d, causal, scale = case
    q, k, v, do = inputs(B, Nq, Nk, Hq, Hkv, d, seed=100 * seed + Nq + Nk + d, q_std=1.0 + 2.0 * seed)
    o, lse = rounded_forward(q, k, v, scale, causal)
    for b in range(B):
        for hk in range(Hkv):
            ivs = bwd_intervals(q, k, v, do, o, lse, scale, causal, b, hk)
            for name, (lo, hi), m in zip(("dq", "dk", "dv"), ivs, emulate(q, k, v, do, o, lse, scale, causal, b, hk)):
                out = (m < lo) | (m > hi)
                assert not out.any(), f"{name} ({b},{hk}): {int(out.sum())} outside, e.g. {m[out][:3]}"
                # and tight: the median interval spans at most two bf16 units of the value
                nz = np.abs(m) > 0
                if nz.any():
                    unit = 2.0 ** (np.floor(np.log2(np.abs(m[nz]))) - 7)
                    assert np.median((hi - lo)[nz] / unit) <= 2.0, name


@pytest.mark.parametrize("mistake", ["no_delta", "dq_unscaled", "natural_log", "top_left", "dv_from_ds"])
def test_planted_mistakes_fall_outside(mistake):
    caught = False
    for case in CASES:
        B, Nq, Nk, Hq, Hkv, d, causal, scale = case
        if mistake == "top_left" and not (causal and Nq != Nk):
            continue
        q, k, v, do = inputs(B, Nq, Nk, Hq, Hkv, d, seed=Nq + Nk + d)
        o, lse = rounded_forward(q, k, v, scale, causal)
        for b in range(B):
            for hk in range(Hkv):
                ivs = bwd_intervals(q, k, v, do, o, lse, scale, causal, b, hk)
                emu = emulate(q, k, v, do, o, lse, scale, causal, b, hk, mistake=mistake)
                caught |= any(((m < lo) | (m > hi)).any() for (lo, hi), m in zip(ivs, emu))
    assert caught, mistake
