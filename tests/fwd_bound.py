"""The per-element bound of the forward GPU tests: an interval for every
output element and log-sum-exp, derived from the arithmetic the forward
kernels perform ("FlashAttention：IO 感知的精确注意力", sections 5 and 7.1;
"[Attention优化] 从Online-Softmax到FlashAttention V1/V2/V3", sections 0x04
and 0x05; the split merge of the first page's section 12.1), written out in
fp64 here.

For a query row and its visible keys j, every forward path (bf16 and fp32,
whole or split key range, the decoding kernel) computes

  s_j = q.k_j              fp32 accumulation of exact (bf16) or rounded (fp32) products
  p_j = 2^(c s_j - m)      c = fp32(|scale| log2 e), one fma, the hardware exp2; m a
                           reference of the kernel's choosing (any m gives the same softmax)
  O = sum_j P_j v_j / sum_j P_j
                           P_j = p_j rounded to bf16 (bf16 paths) or p_j itself (fp32),
                           times the rescale factors 2^(m_old - m_new) (fp32, rounded)
                           applied since it was added; fp32 sums
  lse = m ln 2 + ln sum_j p_j   (fp32 sum of the unrounded p_j)

and a split call merges the ranges' normalised (O_r, lse_r) with weights
exp(lse_r - M), M = max_r lse_r, in fp32.  So the kernel's O is a weighted
average of the v_j whose weights are omega_j = p_j (1 + delta_j) up to one
common factor, where |delta_j| <= Delta_j collects, as relative factors:
bf16 rounding of P (2^-8), the exp2 error (4u), the exponent argument's error
(c gamma_{d+2} sum|q||k| for the scores, 2u |c s| for c and the fma, 2u |m|
for the reference), the rescales (each re-weights the keys added before it by
its exp2 error, 4u, at most one per tile the row sees, plus the fp32
differences' rounding, at most 2u |m| over the reference's whole climb), and
for a merged split call the ranges' normalisation (a range is normalised by
the sum of its rounded probabilities and weighted by the sum of the unrounded
ones: a factor within (1 + 2^-8)/(1 - 2^-8), fp32 sums aside) and the merge
weights' fp32 logarithms and exponentials.  With W the exact weights and O
the exact average (sum_j W_j (v_j - O) = 0):

  |O' - O| <= sum_j p_j Delta_j |v_j - O| / sum_j p_j (1 - Delta_j)

and the fp32 accumulations add gamma_n times the sums of magnitudes, n the
roundings a term can pass through (at most the keys of one range, one per
rescale, one per range in the merge); the final division adds a few units u;
both ends of O +- that radius are rounded to the output format (rounding is
monotone).  u = 2^-24; gamma_n = n u / (1 - n u).
exact=True drops every rounding, so the intervals collapse to exact attention
(which pins the formulas to the oracle)."""
from __future__ import annotations

import numpy as np

U = 2.0 ** -24
U_BF16 = 2.0 ** -8          # unit roundoff of bf16 (8 significant bits), round to nearest
LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453
_TINY = 2.0 ** -125         # absolute error of a probability that flushes or rounds below fp32's normal range


def gamma(n):
    n = np.asarray(n, dtype=np.float64)
    return n * U / (1.0 - n * U)


def bf16r(x):
    """x rounded to fp32 and then to bfloat16 (both to nearest even), as fp64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def _host(t):
    if hasattr(t, "detach"):
        t = t.detach().cpu()
        return t.float().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def visible(Nq, Nk, causal, qi, h=0, block_mask=None, block=(128, 64)):
    """[len(qi), Nk] bool: key j visible to query qi (bottom-right causal
    alignment; block mask entries of (block[0] queries x block[1] keys))."""
    qi = np.asarray(qi)
    vis = np.ones((len(qi), Nk), dtype=bool)
    if causal:
        vis &= np.arange(Nk)[None, :] <= qi[:, None] + (Nk - Nq)
    if block_mask is not None:
        m = _host(block_mask)[h] != 0
        vis &= m[qi // block[0]][:, np.arange(Nk) // block[1]]
    return vis


def fwd_intervals(q, k, v, scale, causal, rows, kind="bf16", block_mask=None, block=(128, 64), exact=False,
                  split=True, range_keys=None, loose_above=5e7):
    """Intervals for the forward outputs of the listed (b, h, i) rows:
    (o_lo, o_hi [R, d], lse_lo, lse_hi [R]) as fp64 arrays.  kind: "bf16"
    (bf16 probabilities and output) or "fp32".  split: the call may merge
    several key ranges (True covers both); range_keys: an upper bound on the
    keys of one range (None: all of them), which bounds the length of each
    accumulation chain (one rounding per key of the range, at most, and one
    per range in the merge) and the rescales.  Rows without a visible key get
    O = 0 and lse = -inf exactly.  Where a head's rows x keys x d exceeds
    loose_above, |v_j - O| is bounded by |v_j| + |O| (two products instead of
    a per-row pass)."""
    q, k, v = _host(q), _host(k), _host(v)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    rows = np.asarray(rows).reshape(-1, 3)
    R = len(rows)
    u = 0.0 if exact else U
    up = 0.0 if (exact or kind == "fp32") else U_BF16
    gam = (lambda n: 0.0 * np.asarray(n, dtype=np.float64)) if exact else gamma
    s32 = float(np.float32(scale))
    sign = 1.0 if s32 > 0 else (-1.0 if s32 < 0 else 0.0)
    c_ex = abs(s32) * LOG2E                                  # exact base-2 factor of the oracle
    c32 = float(np.float32(c_ex)) if s32 != 0 else 0.0
    rk = Nk if range_keys is None else min(Nk, int(range_keys))
    nranges = -(-Nk // rk)
    nres = rk // 32 + 2                                      # rescales per row and range (tiles of >= 32 keys)
    depth_cap = rk + nranges + nres + 200                    # roundings a term passes through, at most
    o_lo = np.zeros((R, d)); o_hi = np.zeros((R, d))
    l_lo = np.full(R, -np.inf); l_hi = np.full(R, -np.inf)
    groups = []
    for (b, h) in sorted({(int(r[0]), int(r[1])) for r in rows}):
        sel_all = np.nonzero((rows[:, 0] == b) & (rows[:, 1] == h))[0]
        step = max(1, (1 << 24) // Nk)                       # rows per pass: at most 2^24 scores
        groups.extend((b, h, sel_all[i:i + step]) for i in range(0, len(sel_all), step))
    for (b, h, sel) in groups:
        qi = rows[sel, 2]
        hk = h // g
        Q, K, V = q[b, qi, h], k[b, :, hk], v[b, :, hk]
        vis = visible(Nq, Nk, causal, qi, h, block_mask, block)
        live = vis.any(axis=1)
        nvis = vis.sum(axis=1)
        nr = np.minimum(nvis, nres)                           # a rescale needs a tile the row sees
        S = sign * (Q @ K.T)
        S1 = np.abs(Q) @ np.abs(K).T
        A = np.where(vis, c_ex * S, -np.inf)                  # exact base-2 exponents
        mx = np.where(live, A.max(axis=1), 0.0)
        P = np.where(vis, np.exp2(np.where(vis, A - mx[:, None], 0.0)), 0.0)
        sp = P.sum(axis=1)
        sp1 = np.where(live, sp, 1.0)
        W = P / sp1[:, None]
        O = W @ V
        lse = np.where(live, LN2 * (mx + np.log2(sp1)), -np.inf)
        # reference magnitude: |m| <= max |c s| + 8 (the lazy threshold) + 1
        mb = np.where(live, np.max(np.where(vis, np.abs(A), 0.0), axis=1), 0.0) + 9.0
        darg = c32 * gam(d + 2) * S1 + 2 * u * np.abs(np.where(vis, A, 0.0)) + 2 * u * mb[:, None]
        # A rescale multiplies a row's numerator and denominator by the same
        # rounded 2^(m_old - m_new), so its error only re-weights the keys
        # added before it: the exp2 error (4u) each time, and the fp32
        # differences' rounding, u |m_old - m_new| each, at most 2u mb over
        # the reference's whole climb.  (The multiplications' own roundings
        # count among the accumulations' roundings.)
        resc = (1 + 4 * u) ** nr * np.exp(LN2 * u * 2 * mb)
        base = (1 + 4 * u) * np.exp(LN2 * darg) * resc[:, None]
        Dl = np.where(vis, base - 1.0, 0.0)                    # unrounded probabilities (the lse sum)
        Dp = np.where(vis, (1 + up) * base - 1.0, 0.0)         # the probabilities the products take
        # split calls: a range is normalised by its sum of the probabilities
        # the products take, and weighted by its sum of the unrounded ones,
        # which differ by the bf16 rounding alone (and the fp32 sums); and
        # the merge weights' fp32 logarithms and exponentials
        Lmag = np.where(live, np.abs(lse), 0.0) + LN2 * mb
        e_w = np.where(live, (1 + 4 * u) * np.exp(4 * u * Lmag + 2 * u * np.abs(np.log(sp1))) - 1.0, 0.0)
        if split:
            gr = gam(np.minimum(nvis, rk) + nr + 8)
            fac = (1 + e_w) * (1 + gr) ** 2 / ((1 - up) * (1 - gr))
            Dt = np.where(vis, (1 + Dp) * fac[:, None] - 1.0, 0.0)
        else:
            Dt = Dp
        dtmax = np.max(Dt, axis=1)
        PD = P * Dt
        den = np.maximum((P * (1 - Dt)).sum(axis=1), 1e-300)
        if len(qi) * Nk * d > loose_above:
            E1 = (PD @ np.abs(V) + np.abs(O) * PD.sum(axis=1)[:, None]) / den[:, None]
        else:
            E1 = np.empty_like(O)
            for r0 in range(0, len(qi), 16):
                blk = np.abs(V[None, :, :] - O[r0:r0 + 16, None, :])           # [r, Nk, d]
                E1[r0:r0 + 16] = np.einsum("rj,rjd->rd", PD[r0:r0 + 16], blk) / den[r0:r0 + 16, None]
        grow = ((1 + dtmax) / (1 - dtmax))[:, None]
        E2 = gam(np.minimum(nvis + nr + 200, depth_cap))[:, None] * (W @ np.abs(V) + np.abs(O) + E1) * grow
        E3 = 6 * u * (np.abs(O) + E1 + E2)
        E4 = (nvis * _TINY * (0.0 if exact else 2.0))[:, None] * np.max(np.abs(V))
        E = E1 + E2 + E3 + E4
        lo, hi = O - E, O + E
        if kind == "bf16" and not exact:
            lo, hi = bf16r(lo), bf16r(hi)
        elif not exact:
            lo, hi = lo - u * np.abs(lo), hi + u * np.abs(hi)
        lo = np.where(live[:, None], lo, 0.0)
        hi = np.where(live[:, None], hi, 0.0)
        # log-sum-exp: the unrounded sum's relative error, the fp32 logarithm,
        # m ln 2, the additions, and the merge (split calls)
        dl = np.max(Dl, axis=1) + gam(np.minimum(nvis + nr + 8, depth_cap)) * (1 + np.max(Dl, axis=1))
        El = -np.log1p(-np.minimum(dl, 0.5)) + 8 * u * Lmag + (2 * e_w if split else 0.0)
        El = np.where(live, El + u * np.abs(np.where(live, lse, 0.0)), 0.0)
        o_lo[sel], o_hi[sel] = lo, hi
        l_lo[sel] = np.where(live, lse - El, -np.inf)
        l_hi[sel] = np.where(live, lse + El, -np.inf)
    return o_lo, o_hi, l_lo, l_hi
