"""Step-by-step CPU forms of the softmax / attention recurrences on the pages.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.

Every function here follows one algorithm the pages describe, in the pages'
order and notation, with plain loops over numpy vectors.  Nothing is blocked,
fused or reordered beyond what that algorithm states.  They serve two roles:

* they are pinned directly against the numbers the pages print for their
  hand-worked example, and
* they give independent routes (1-pass, 2-pass, tiled) to the same result as
  the 3-pass definition in ``ref.c``, so that the tests can hold the routes
  against each other ("the result is the same up to floating-point rounding").

``dtype`` selects the working precision (float64 by default; float32 for the
rounding-error exercise of the second page).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def softmax_3pass(x, dtype=np.float64):
    """Safe softmax in three passes.

    "[Attention优化] 从Online-Softmax到FlashAttention V1/V2/V3", section 0x02:
    pass 1 finds the maximum, pass 2 sums exp(x - max), pass 3 divides.
    """
    x = np.asarray(x, dtype=dtype)
    m = dtype(NEG_INF)
    for xi in x:                      # pass 1
        m = max(m, xi)
    d = dtype(0)
    for xi in x:                      # pass 2
        d = d + np.exp(xi - m)
    return np.array([np.exp(xi - m) / d for xi in x], dtype=dtype)  # pass 3


def online_softmax_2pass(x, dtype=np.float64):
    """Online softmax: the max and the normaliser in one pass, then normalise.

    Same page, section 0x03; "Flash-attention 学习", section 0 (Online Softmax):
        m_i  = max(m_{i-1}, x_i)
        d'_i = d'_{i-1} * exp(m_{i-1} - m_i) + exp(x_i - m_i)
    and a_i = exp(x_i - m_N) / d'_N in the second pass.
    Returns (a, m_N, d'_N).
    """
    x = np.asarray(x, dtype=dtype)
    m = dtype(NEG_INF)
    dp = dtype(0)
    for xi in x:
        m_new = max(m, xi)
        dp = dp * np.exp(m - m_new) + np.exp(xi - m_new)
        m = m_new
    a = np.array([np.exp(xi - m) / dp for xi in x], dtype=dtype)
    return a, m, dp


def attention_1pass_row(x, V, dtype=np.float64):
    """1-pass attention for one query row: scores x (length N), values V [N, d].

    "Flash-attention 学习", section 1 (and section 0x04 of the first page):
        o'_i = exp(m_{i-1} - m_i) * (d'_{i-1} / d'_i) * o'_{i-1}
               + exp(x_i - m_i) / d'_i * V[i, :]
    Returns (o'_N, m_N, d'_N).
    """
    x = np.asarray(x, dtype=dtype)
    V = np.asarray(V, dtype=dtype)
    m = dtype(NEG_INF)
    dp = dtype(0)
    o = np.zeros(V.shape[1], dtype=dtype)
    for i, xi in enumerate(x):
        m_new = max(m, xi)
        dp_new = dp * np.exp(m - m_new) + np.exp(xi - m_new)
        o = np.exp(m - m_new) * (dp / dp_new) * o + (np.exp(xi - m_new) / dp_new) * V[i]
        m, dp = m_new, dp_new
    return o, m, dp


def blocked_row(s, V, sizes, mode="fa1", dtype=np.float64):
    """Merge one score row block by block with the running (m, l, O) state.

    ``sizes`` is the list of block lengths (they must add up to len(s)).

    mode "fa1": the normalised update of "FlashAttention：IO 感知的精确注意力",
    section 5 and Algorithm 1 steps 8-11 (section 7.1):
        m~ = max(block), P~ = exp(block - m~), l~ = sum P~
        m_new = max(m, m~)
        l_new = exp(m - m_new) l + exp(m~ - m_new) l~
        O_new = (exp(m - m_new) l O + exp(m~ - m_new) P~ V_block) / l_new

    mode "fa2": the deferred normalisation of the FlashAttention-2 discussion
    (first page section 0x05; "Flash-attention 学习" section 2.1): the
    accumulator stays unnormalised and is only rescaled by exp(m - m_new);
    the single division by l happens after the last block.

    Returns a list with one dict per block: m, l, and O (normalised output of
    the prefix seen so far; for "fa2" also ``acc``, the unnormalised sum).
    Initial state m = -inf, l = 0, O = 0 (Algorithm 1 step 2).  A block row
    whose entries are all -inf contributes nothing (its P~ is taken as 0).
    """
    s = np.asarray(s, dtype=dtype)
    V = np.asarray(V, dtype=dtype)
    if V.ndim == 1:
        V = V[:, None]
    assert sum(sizes) == len(s)
    m = dtype(NEG_INF)
    l = dtype(0)
    O = np.zeros(V.shape[1], dtype=dtype)
    acc = np.zeros(V.shape[1], dtype=dtype)
    trace = []
    start = 0
    for size in sizes:
        blk = s[start:start + size]
        vb = V[start:start + size]
        start += size
        mt = blk.max()
        if mt == NEG_INF:
            Pt = np.zeros_like(blk)
        else:
            Pt = np.exp(blk - mt)
        lt = Pt.sum(dtype=dtype)
        m_new = max(m, mt)
        a_old = dtype(0) if m == NEG_INF else np.exp(m - m_new)
        a_new = dtype(0) if mt == NEG_INF else np.exp(mt - m_new)
        l_new = a_old * l + a_new * lt
        if mode == "fa1":
            O = (a_old * l * O + a_new * (Pt @ vb)) / l_new
            trace.append({"m": m_new, "l": l_new, "O": O.copy()})
        elif mode == "fa2":
            # P~ taken relative to the running maximum directly, then the
            # accumulator is rescaled by exp(m - m_new) only.
            Pm = np.zeros_like(blk) if m_new == NEG_INF else np.exp(blk - m_new)
            acc = a_old * acc + Pm @ vb
            trace.append({"m": m_new, "l": l_new, "acc": acc.copy(), "O": acc / l_new})
        else:
            raise ValueError(mode)
        m, l = m_new, l_new
    return trace


def _scores(Q, K, scale, causal, dtype):
    S = (Q @ K.T) * dtype(scale)
    if causal:
        n = S.shape[0]
        S = np.where(np.arange(n)[None, :] <= np.arange(n)[:, None], S, NEG_INF)
    return S


def fa1_forward(Q, K, V, Br, Bc, scale=1.0, causal=False, dtype=np.float64):
    """FlashAttention-1 forward for one head, loop order of Algorithm 1.

    "FlashAttention：IO 感知的精确注意力", section 7.1: the outer loop walks the
    K/V blocks, the inner loop walks the Q blocks, and O, l, m of every Q block
    are read and written back on each inner step.  The score block is
    Q_i K_j^T (scaled; causal entries with key > query set to -inf).
    Returns (O, lse) with lse = m + ln l.
    """
    Q = np.asarray(Q, dtype=dtype)
    K = np.asarray(K, dtype=dtype)
    V = np.asarray(V, dtype=dtype)
    N, d = Q.shape
    O = np.zeros((N, d), dtype=dtype)
    l = np.zeros(N, dtype=dtype)
    m = np.full(N, NEG_INF, dtype=dtype)
    for j0 in range(0, N, Bc):                       # K/V blocks
        Kj, Vj = K[j0:j0 + Bc], V[j0:j0 + Bc]
        for i0 in range(0, N, Br):                   # Q blocks
            Qi = Q[i0:i0 + Br]
            S = (Qi @ Kj.T) * dtype(scale)
            if causal:
                qi = np.arange(i0, i0 + Qi.shape[0])[:, None]
                kj = np.arange(j0, j0 + Kj.shape[0])[None, :]
                S = np.where(kj <= qi, S, NEG_INF)
            for r in range(Qi.shape[0]):
                row = i0 + r
                mt = S[r].max()
                if mt == NEG_INF:
                    continue                          # nothing visible in this block
                Pt = np.exp(S[r] - mt)
                lt = Pt.sum(dtype=dtype)
                m_new = max(m[row], mt)
                a_old = dtype(0) if m[row] == NEG_INF else np.exp(m[row] - m_new)
                a_new = np.exp(mt - m_new)
                l_new = a_old * l[row] + a_new * lt
                O[row] = (a_old * l[row] * O[row] + a_new * (Pt @ Vj)) / l_new
                m[row], l[row] = m_new, l_new
    return O, m + np.log(l)


def fa2_forward(Q, K, V, Br, Bc, scale=1.0, causal=False, dtype=np.float64):
    """FlashAttention-2 forward for one head: Q-block outer loop, deferred 1/l.

    First page section 0x05 and "Flash-attention 学习" section 2.2: each Q
    block is independent and loops over all K/V blocks it can see (blocks
    entirely above the causal diagonal are skipped, first page section 0x09);
    the accumulator is rescaled by exp(m_old - m_new) and divided by l once at
    the end.  Returns (O, lse).
    """
    Q = np.asarray(Q, dtype=dtype)
    K = np.asarray(K, dtype=dtype)
    V = np.asarray(V, dtype=dtype)
    N, d = Q.shape
    O = np.zeros((N, d), dtype=dtype)
    lse = np.zeros(N, dtype=dtype)
    for i0 in range(0, N, Br):
        Qi = Q[i0:i0 + Br]
        nr = Qi.shape[0]
        acc = np.zeros((nr, d), dtype=dtype)
        l = np.zeros(nr, dtype=dtype)
        m = np.full(nr, NEG_INF, dtype=dtype)
        j_end = min(N, i0 + nr) if causal else N
        for j0 in range(0, j_end, Bc):
            Kj, Vj = K[j0:j0 + Bc], V[j0:j0 + Bc]
            S = (Qi @ Kj.T) * dtype(scale)
            if causal:
                qi = np.arange(i0, i0 + nr)[:, None]
                kj = np.arange(j0, j0 + Kj.shape[0])[None, :]
                S = np.where(kj <= qi, S, NEG_INF)
            m_new = np.maximum(m, S.max(axis=1))
            safe = np.where(m_new == NEG_INF, dtype(0), m_new)
            alpha = np.where(m == NEG_INF, dtype(0), np.exp(m - safe))
            P = np.exp(S - safe[:, None])
            l = alpha * l + P.sum(axis=1, dtype=dtype)
            acc = alpha[:, None] * acc + P @ Vj
            m = m_new
        O[i0:i0 + nr] = acc / l[:, None]
        lse[i0:i0 + nr] = m + np.log(l)
    return O, lse
