"""Pins for the fp64 attention oracle: facts fixed by the pages or by mathematics.

Each pin takes an ``attention(q, k, v, scale, causal, rows=None)`` callable
with the signature of ``oracle.attention`` and raises AssertionError when the
callable disagrees with the fact.  The same pins run against the real oracle
(tests/test_oracle_pins.py) and against copies of it with a planted mistake
(tests/test_oracle_mutations.py), which must each fail at least one pin.
"""
from __future__ import annotations

import math
import os
from decimal import Decimal, getcontext

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name="worked_example.txt"):
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            vals = [float(t) for t in val.split()]
            out[key] = vals if len(vals) > 1 else vals[0]
    return out


def rand(shape, seed, scale=1.0):
    r = np.random.default_rng(seed)
    return (r.standard_normal(shape) * scale).astype(np.float32)


# ---------------------------------------------------------------- brute force
def brute_decimal(q, k, v, scale, causal, prec=40):
    """The raw (not max-shifted) softmax definition in 40-digit decimals.

    O_i = sum_j exp(s_ij) v_j / sum_j exp(s_ij), lse_i = ln sum_j exp(s_ij),
    s_ij = scale * q_i . k_j over visible keys.  Independent of the max
    subtraction the oracle performs (first page, section 0x02: the original
    softmax before the safe form).  Tiny inputs only.
    """
    getcontext().prec = prec
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    sc = Decimal(float(np.float32(scale)))
    O = np.zeros((B, Hq, Nq, d))
    L = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            for i in range(Nq):
                # causal: key j kept iff j - i <= Nk - Nq (bottom-right corner)
                J = [j for j in range(Nk) if not causal or j - i <= Nk - Nq]
                if not J:
                    L[b, h, i] = -math.inf
                    continue
                w = []
                for j in J:
                    s = sum(Decimal(float(q[b, i, h, x])) * Decimal(float(k[b, j, h // g, x])) for x in range(d))
                    w.append((sc * s).exp())
                tot = sum(w)
                for x in range(d):
                    O[b, h, i, x] = float(sum(wj * Decimal(float(v[b, j, h // g, x])) for wj, j in zip(w, J)) / tot)
                L[b, h, i] = float(tot.ln())
    return O, L


def _full(att, q, k, v, scale, causal):
    o, lse = att(q, k, v, scale, causal)
    B, N, Hq, d = q.shape
    return o.reshape(B, Hq, N, d), lse.reshape(B, Hq, N)


def pin_brute_force(att):
    for seed, (B, Hq, Hkv, Nq, Nk, d), causal in [
        (1, (1, 1, 1, 5, 5, 3), False), (2, (1, 2, 1, 7, 7, 4), True),
        (3, (2, 2, 2, 4, 4, 8), False), (4, (1, 4, 2, 9, 9, 2), True),
        (5, (1, 2, 1, 3, 8, 4), True), (6, (1, 2, 2, 8, 3, 4), True),
        (7, (2, 1, 1, 1, 6, 3), True), (8, (1, 2, 1, 6, 4, 2), False),
    ]:
        q = rand((B, Nq, Hq, d), seed)
        k = rand((B, Nk, Hkv, d), seed + 100)
        v = rand((B, Nk, Hkv, d), seed + 200)
        o, l = _full(att, q, k, v, 0.7, causal)
        ob, lb = brute_decimal(q, k, v, 0.7, causal)
        assert np.max(np.abs(o - ob)) < 1e-12, "O differs from the decimal brute force"
        fin = np.isfinite(lb)
        assert np.array_equal(np.isfinite(l), fin), "rows without keys must have lse = -inf"
        assert np.all(l[~fin] == -math.inf), "rows without keys must have lse = -inf"
        assert np.max(np.abs(l[fin] - lb[fin])) < 1e-12, "LSE differs from the decimal brute force"


def pin_bottom_right_masks(att):
    """The two causal masks printed for unequal lengths, first page, section 0x09.

    With scale = 0 every kept key gets the same weight, and with v_j the j-th
    unit vector the output row i is mask[i] / sum(mask[i]), or zero for a row
    whose mask is all zero.  lse_i = ln(number of kept keys).
    """
    gold = read_golden("causal_bottom_right.txt")
    for name, nq, nk in (("q2_k5", 2, 5), ("q5_k2", 5, 2)):
        mask = np.array([gold[f"{name}.row{i}"] if nk > 1 else [gold[f"{name}.row{i}"]]
                         for i in range(nq)], dtype=np.float64).reshape(nq, nk)
        q = rand((1, nq, 1, nk), 61)
        k = rand((1, nk, 1, nk), 62)
        v = np.eye(nk, dtype=np.float32).reshape(1, nk, 1, nk)
        o, l = _full(att, q, k, v, 0.0, True)
        for i in range(nq):
            n = mask[i].sum()
            want = mask[i] / n if n else np.zeros(nk)
            assert np.array_equal(o[0, 0, i], want), f"{name}: row {i} does not follow the printed mask"
            assert l[0, 0, i] == (math.log(n) if n else -math.inf), f"{name}: lse of row {i}"


# -------------------------------------------------------------- worked example
def pin_worked_example(att):
    """Scores (sqrt2, 1/sqrt2, 1/sqrt2) and v = (1, 0, 1): the page's example.

    "FlashAttention：IO 感知的精确注意力", section 8: the whole-row softmax gives
    a = (0.5035, 0.2483, 0.2483) and O = 0.752.  Embedded as d = 2 attention:
    q = (1, 1), k_0 = (1, 1), k_1 = (1, 0), k_2 = (0, 1), scale = 1/sqrt2.
    """
    gold = read_golden()
    q = np.array([[1, 1]] * 3, dtype=np.float32).reshape(1, 3, 1, 2)
    k = np.array([[1, 1], [1, 0], [0, 1]], dtype=np.float32).reshape(1, 3, 1, 2)
    v = np.array([[1, 7], [0, 7], [1, 7]], dtype=np.float32).reshape(1, 3, 1, 2)
    o, l = _full(att, q, k, v, 1 / math.sqrt(2), False)
    for i in range(3):
        assert abs(o[0, 0, i, 0] - gold["softmax.O"]) < 5e-4, "worked example O"
        assert abs(o[0, 0, i, 0] - gold["softmax.O4"]) < 1e-4, "worked example O (4 d.p.)"
        assert abs(o[0, 0, i, 1] - 7.0) < 1e-12, "weights must sum to one"
    # lse = ln(e^1.414 + 2 e^0.707) with the exact scores
    s = np.float32(1 / math.sqrt(2))
    want = math.log(math.exp(2 * float(s)) + 2 * math.exp(float(s)))
    assert abs(l[0, 0, 0] - want) < 1e-12


# ---------------------------------------------------------------- closed forms
def pin_closed_forms(att):
    # N = 1: O = v_0 and lse = s_00 (causal and not)
    q, k, v = rand((2, 1, 3, 16), 11), rand((2, 1, 3, 16), 12), rand((2, 1, 3, 16), 13)
    for causal in (False, True):
        o, l = _full(att, q, k, v, 0.25, causal)
        for b in range(2):
            for h in range(3):
                assert np.allclose(o[b, h, 0], v[b, 0, h], atol=1e-15, rtol=0)
                s00 = float(np.float32(0.25)) * float(np.dot(q[b, 0, h].astype(np.float64), k[b, 0, h].astype(np.float64)))
                assert abs(l[b, h, 0] - s00) < 1e-12
    # causal row 0 of a longer sequence: O = v_0, lse = s_00
    N = 9
    q, k, v = rand((1, N, 2, 8), 21), rand((1, N, 2, 8), 22), rand((1, N, 2, 8), 23)
    o, l = _full(att, q, k, v, 0.5, True)
    for h in range(2):
        assert np.allclose(o[0, h, 0], v[0, 0, h], atol=1e-15, rtol=0)
    # q = 0: every visible key has the same score, O_i = mean of visible v,
    # lse_i = ln |J| (causal: ln(i + 1))
    q0 = np.zeros((1, N, 2, 8), dtype=np.float32)
    for causal in (False, True):
        o, l = _full(att, q0, k, v, 0.5, causal)
        for h in range(2):
            for i in range(N):
                n = i + 1 if causal else N
                mean = v[0, :n, h].astype(np.float64).mean(axis=0)
                assert np.allclose(o[0, h, i], mean, atol=1e-14, rtol=0), "q=0 must average the visible v"
                assert abs(l[0, h, i] - math.log(n)) < 1e-14, "q=0 lse must be ln|J|"
    # scale = 0 is the same as q = 0
    o, l = _full(att, q, k, v, 0.0, True)
    for i in range(N):
        assert np.allclose(o[0, 1, i], v[0, :i + 1, 1].astype(np.float64).mean(axis=0), atol=1e-14, rtol=0)
    # one dominant key: key 5 aligned with every query, huge scale -> O -> v_5
    d = 8
    qd = np.zeros((1, N, 1, d), dtype=np.float32)
    qd[..., 0] = 1.0
    kd = np.zeros((1, N, 1, d), dtype=np.float32)
    kd[0, 5, 0, 0] = 1.0
    vd = rand((1, N, 1, d), 31)
    o, l = _full(att, qd, kd, vd, 200.0, False)
    assert np.allclose(o[0, 0], np.broadcast_to(vd[0, 5, 0], (N, d)), atol=1e-12)
    assert np.allclose(l[0, 0], 200.0, atol=1e-12)


# ------------------------------------------------------------------ invariants
def pin_invariants(att):
    B, N, Hq, Hkv, d = 2, 37, 4, 2, 16
    q, k = rand((B, N, Hq, d), 41, 2.0), rand((B, N, Hkv, d), 42)
    v = rand((B, N, Hkv, d), 43)
    for causal in (False, True):
        # rows of P sum to one: a column of ones in V comes out as ones
        v1 = v.copy()
        v1[..., 3] = 1.0
        o, l = _full(att, q, k, v1, 0.3, causal)
        assert np.max(np.abs(o[..., 3] - 1.0)) < 1e-14, "rows of P must sum to one"
        # every output coordinate lies within [min, max] of the visible v
        g = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                for i in range(N):
                    vis = v1[b, :(i + 1 if causal else N), h // g].astype(np.float64)
                    assert np.all(o[b, h, i] >= vis.min(axis=0) - 1e-14)
                    assert np.all(o[b, h, i] <= vis.max(axis=0) + 1e-14)
        # shift invariance: adding c_i to every score of row i leaves O and
        # moves lse by c_i.  Realised by an extra coordinate: k[..., -1] = 1,
        # q[..., -1] = c_i / scale (exact in float32 here: scale = 0.5).
        qa = np.concatenate([q, np.zeros((B, N, Hq, 1), np.float32)], axis=-1)
        ka = np.concatenate([k, np.ones((B, N, Hkv, 1), np.float32)], axis=-1)
        va = np.concatenate([v, np.zeros((B, N, Hkv, 1), np.float32)], axis=-1)
        o0, l0 = _full(att, qa, ka, va, 0.5, causal)
        c = np.random.default_rng(44).integers(-20, 21, size=(B, N, Hq)).astype(np.float32) * 0.75
        qs = qa.copy()
        qs[..., -1] = c / np.float32(0.5)
        o1, l1 = _full(att, qs, ka, va, 0.5, causal)
        assert np.max(np.abs(o1 - o0)) < 1e-12, "O must not move when a row is shifted"
        assert np.max(np.abs((l1 - l0) - c.transpose(0, 2, 1))) < 1e-12, "lse must move by the shift"
        # GQA by indexing == MHA with each K/V head repeated g times
        kr, vr = np.repeat(k, g, axis=2), np.repeat(v, g, axis=2)
        og, lg = _full(att, q, k, v, 0.3, causal)
        om, lm = _full(att, q, kr, vr, 0.3, causal)
        assert np.max(np.abs(og - om)) == 0 and np.max(np.abs(lg - lm)) == 0, "GQA must equal repeated-KV MHA"
    # causal row i == non-causal attention over the prefix 0..i
    o, l = _full(att, q, k, v, 0.3, True)
    for i in (0, 1, 7, 20, N - 1):
        op, lp = _full(att, np.ascontiguousarray(q[:, :i + 1]), np.ascontiguousarray(k[:, :i + 1]),
                       np.ascontiguousarray(v[:, :i + 1]), 0.3, False)
        assert np.max(np.abs(o[:, :, i] - op[:, :, i])) < 1e-14
        assert np.max(np.abs(l[:, :, i] - lp[:, :, i])) < 1e-13


# ------------------------------------------------------------ library routine
def pin_torch_sdpa(att):
    """torch's scaled_dot_product_attention on the CPU in float64.

    A library routine that computes softmax(scale Q K^T + mask) V; GQA is
    compared through explicitly repeated K/V heads.
    """
    import torch
    import torch.nn.functional as F
    for seed, (B, Hq, Hkv, N, d), causal in [
        (51, (2, 4, 4, 70, 32), False), (52, (1, 8, 2, 129, 64), True), (53, (1, 2, 1, 33, 128), True),
    ]:
        q, k, v = rand((B, N, Hq, d), seed), rand((B, N, Hkv, d), seed + 1), rand((B, N, Hkv, d), seed + 2)
        sc = 1 / math.sqrt(d)
        o, l = _full(att, q, k, v, sc, causal)
        g = Hq // Hkv
        tq = torch.from_numpy(q).double().permute(0, 2, 1, 3)
        tk = torch.from_numpy(np.repeat(k, g, axis=2)).double().permute(0, 2, 1, 3)
        tv = torch.from_numpy(np.repeat(v, g, axis=2)).double().permute(0, 2, 1, 3)
        ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=float(np.float32(sc)))
        assert np.max(np.abs(o - ref.numpy())) < 1e-12, "O differs from torch sdpa (fp64)"
        s = torch.matmul(tq, tk.transpose(-1, -2)) * float(np.float32(sc))
        if causal:
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        assert np.max(np.abs(l - torch.logsumexp(s, dim=-1).numpy())) < 1e-12, "LSE differs from torch logsumexp"
    # unequal lengths (decode-like and chunked-prefill-like), the bottom-right
    # causal mask given to sdpa explicitly as a boolean keep-matrix
    for seed, (B, Hq, Hkv, Nq, Nk, d), causal in [
        (54, (2, 8, 2, 1, 300, 128), True), (55, (1, 4, 1, 40, 257, 64), True),
        (56, (1, 2, 2, 70, 33, 32), False),
    ]:
        q, k, v = rand((B, Nq, Hq, d), seed), rand((B, Nk, Hkv, d), seed + 1), rand((B, Nk, Hkv, d), seed + 2)
        sc = 1 / math.sqrt(d)
        o, l = _full(att, q, k, v, sc, causal)
        g = Hq // Hkv
        tq = torch.from_numpy(q).double().permute(0, 2, 1, 3)
        tk = torch.from_numpy(np.repeat(k, g, axis=2)).double().permute(0, 2, 1, 3)
        tv = torch.from_numpy(np.repeat(v, g, axis=2)).double().permute(0, 2, 1, 3)
        keep = torch.ones(Nq, Nk, dtype=torch.bool)
        if causal:
            keep = torch.ones(Nq, Nk, dtype=torch.bool).tril(Nk - Nq)
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=keep, scale=float(np.float32(sc)))
        assert np.max(np.abs(o - ref.numpy())) < 1e-12, "O differs from torch sdpa (fp64, unequal lengths)"
        s = (torch.matmul(tq, tk.transpose(-1, -2)) * float(np.float32(sc))).masked_fill(~keep, float("-inf"))
        assert np.max(np.abs(l - torch.logsumexp(s, dim=-1).numpy())) < 1e-12, "LSE differs (unequal lengths)"


ALL_PINS = [pin_worked_example, pin_closed_forms, pin_invariants, pin_brute_force, pin_torch_sdpa,
            pin_bottom_right_masks]
