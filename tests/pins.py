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


# ==================================================================== backward
# Pins for oracle.attention_bwd.  Each takes (att, bwd) callables with the
# signatures of oracle.attention and oracle.attention_bwd.

def _full_bwd(bwd, q, k, v, do, scale, causal):
    """dq [B, Hq, Nq, d], dk and dv [B, Hkv, Nk, d] from the grouped output."""
    dq, dk, dv = bwd(q, k, v, do, scale, causal)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    return dq.reshape(B, Hq, Nq, d), dk.reshape(B, Hkv, Nk, d), dv.reshape(B, Hkv, Nk, d)


def pin_bwd_finite_differences(att, bwd):
    """Central differences of L = sum(dO * O) through the forward oracle.

    Each input coordinate is moved by +-h and +-2h (h = 2^-9, exact in
    float32 for these magnitudes) and the two central differences are
    combined by Richardson extrapolation (error O(h^4)).  Checks that the
    gradients are those of the (separately pinned) forward definition,
    including grouped heads, the bottom-right causal mask and rows that see
    no key."""
    h = 2.0 ** -9
    for seed, (B, Hq, Hkv, Nq, Nk, d), causal in [
        (71, (1, 2, 1, 4, 6, 3), True), (72, (1, 2, 2, 5, 3, 2), True), (73, (2, 2, 1, 3, 3, 2), False),
    ]:
        # inputs on a 2^-20 grid, so that x +- h and x +- 2h are exact in float32
        q, k, v = (np.round(rand(s_, seed + o_) * 2.0 ** 20) / 2.0 ** 20 for s_, o_ in
                   (((B, Nq, Hq, d), 0), ((B, Nk, Hkv, d), 1), ((B, Nk, Hkv, d), 2)))
        q, k, v = q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)
        do = rand((B, Nq, Hq, d), seed + 3)
        sc = 0.8
        dq, dk, dv = _full_bwd(bwd, q, k, v, do, sc, causal)

        def loss(qq, kk, vv):
            o, _ = att(qq, kk, vv, sc, causal)
            return float(np.sum(o * do.transpose(0, 2, 1, 3).reshape(-1, d).astype(np.float64)))

        for name, x, grad in (("q", q, dq.transpose(0, 2, 1, 3)), ("k", k, dk.transpose(0, 2, 1, 3)),
                              ("v", v, dv.transpose(0, 2, 1, 3))):
            num = np.zeros(x.shape)
            for idx in np.ndindex(*x.shape):
                vals = []
                for step in (h, 2 * h):
                    xp, xm = x.copy(), x.copy()
                    xp[idx] += np.float32(step)
                    xm[idx] -= np.float32(step)
                    args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                    args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                    vals.append((loss(*args_p) - loss(*args_m)) / (2 * step))
                num[idx] = (4 * vals[0] - vals[1]) / 3
            err = np.max(np.abs(num - grad))
            assert err < 1e-9, f"d{name} differs from finite differences of the forward by {err}"


def pin_bwd_torch_autograd(att, bwd):
    """fp64 torch autograd through scaled_dot_product_attention (a library
    routine), grouped heads by repeating K/V (autograd sums the copies), the
    bottom-right causal mask given explicitly."""
    import torch
    import torch.nn.functional as F
    for seed, (B, Hq, Hkv, Nq, Nk, d), causal in [
        (81, (2, 4, 2, 33, 33, 16), True), (82, (1, 4, 1, 7, 40, 32), True), (83, (1, 2, 2, 20, 9, 8), False),
        (84, (1, 2, 1, 1, 65, 64), True),
    ]:
        q, k, v = rand((B, Nq, Hq, d), seed), rand((B, Nk, Hkv, d), seed + 1), rand((B, Nk, Hkv, d), seed + 2)
        do = rand((B, Nq, Hq, d), seed + 3)
        sc = float(np.float32(1 / math.sqrt(d)))
        dq, dk, dv = _full_bwd(bwd, q, k, v, do, sc, causal)
        g = Hq // Hkv
        tq = torch.from_numpy(q).double().permute(0, 2, 1, 3).requires_grad_()
        tk = torch.from_numpy(k).double().permute(0, 2, 1, 3).requires_grad_()
        tv = torch.from_numpy(v).double().permute(0, 2, 1, 3).requires_grad_()
        keep = torch.ones(Nq, Nk, dtype=torch.bool).tril(Nk - Nq) if causal else None
        out = F.scaled_dot_product_attention(tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1),
                                             attn_mask=keep, scale=sc)
        out.backward(torch.from_numpy(do).double().permute(0, 2, 1, 3))
        for name, mine, ref in (("dq", dq, tq.grad), ("dk", dk, tk.grad), ("dv", dv, tv.grad)):
            err = float(np.max(np.abs(mine - ref.numpy())))
            assert err < 1e-12, f"{name} differs from torch autograd by {err}"


def pin_bwd_closed_forms(att, bwd):
    # a single key: P = 1 for every row, so dq = dk = 0 and dv = sum of dO
    # over the rows and the query heads of the group
    q, k, v = rand((2, 9, 4, 8), 91), rand((2, 1, 2, 8), 92), rand((2, 1, 2, 8), 93)
    do = rand((2, 9, 4, 8), 94)
    for causal in (False, True):
        dq, dk, dv = _full_bwd(bwd, q, k, v, do, 0.7, causal)
        nvis_rows = 1 if causal else 9        # causal, Nk = 1: only the last query row sees the key
        assert np.max(np.abs(dq)) < 1e-15 and np.max(np.abs(dk)) < 1e-15, "one key: dq and dk must vanish"
        for b in range(2):
            for hk in range(2):
                want = do[b, 9 - nvis_rows:, 2 * hk:2 * hk + 2].astype(np.float64).sum(axis=(0, 1))
                assert np.allclose(dv[b, hk, 0], want, atol=1e-13, rtol=0), "one key: dv = sum of dO"
    # scale 0: uniform weights over the visible keys; dq = dk = 0 and
    # dv_j = sum over the rows i that see j of dO_i / |visible keys of i|
    N = 6
    q, k, v, do = rand((1, N, 1, 4), 95), rand((1, N, 1, 4), 96), rand((1, N, 1, 4), 97), rand((1, N, 1, 4), 98)
    dq, dk, dv = _full_bwd(bwd, q, k, v, do, 0.0, True)
    assert np.max(np.abs(dq)) == 0 and np.max(np.abs(dk)) == 0
    for j in range(N):
        want = sum(do[0, i, 0].astype(np.float64) / (i + 1) for i in range(j, N))
        assert np.allclose(dv[0, 0, j], want, atol=1e-14, rtol=0), "scale 0: dv"
    # invariants on random inputs: sum_j dk_j = 0 (a common shift of every
    # key moves each row's scores by a constant), sum_j dv_j = sum of dO over
    # rows that see a key, and linearity in dO
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 11, 8, 8
    q, k, v = rand((B, Nq, Hq, d), 101, 2.0), rand((B, Nk, Hkv, d), 102), rand((B, Nk, Hkv, d), 103)
    do1, do2 = rand((B, Nq, Hq, d), 104), rand((B, Nq, Hq, d), 105)
    for causal in (False, True):
        g1 = _full_bwd(bwd, q, k, v, do1, 0.5, causal)
        g2 = _full_bwd(bwd, q, k, v, do2, 0.5, causal)
        g12 = _full_bwd(bwd, q, k, v, (do1.astype(np.float64) + do2).astype(np.float32), 0.5, causal)
        assert np.max(np.abs(g1[1].sum(axis=2))) < 1e-13, "sum over keys of dk must vanish"
        first = max(0, Nq - Nk) if causal else 0            # rows before this see no key
        for hk in range(Hkv):
            want = do1[0, first:, 2 * hk:2 * hk + 2].astype(np.float64).sum(axis=(0, 1))
            assert np.allclose(g1[2][0, hk].sum(axis=0), want, atol=1e-13, rtol=0), "sum over keys of dv"
        s12 = (do1.astype(np.float64) + do2).astype(np.float32)
        if np.array_equal(s12.astype(np.float64), do1.astype(np.float64) + do2):   # exact sum only
            for a, b_, c in zip(g1, g2, g12):
                assert np.max(np.abs(a + b_ - c)) < 1e-12, "gradients must be linear in dO"


BWD_PINS = [pin_bwd_closed_forms, pin_bwd_torch_autograd, pin_bwd_finite_differences]


# ---------------------------------------------------------- block-sparse mask
def expand_block_mask(mask, Nq, Nk, bq, bk):
    """[H, nqb, nkb] block mask -> [H, Nq, Nk] boolean keep-matrix."""
    m = np.asarray(mask, dtype=bool)
    return np.repeat(np.repeat(m, bq, axis=1), bk, axis=2)[:, :Nq, :Nk]


def pin_block_mask(att):
    """The block-sparse variant (first page, section 0x04): keys of skipped
    blocks take no part in a row's softmax."""
    rng = np.random.default_rng(111)
    # all-ones mask: identical to the dense result (same arithmetic, same order)
    B, Hq, Hkv, N, d, bq, bk = 1, 4, 2, 37, 8, 8, 4
    q, k, v = rand((B, N, Hq, d), 112), rand((B, N, Hkv, d), 113), rand((B, N, Hkv, d), 114)
    ones = np.ones((Hq, -(-N // bq), -(-N // bk)), np.uint8)
    for causal in (False, True):
        a = att(q, k, v, 0.4, causal)
        b = att(q, k, v, 0.4, causal, block_mask=ones, block=(bq, bk))
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), "all-ones mask must equal dense"
    # one kept key block per query block: equals dense attention over that
    # slice of K/V; an all-zero mask row gives O = 0 and lse = -inf
    nqb, nkb = -(-N // bq), -(-N // bk)
    keep = rng.integers(0, nkb, size=(Hq, nqb))
    m1 = np.zeros((Hq, nqb, nkb), np.uint8)
    for h in range(Hq):
        for a_ in range(nqb):
            m1[h, a_, keep[h, a_]] = 1
    m1[1, 2, :] = 0
    o, l = att(q, k, v, 0.4, False, block_mask=m1, block=(bq, bk))
    o = o.reshape(B, Hq, N, d)
    l = l.reshape(B, Hq, N)
    for h in range(Hq):
        for i in range(N):
            if h == 1 and i // bq == 2:
                assert np.all(o[0, h, i] == 0) and l[0, h, i] == -math.inf, "empty mask row must give zeros"
                continue
            c = keep[h, i // bq]
            sl = slice(c * bk, min(N, (c + 1) * bk))
            os_, ls_ = att(np.ascontiguousarray(q[:, i:i + 1]), np.ascontiguousarray(k[:, sl]),
                           np.ascontiguousarray(v[:, sl]), 0.4, False)
            os_ = os_.reshape(B, Hq, 1, d)
            assert np.array_equal(o[0, h, i], os_[0, h, 0]), "one kept block must equal attention on that slice"
            assert l[0, h, i] == ls_.reshape(B, Hq)[0, h], "lse over one kept block"
    # random masks, causal and not: decimal brute force (tiny) and fp64 sdpa
    import torch
    import torch.nn.functional as F
    for seed, (B, Hq, Hkv, N, d, bq, bk), causal in [
        (115, (1, 2, 1, 9, 3, 2, 3), True), (116, (2, 2, 2, 7, 2, 4, 2), False),
    ]:
        q, k, v = rand((B, N, Hq, d), seed), rand((B, N, Hkv, d), seed + 1), rand((B, N, Hkv, d), seed + 2)
        m = (np.random.default_rng(seed).random((Hq, -(-N // bq), -(-N // bk))) < 0.6).astype(np.uint8)
        o, l = att(q, k, v, 0.7, causal, block_mask=m, block=(bq, bk))
        o, l = o.reshape(B, Hq, N, d), l.reshape(B, Hq, N)
        keepm = expand_block_mask(m, N, N, bq, bk)
        if causal:
            keepm = keepm & np.tril(np.ones((N, N), bool))[None]
        g = Hq // Hkv
        getcontext().prec = 40
        for b in range(B):
            for h in range(Hq):
                for i in range(N):
                    J = [j for j in range(N) if keepm[h, i, j]]
                    if not J:
                        assert np.all(o[b, h, i] == 0) and l[b, h, i] == -math.inf
                        continue
                    w = [(Decimal(float(np.float32(0.7))) * sum(Decimal(float(q[b, i, h, x])) * Decimal(float(k[b, j, h // g, x]))
                                                               for x in range(d))).exp() for j in J]
                    tot = sum(w)
                    for x in range(d):
                        ref = float(sum(wj * Decimal(float(v[b, j, h // g, x])) for wj, j in zip(w, J)) / tot)
                        assert abs(o[b, h, i, x] - ref) < 1e-12, "masked O differs from the decimal brute force"
                    assert abs(l[b, h, i] - float(tot.ln())) < 1e-12
    B, Hq, Hkv, N, d, bq, bk = 1, 4, 2, 150, 32, 32, 16
    q, k, v = rand((B, N, Hq, d), 117), rand((B, N, Hkv, d), 118), rand((B, N, Hkv, d), 119)
    m = (np.random.default_rng(120).random((Hq, -(-N // bq), -(-N // bk))) < 0.5).astype(np.uint8)
    m[:, :, 0] = 1                                   # every row keeps a block
    for causal in (False, True):
        o, l = att(q, k, v, 0.25, causal, block_mask=m, block=(bq, bk))
        keepm = torch.from_numpy(expand_block_mask(m, N, N, bq, bk))
        if causal:
            keepm = keepm & torch.ones(N, N, dtype=torch.bool).tril()
        g = Hq // Hkv
        tq = torch.from_numpy(q).double().permute(0, 2, 1, 3)
        tk = torch.from_numpy(np.repeat(k, g, axis=2)).double().permute(0, 2, 1, 3)
        tv = torch.from_numpy(np.repeat(v, g, axis=2)).double().permute(0, 2, 1, 3)
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=keepm[None], scale=float(np.float32(0.25)))
        assert np.max(np.abs(o.reshape(B, Hq, N, d) - ref.numpy())) < 1e-12, "masked O differs from sdpa"


ALL_PINS.append(pin_block_mask)
