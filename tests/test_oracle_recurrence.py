"""The pages' recurrences (oracle/recurrence.py) against the worked example,
the induction invariant, the 3-pass definition and the fp32 error exercise."""
import math

import numpy as np
import pytest

import oracle
from oracle import recurrence as R
from tests import pins

G = pins.read_golden()
S = np.array(G["scores"])
V = np.array(G["v"])


def close(a, b, tol=6e-4):
    return abs(float(a) - float(b)) <= tol


@pytest.mark.parametrize("mode", ["fa1", "fa2"])
def test_worked_example_split_2_1(mode):
    # "FlashAttention：IO 感知的精确注意力", section 8
    t = R.blocked_row(S, V, [2, 1], mode)
    assert close(t[0]["m"], G["split_2_1.block1.m"])
    assert close(t[0]["l"], G["split_2_1.block1.l"])
    assert close(t[0]["O"][0], G["split_2_1.block1.O"])
    assert np.allclose(np.exp(S[:2] - S[:2].max()), G["split_2_1.block1.Ptilde"], atol=6e-4)
    assert close(t[1]["m"], G["split_2_1.block2.m"])
    assert close(t[1]["l"], G["split_2_1.block2.l"])
    assert close(t[1]["O"][0], G["split_2_1.block2.O"])
    if mode == "fa2":  # unnormalised accumulator after block 1 is 1*1 + 0.493*0
        assert close(t[0]["acc"][0], 1.0)


@pytest.mark.parametrize("mode", ["fa1", "fa2"])
def test_worked_example_split_1_2(mode):
    # same page, section 14 exercise 2
    t = R.blocked_row(S, V, [1, 2], mode)
    assert close(t[0]["m"], G["split_1_2.block1.m"])
    assert close(t[0]["l"], G["split_1_2.block1.l"])
    assert close(t[0]["O"][0], G["split_1_2.block1.O"])
    blk = S[1:]
    assert np.allclose(np.exp(blk - blk.max()), G["split_1_2.block2.Ptilde"])
    assert close(np.exp(blk - blk.max()).sum(), G["split_1_2.block2.ltilde"])
    assert close(t[1]["m"], G["split_1_2.block2.m"])
    assert close(t[1]["l"], G["split_1_2.block2.l"])
    assert close(t[1]["O"][0], G["split_1_2.block2.O"])


def test_worked_example_whole_row():
    for f in (R.softmax_3pass, lambda x: R.online_softmax_2pass(x)[0]):
        a = f(S)
        assert np.allclose(a, G["softmax.a"], atol=6e-5)
        assert close(a @ V, G["softmax.O4"], 1e-4)
    o, m, dp = R.attention_1pass_row(S, V[:, None])
    assert close(o[0], G["softmax.O"])


def test_induction_invariant():
    # section 14 exercise 1: after block j, l = sum_{k<=j} exp(s_k - m) and
    # O = softmax(s_{1:j}) V_{1:j}
    r = np.random.default_rng(7)
    s = r.standard_normal(40) * 3
    v = r.standard_normal((40, 5))
    sizes = [3, 1, 7, 8, 2, 19]
    for mode in ("fa1", "fa2"):
        t = R.blocked_row(s, v, sizes, mode)
        end = 0
        for blk, st in zip(sizes, t):
            end += blk
            pre = s[:end]
            assert st["m"] == pre.max()
            assert abs(st["l"] - np.exp(pre - st["m"]).sum()) < 1e-12 * st["l"]
            w = np.exp(pre - pre.max())
            assert np.allclose(st["O"], (w / w.sum()) @ v[:end], atol=1e-13, rtol=0)


@pytest.mark.parametrize("block", [1, 2, 3, 8, 32, 128])
def test_tiled_equals_three_pass(block):
    r = np.random.default_rng(block)
    s = r.standard_normal(301) * 4
    v = r.standard_normal((301, 6))
    sizes = [block] * (301 // block) + ([301 % block] if 301 % block else [])
    a = R.softmax_3pass(s)
    want = a @ v
    for mode in ("fa1", "fa2"):
        got = R.blocked_row(s, v, sizes, mode)[-1]["O"]
        assert np.max(np.abs(got - want)) < 1e-13
    o1, _, _ = R.attention_1pass_row(s, v)
    assert np.max(np.abs(o1 - want)) < 1e-13


def test_fp32_error_exercise():
    # section 14 exercise 6: online vs whole-row softmax agree to ~1e-7 in fp32
    r = np.random.default_rng(3)
    x = (r.standard_normal(512) * 3).astype(np.float32)
    v = np.eye(512, dtype=np.float32)
    a32 = R.softmax_3pass(x, np.float32)
    for B in (2, 8, 32, 128):
        sizes = [B] * (512 // B)
        o = R.blocked_row(x, v, sizes, "fa1", np.float32)[-1]["O"]
        err = np.max(np.abs(o - a32))
        assert err < 1e-6, (B, err)
    exact = R.softmax_3pass(x.astype(np.float64))
    assert np.max(np.abs(a32 - exact)) < 1e-6


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Br,Bc", [(1, 1), (4, 3), (16, 16), (5, 64)])
def test_tiled_forwards_match_c_oracle(causal, Br, Bc):
    N, d = 45, 12
    q, k, v = pins.rand((1, N, 1, d), 61, 2.0), pins.rand((1, N, 1, d), 62), pins.rand((1, N, 1, d), 63)
    sc = float(np.float32(0.3))
    o, l = oracle.attention(q, k, v, sc, causal)
    for fwd in (R.fa1_forward, R.fa2_forward):
        of, lf = fwd(q[0, :, 0], k[0, :, 0], v[0, :, 0], Br, Bc, sc, causal)
        assert np.max(np.abs(of - o)) < 1e-13
        assert np.max(np.abs(lf - l)) < 1e-13
