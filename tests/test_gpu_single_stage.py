"""LDS stage discipline: the debug build libfa_single_stage.so keeps one LDS
stage per streamed tile (K/V in the forward kernels and the dQ kernel, Q/dO
in the dK/dV kernel) and loads each tile only after a barrier has ended
every read of it, so no load overlaps a read.  The double-buffered libfa.so
must give the same outputs bit for bit; a missing wait or barrier in its
schedule (a read of a stage still being filled, or a load into a stage still
being read) shows up as a difference.  Covers every entry point that runs
these kernels: the bf16 forward (whole-sequence, split key ranges, block
mask; d = 64, 128, 256), the fp32 forward (whole-sequence and split), the
fp8 forward in both scale forms, and the backward."""
import contextlib

import pytest
import torch

import exact_attention_93_amd as fa
from exact_attention_93_amd import workloads as W
from tests.fp8_util import fp8_inputs
from tests.gpu_util import rand_inputs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    main = fa.load_library()
    dbg = fa.load_library(fa.SINGLE_STAGE_LIB_PATH)
    assert main.fa_lds_stages() == 2 and dbg.fa_lds_stages() == 1
    assert main.fa_version() == dbg.fa_version()
    return main, dbg


@contextlib.contextmanager
def using(lib, main):
    fa._lib = lib
    try:
        yield
    finally:
        fa._lib = main


def run_both(libs, call):
    """call() under each library; returns the two tuples of host tensors."""
    main, dbg = libs
    outs = []
    for lib in (main, dbg):
        with using(lib, main):
            res = call()
            torch.cuda.synchronize()
            outs.append(tuple(t.cpu() for t in res))
    return outs


def _bits(t):
    return t.view({2: torch.int16, 4: torch.int32}[t.element_size()])


def assert_bitwise(outs, label, names=("o", "lse")):
    diffs = []
    for name, a, b in zip(names, *outs):
        if not torch.equal(_bits(a), _bits(b)):
            diffs.append(f"{int((_bits(a) != _bits(b)).sum())} of {name}")
    if diffs:
        pytest.fail(f"{label}: double-buffered and single-stage builds differ in " + ", ".join(diffs))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 300, 1000])
def test_dense(libs, N, causal, d):
    say(f"case single-stage dense N={N} causal={causal} d={d}")
    q, k, v = rand_inputs(2, N, 8, 2, d, "bf16", seed=4000 + N + d + causal)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    assert_bitwise(run_both(libs, lambda: fa.fwd(qd, kd, vd, causal=causal)), f"dense N={N} d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_scores_past_the_reference_maximum(libs, d):
    """q scaled by 6: later tiles' sums pass the bound and are redone with
    their own maximum, a path the double-buffered schedule must also keep
    ordered."""
    say(f"case single-stage growing scores d={d}")
    q, k, v = rand_inputs(1, 1000, 4, 4, d, "bf16", seed=4100 + d, q_std=6.0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    assert_bitwise(run_both(libs, lambda: fa.fwd(qd, kd, vd, causal=True)), f"growing d={d}")


@pytest.mark.parametrize("splits", [1, 4])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(3, 1000), (129, 1000), (1000, 129), (257, 256)], ids=lambda s: f"q{s[0]}k{s[1]}")
def test_split_key_ranges(libs, shape, causal, splits):
    Nq, Nk = shape
    say(f"case single-stage split Nq={Nq} Nk={Nk} causal={causal} splits={splits}")
    q, k, v = rand_inputs(2, Nq, 8, 2, 128, "bf16", seed=4200 + Nq + Nk, Nk=Nk)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    assert_bitwise(run_both(libs, lambda: fa.fwd(qd, kd, vd, causal=causal, num_splits=splits)),
                   f"split {shape} splits={splits}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1), (300, 300), (1000, 1000), (129, 1000), (1000, 129)],
                         ids=lambda s: f"q{s[0]}k{s[1]}")
def test_fp32(libs, shape, causal, d):
    Nq, Nk = shape
    say(f"case single-stage fp32 Nq={Nq} Nk={Nk} causal={causal} d={d}")
    q, k, v = rand_inputs(2, Nq, 4, 2, d, "fp32", seed=4400 + Nq + Nk + d, Nk=Nk)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    assert_bitwise(run_both(libs, lambda: fa.fwd(qd, kd, vd, causal=causal)), f"fp32 {shape} d={d}")
    if Nk >= 256:
        assert_bitwise(run_both(libs, lambda: fa.fwd(qd, kd, vd, causal=causal, num_splits=3)),
                       f"fp32 split {shape} d={d}")


@pytest.mark.parametrize("name", list(W.FP32_WORKLOADS))
def test_fp32_workloads(libs, name):
    w = W.FP32_WORKLOADS[name]
    say(f"case single-stage workload {name}")
    q, k, v = (t.cuda() for t in W.gen_inputs(w))
    assert_bitwise(run_both(libs, lambda: fa.fwd(q, k, v, causal=w.causal, scale=w.scale, num_splits=w.splits)),
                   name)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [300, 1000])
def test_block_mask(libs, N, causal, d):
    say(f"case single-stage block mask N={N} causal={causal} d={d}")
    q, k, v = rand_inputs(1, N, 4, 2, d, "bf16", seed=4300 + N + d)
    mask = W.random_block_mask(4, N, 0.5, seed=4400 + N).cuda()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    assert_bitwise(run_both(libs, lambda: fa.fwd_blocksparse(qd, kd, vd, mask, causal=causal)),
                   f"block mask N={N} d={d}")


@pytest.mark.parametrize("name", ["causal_bf16_B2_H32_N4096_d128", "mha_bf16_B4_H16_N2048_d64",
                                  "causal_bf16_B2_H16_N4096_d256", "butterfly_bf16_B1_H32_N16384_d128"])
def test_full_size_workloads(libs, name):
    w = W.ALL_WORKLOADS[name]
    say(f"case single-stage workload {name}")
    q, k, v = (t.cuda() for t in W.gen_inputs(w))
    if getattr(w, "mask", None):
        mask = w.block_mask().cuda()
        call = lambda: fa.fwd_blocksparse(q, k, v, mask, causal=w.causal, scale=w.scale)
    else:
        call = lambda: fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    assert_bitwise(run_both(libs, call), name)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 300, 1000])
def test_fp8_head_scales(libs, N, causal):
    say(f"case single-stage fp8 N={N} causal={causal}")
    t = [a.cuda() for a in fp8_inputs(2, N, 8, 2, 128, seed=4500 + N)]
    assert_bitwise(run_both(libs, lambda: fa.fwd_fp8(*t, causal=causal)), f"fp8 N={N}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 300, 1000])
def test_fp8_block_scales(libs, N, causal):
    say(f"case single-stage fp8 block N={N} causal={causal}")
    (qc, qe), (kc, ke), (vc, ve) = (W.random_block_codes(2, N, h, 128, seed=4600 + N + s)
                                    for h, s in ((8, 0), (2, 100), (2, 200)))
    t = [a.cuda() for a in (qc, kc, vc, qe, ke, ve)]
    assert_bitwise(run_both(libs, lambda: fa.fwd_fp8_block(*t, causal=causal, scale=0.0884)), f"fp8 block N={N}")


def test_fp8_headline_shape(libs):
    """B=2, H=32, N=4096, d=128, causal, in both scale forms."""
    say("case single-stage fp8 B=2 H=32 N=4096")
    t = [a.cuda() for a in fp8_inputs(2, 4096, 32, 32, 128, seed=4700)]
    assert_bitwise(run_both(libs, lambda: fa.fwd_fp8(*t, causal=True)), "fp8 headline shape")
    (qc, qe), (kc, ke), (vc, ve) = (W.random_block_codes(2, 4096, 32, 128, seed=4800 + s) for s in (0, 1, 2))
    t = [a.cuda() for a in (qc, kc, vc, qe, ke, ve)]
    assert_bitwise(run_both(libs, lambda: fa.fwd_fp8_block(*t, causal=True, scale=0.0884)), "fp8 block headline shape")


def _fwd_bwd(q, k, v, do, causal):
    o, lse = fa.fwd(q, k, v, causal=causal)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal)
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1), (65, 65), (300, 300), (1000, 1000), (129, 1000), (1000, 129)],
                         ids=lambda s: f"q{s[0]}k{s[1]}")
def test_backward(libs, shape, causal, d):
    Nq, Nk = shape
    say(f"case single-stage bwd Nq={Nq} Nk={Nk} causal={causal} d={d}")
    q, k, v = rand_inputs(2, Nq, 8, 2, d, "bf16", seed=4900 + Nq + Nk + d, Nk=Nk)
    g = torch.Generator().manual_seed(4901 + Nq)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    t = [a.cuda() for a in (q, k, v, do)]
    assert_bitwise(run_both(libs, lambda: _fwd_bwd(*t, causal)), f"bwd {shape} d={d}",
                   names=("o", "lse", "dq", "dk", "dv"))


def test_backward_headline_shape(libs):
    say("case single-stage bwd causal_bf16_B2_H32_N4096_d128")
    w = W.ALL_WORKLOADS["causal_bf16_B2_H32_N4096_d128"]
    q, k, v = (a.cuda() for a in W.gen_inputs(w))
    g = torch.Generator().manual_seed(5000)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16).cuda()
    assert_bitwise(run_both(libs, lambda: _fwd_bwd(q, k, v, do, True)), "bwd headline shape",
                   names=("o", "lse", "dq", "dk", "dv"))
