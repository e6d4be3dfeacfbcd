"""LDS stage discipline of the bf16 forward kernels: the debug build
libfa_single_stage.so keeps one K stage and one V stage and loads each tile
only after a barrier has ended every read of it, so it has no overlap of
loads with reads at all.  The double-buffered libfa.so must give the same
outputs bit for bit; a missing wait or barrier in its schedule (a read of a
stage still being filled, or a load into a stage still being read) shows up
as a difference.  Covers every bf16 forward entry point that runs these
kernels (whole-sequence, split key ranges, block mask) at d = 64, 128, 256."""
import contextlib

import pytest
import torch

import exact_attention_93_amd as fa
from exact_attention_93_amd import workloads as W
from tests.gpu_util import rand_inputs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    main = fa.load_library()
    dbg = fa.load_library(fa.SINGLE_STAGE_LIB_PATH)
    assert main.fa_fwd_lds_stages() == 2 and dbg.fa_fwd_lds_stages() == 1
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
    main, dbg = libs
    outs = []
    for lib in (main, dbg):
        with using(lib, main):
            o, lse = call()
            torch.cuda.synchronize()
            outs.append((o.cpu(), lse.cpu()))
    return outs


def assert_bitwise(outs, label):
    (o2, l2), (o1, l1) = outs
    same_o = torch.equal(o2.view(torch.int16), o1.view(torch.int16))
    same_l = torch.equal(l2.view(torch.int32), l1.view(torch.int32))
    if not (same_o and same_l):
        nd_o = int((o2.view(torch.int16) != o1.view(torch.int16)).sum())
        nd_l = int((l2.view(torch.int32) != l1.view(torch.int32)).sum())
        pytest.fail(f"{label}: double-buffered and single-stage builds differ in {nd_o} outputs, {nd_l} lse")


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
