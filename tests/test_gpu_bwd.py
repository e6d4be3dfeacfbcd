"""Backward (fa_bwd) against the fp64 oracle: dq, dk, dv on small shapes
(several tiles, ragged tails, grouped heads, both head dims, causal and
not, unequal lengths, rows without keys, scale signs) and on the causal
B=2 H=32 N=4096 d=128 workload (a sample of K/V head groups)."""
import math

import pytest
import torch

import exact_attention_93_amd as fa
from exact_attention_93_amd import workloads as W
from tests.bwd_util import compare_bwd, gpu_fwd_bwd
from tests.gpu_util import rand_inputs, say

pytestmark = pytest.mark.gpu


def grad_inputs(B, Nq, Hq, Hkv, d, seed, Nk=None):
    q, k, v = rand_inputs(B, Nq, Hq, Hkv, d, "bf16", seed, Nk=Nk)
    g = torch.Generator().manual_seed(seed + 7)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    return q, k, v, do


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 129, 300])
def test_bwd_small(N, causal, d):
    say(f"case bwd N={N} causal={causal} d={d}")
    q, k, v, do = grad_inputs(2, N, 4, 2, d, seed=N + d + causal)
    grads = gpu_fwd_bwd(q, k, v, do, causal, 1 / math.sqrt(d))
    compare_bwd(q, k, v, do, causal, 1 / math.sqrt(d), *grads, label=f"N={N}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 300), (40, 257), (300, 17), (129, 1000), (1000, 129)],
                         ids=lambda s: f"q{s[0]}k{s[1]}")
def test_bwd_unequal(shape, causal):
    Nq, Nk = shape
    say(f"case bwd unequal Nq={Nq} Nk={Nk} causal={causal}")
    q, k, v, do = grad_inputs(1, Nq, 8, 2, 128, seed=Nq * 3 + Nk, Nk=Nk)
    grads = gpu_fwd_bwd(q, k, v, do, causal, 0.0884)
    compare_bwd(q, k, v, do, causal, 0.0884, *grads, label=f"Nq={Nq} Nk={Nk}")


@pytest.mark.parametrize("heads", [(1, 1), (8, 1), (6, 3)])
def test_bwd_heads(heads):
    Hq, Hkv = heads
    say(f"case bwd heads={heads}")
    q, k, v, do = grad_inputs(2, 200, Hq, Hkv, 64, seed=Hq * 10 + Hkv)
    for causal in (False, True):
        grads = gpu_fwd_bwd(q, k, v, do, causal, 0.125)
        compare_bwd(q, k, v, do, causal, 0.125, *grads, label=f"heads={heads} causal={causal}")


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.3])
def test_bwd_scales(scale):
    say(f"case bwd scale={scale}")
    q, k, v, do = grad_inputs(1, 150, 4, 4, 64, seed=11)
    for causal in (False, True):
        grads = gpu_fwd_bwd(q, k, v, do, causal, scale)
        if scale == 0.0:
            assert torch.all(grads[0] == 0) and torch.all(grads[1] == 0), "scale 0: dq and dk vanish"
        compare_bwd(q, k, v, do, causal, scale, *grads, label=f"scale={scale} causal={causal}")


def test_bwd_deterministic():
    q, k, v, do = grad_inputs(1, 333, 8, 2, 128, seed=5)
    a = gpu_fwd_bwd(q, k, v, do, True, 0.0884)
    b = gpu_fwd_bwd(q, k, v, do, True, 0.0884)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_bwd_headline_workload_sampled():
    """The causal B=2 H=32 N=4096 d=128 workload, launched as the benchmark
    launches it; four whole head groups are checked (every dq, dk, dv element
    of those heads, whose o and lse come from the oracle)."""
    w = W.WORKLOADS[W.HEADLINE]
    q, k, v = W.gen_inputs(w)
    g = torch.Generator().manual_seed(w.seed + 50)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    groups = [(0, 0), (0, 17), (1, 5), (1, 31)]
    grads = gpu_fwd_bwd(q, k, v, do, w.causal, w.scale, groups=groups)
    compare_bwd(q, k, v, do, w.causal, w.scale, *grads, groups=groups, label=w.name)
