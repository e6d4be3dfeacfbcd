"""Seeded random configurations against the fp64 oracle: batch, head
grouping, query and key lengths (equal or not), head dimension, dtype,
causal or not, and the number of key ranges, drawn together so that the
dense, split, decoding and d = 256 paths meet shapes the hand-picked cases
do not; and a sweep of the backward the same way."""
import math
import random

import pytest
import torch

import exact_attention_93_amd as fa
from tests.bwd_util import compare_bwd, gpu_fwd_bwd
from tests.gpu_util import compare, rand_inputs, say

pytestmark = pytest.mark.gpu


def draw(i):
    r = random.Random(7000 + i)
    dtype = r.choice(["bf16", "bf16", "fp32"])
    d = r.choice([64, 128, 256] if dtype == "bf16" else [64, 128])
    Hkv = r.randint(1, 3)
    Hq = Hkv * r.choice([1, 2, 3, 4, 8])
    B = r.randint(1, 3)
    Nq = r.choice([1, 2, r.randint(1, 80), r.randint(1, 700)])
    Nk = Nq if r.random() < 0.4 else r.choice([r.randint(1, 80), r.randint(1, 1500)])
    splits = 1 if Nk == Nq and r.random() < 0.5 else r.choice([0, 1, 2, r.randint(2, 9)])
    causal = r.random() < 0.6
    return dict(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype=dtype, causal=causal, splits=splits)


@pytest.mark.parametrize("i", range(160))
def test_random_configuration(i):
    c = draw(i)
    say(f"case random {i}: {c}")
    q, k, v = rand_inputs(c["B"], c["Nq"], c["Hq"], c["Hkv"], c["d"], c["dtype"], seed=8000 + i, Nk=c["Nk"])
    scale = 1 / math.sqrt(c["d"])
    o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=c["causal"], scale=scale, num_splits=c["splits"])
    torch.cuda.synchronize()
    compare(q, k, v, c["causal"], scale, o.cpu(), lse.cpu(), label=f"random {i}", num_splits=c["splits"])


def draw_bwd(i):
    r = random.Random(9000 + i)
    Hkv = r.randint(1, 2)
    Nq = r.choice([1, r.randint(1, 100), r.randint(1, 400)])
    Nk = Nq if r.random() < 0.5 else r.choice([r.randint(1, 100), r.randint(1, 600)])
    return dict(B=r.randint(1, 2), Hq=Hkv * r.choice([1, 2, 4]), Hkv=Hkv, Nq=Nq, Nk=Nk, d=r.choice([64, 128]),
                causal=r.random() < 0.6)


@pytest.mark.parametrize("i", range(32))
def test_random_backward(i):
    c = draw_bwd(i)
    say(f"case random bwd {i}: {c}")
    q, k, v = rand_inputs(c["B"], c["Nq"], c["Hq"], c["Hkv"], c["d"], "bf16", seed=9500 + i, Nk=c["Nk"])
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(9600 + i)).to(torch.bfloat16)
    scale = 1 / math.sqrt(c["d"])
    grads = gpu_fwd_bwd(q, k, v, do, c["causal"], scale)
    compare_bwd(q, k, v, do, c["causal"], scale, *grads, label=f"random bwd {i}")
