"""The five named workloads at full size, launched exactly as the benchmark
launches them; the oracle checks every row of the fp32 case and a seeded
sample of 512 query rows per (batch, head) elsewhere.  Also the two fp32
workloads at scale (the headline shape, and a split call against 64K keys),
at the fp32 bounds verbatim."""
import pytest
import torch

import exact_attention_93_amd as fa
from exact_attention_93_amd import workloads as W
from tests.gpu_util import compare, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", W.ORDER)
def test_workload(name):
    w = W.WORKLOADS[name]
    say(f"case workload {name}")
    q, k, v = W.gen_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = fa.fwd(qd, kd, vd, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    rows = None if w.dtype == "fp32" else W.sample_rows(w)
    compare(q, k, v, w.causal, w.scale, o, lse, rows=rows, label=name, exact_bounds=True, num_splits=1)


@pytest.mark.parametrize("name", list(W.FP32_WORKLOADS))
def test_fp32_workload(name):
    w = W.FP32_WORKLOADS[name]
    say(f"case fp32 workload {name} splits={fa.fa_splitkv_num_splits(w.B, w.Hq, w.Hkv, w.N, w.Nkv, w.d, w.splits)}")
    q, k, v = W.gen_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = fa.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, num_splits=w.splits)
    torch.cuda.synchronize()
    compare(q, k, v, w.causal, w.scale, o.cpu(), lse.cpu(), rows=W.sample_rows(w), label=name, exact_bounds=True,
            num_splits=w.splits)
