"""The library's launches recorded in a HIP graph (torch.cuda.CUDAGraph):
every replay, with new inputs written in place and eager work and
synchronisations between replays, equals an eager call on the same inputs
bit for bit; one replay per case is also checked against the fp64 oracle.

The entry points allocate nothing and set no memory (no memset node can
enter a graph), so one captured call is a complete step."""
import math

import pytest
import torch

import exact_attention_93_amd as fa
from tests.gpu_util import compare, rand_inputs, say

pytestmark = pytest.mark.gpu

# (label, B, Nq, Nk, Hq, Hkv, d, causal, num_splits): the dense kernel, the
# split forward with its merge, and the decoding kernel with its merge
FWD_CASES = [
    ("dense", 1, 700, 700, 4, 2, 128, True, 1),
    ("split", 2, 129, 1000, 4, 2, 128, True, 3),
    ("decode", 1, 1, 4096, 8, 2, 128, True, 0),
    ("dense_d64", 2, 300, 300, 4, 4, 64, False, 1),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: c[0])
def test_forward_graph_replays(case):
    label, B, Nq, Nk, Hq, Hkv, d, causal, splits = case
    say(f"case graph fwd {label}")
    scale = 1 / math.sqrt(d)
    q, k, v = (t.cuda() for t in rand_inputs(B, Nq, Hq, Hkv, d, "bf16", seed=11, Nk=Nk))
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    need = fa.fa_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, splits)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    call = dict(causal=causal, scale=scale, num_splits=splits, workspace=ws)
    fa.fwd(q, k, v, out=o, lse=lse, **call)          # the first call before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.fwd(q, k, v, out=o, lse=lse, **call)
    torch.cuda.synchronize()
    for r in range(3):
        hq, hk, hv = rand_inputs(B, Nq, Hq, Hkv, d, "bf16", seed=100 + r, Nk=Nk)
        q.copy_(hq.cuda()), k.copy_(hk.cuda()), v.copy_(hv.cuda())
        torch.cuda.synchronize()
        o.fill_(float("nan")), lse.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        go, gl = o.clone(), lse.clone()
        eo, el = fa.fwd(q, k, v, **call)                # eager, fresh outputs
        torch.cuda.synchronize()
        assert torch.equal(go, eo) and torch.equal(gl, el), f"{label}: replay {r} differs from the eager call"
        if r == 0:
            compare(hq, hk, hv, causal, scale, go.cpu(), gl.cpu(), label=f"graph {label}")


def test_backward_graph_replays():
    say("case graph bwd")
    B, N, Hq, Hkv, d = 1, 300, 4, 2, 128
    q, k, v = (t.cuda() for t in rand_inputs(B, N, Hq, Hkv, d, "bf16", seed=21))
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(22)).to(torch.bfloat16).cuda()
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, Hq, N), dtype=torch.uint8, device=q.device)
    fa.bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    for r in range(3):
        do.copy_(torch.randn(q.shape, generator=torch.Generator().manual_seed(30 + r)).to(torch.bfloat16).cuda())
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        g = [t.clone() for t in (dq, dk, dv)]
        e = fa.bwd(q, k, v, o, lse, do, causal=True)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(g, e)), f"backward replay {r} differs from the eager call"
