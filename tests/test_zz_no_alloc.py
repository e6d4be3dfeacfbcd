"""fa_fwd_splitkv_static (the allocation-free split forward, partials in the
library's static device array) against fa_fwd_splitkv with a caller
workspace: the same kernels, so the same bits; two calls in a row, the second
smaller, so the second runs on the array the first one left behind."""
import pytest
import torch

import exact_attention_93_amd as fa
from exact_attention_93_amd import workloads as W
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def run_pair(B, Hq, Hkv, Nq, Nk, d, causal, splits, seed):
    w = W.make(B=B, Hq=Hq, Hkv=Hkv, N=Nq, Nk=Nk, d=d, dtype="bf16", causal=causal, seed=seed, name="noalloc")
    q, k, v = (t.cuda() for t in W.gen_inputs(w))
    st = torch.cuda.current_stream()
    need = fa.fa_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, splits)
    used = fa.fa_splitkv_num_splits(B, Hq, Hkv, Nq, Nk, d, splits)
    say(f"case no-alloc B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} splits={used} scratch={need}")
    assert 0 < need <= fa.STATIC_SCRATCH_BYTES
    o_ref = torch.empty_like(q)
    l_ref = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    assert fa.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_ref.data_ptr(), l_ref.data_ptr(), B, Hq, Hkv,
                             Nq, Nk, d, w.scale, causal, splits, ws.data_ptr(), need, st.cuda_stream) == 0
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device="cuda")
    assert fa.fa_fwd_splitkv_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq,
                                    Hkv, Nq, Nk, d, w.scale, causal, splits, st.cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "outputs differ from the workspace entry point"
    assert torch.equal(lse, l_ref), "lse differs from the workspace entry point"


def test_static_scratch_two_calls_second_smaller():
    run_pair(1, 32, 8, 1, 32768, 128, True, 0, seed=11)          # decoding step, 32 ranges
    run_pair(1, 8, 2, 50, 2000, 64, True, 4, seed=12)            # smaller: 4 ranges, d = 64


def test_static_scratch_prefill_split():
    run_pair(2, 8, 4, 300, 1100, 128, False, 3, seed=13)


def test_static_scratch_without_a_split_and_too_large():
    # one range: no scratch at all, the plain forward
    w = W.make(B=1, Hq=4, Hkv=4, N=200, d=128, dtype="bf16", causal=True, seed=14, name="noalloc1")
    q, k, v = (t.cuda() for t in W.gen_inputs(w))
    st = torch.cuda.current_stream().cuda_stream
    o, lse = torch.empty_like(q), torch.empty((1, 4, 200), dtype=torch.float32, device="cuda")
    assert fa.fa_fwd_splitkv_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    1, 4, 4, 200, 200, 128, w.scale, 1, 1, st) == 0
    o_ref, l_ref = fa.fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(lse, l_ref)
    # a split that needs more than the array holds is refused before any launch
    B, Hq, N = 4, 32, 4096
    assert fa.fa_splitkv_workspace_size(B, Hq, Hq, N, N, 128, 4) > fa.STATIC_SCRATCH_BYTES
    big = torch.zeros((B, N, Hq, 128), dtype=torch.bfloat16, device="cuda")
    ob = torch.full_like(big, 7.0)
    lb = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    rc = fa.fa_fwd_splitkv_static(big.data_ptr(), big.data_ptr(), big.data_ptr(), ob.data_ptr(), lb.data_ptr(),
                                  B, Hq, Hq, N, N, 128, 0.1, 1, 4, st)
    torch.cuda.synchronize()
    assert rc == fa.STATUS["FA_ERR_SCRATCH"]
    assert bool((ob == 7.0).all()), "a refused call must not write its outputs"
