"""Unequal query/key lengths (bottom-right causal alignment, rows without
keys) and the split-key forward with its merge, HIP path vs the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import exact_attention_93_amd as fa
from exact_attention_93_amd import workloads as W
from tests import pins
from tests.gpu_util import compare, gpu_fwd, rand_inputs, say

pytestmark = pytest.mark.gpu

# (Nq, Nk): decode rows, short and long key sequences, ragged tails,
# more queries than keys (leading rows see nothing under causal)
SHAPES = [(1, 1), (1, 300), (3, 1000), (17, 300), (64, 65), (129, 1000), (300, 17), (1000, 129),
          (257, 256), (256, 257)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"q{s[0]}k{s[1]}")
def test_unequal_lengths(shape, causal, d, dtype):
    Nq, Nk = shape
    say(f"case unequal Nq={Nq} Nk={Nk} causal={causal} d={d} dtype={dtype}")
    q, k, v = rand_inputs(2, Nq, 4, 2, d, dtype, seed=Nq * 31 + Nk + d + causal, Nk=Nk)
    o, lse = gpu_fwd(q, k, v, causal, 1 / math.sqrt(d))
    compare(q, k, v, causal, 1 / math.sqrt(d), o, lse, label=f"Nq={Nq} Nk={Nk}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("splits", [2, 3, 7, 0])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1000), (5, 700), (129, 1000), (300, 300), (1000, 300), (600, 129)],
                         ids=lambda s: f"q{s[0]}k{s[1]}")
def test_split(shape, causal, splits, dtype):
    Nq, Nk = shape
    d = 128 if Nq % 2 else 64
    used = fa.fa_splitkv_num_splits(2, 4, 2, Nq, Nk, d, splits)
    say(f"case split Nq={Nq} Nk={Nk} causal={causal} splits={splits} (used {used}) dtype={dtype}")
    q, k, v = rand_inputs(2, Nq, 4, 2, d, dtype, seed=Nq + 7 * Nk + splits, Nk=Nk)
    o, lse = gpu_fwd(q, k, v, causal, 1 / math.sqrt(d), num_splits=splits)
    compare(q, k, v, causal, 1 / math.sqrt(d), o, lse, label=f"Nq={Nq} Nk={Nk} splits={used}", num_splits=splits)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("splits", [1, 2])
def test_printed_masks(dtype, splits):
    """The two causal masks the first page prints for unequal lengths
    (section 0x09): with scale 0 and v_j the j-th unit vector, output row i
    is mask_i / |mask_i|, and zero for a row whose mask is all zero."""
    gold = pins.read_golden("causal_bottom_right.txt")
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    for name, nq, nk in (("q2_k5", 2, 5), ("q5_k2", 5, 2)):
        mask = np.array([np.atleast_1d(gold[f"{name}.row{i}"]) for i in range(nq)], dtype=np.float64)
        q, k, _ = rand_inputs(1, nq, 1, 1, 64, dtype, seed=3, Nk=nk)
        v = torch.zeros(1, nk, 1, 64)
        v[0, :, 0, :nk] = torch.eye(nk)
        v = v.to(dt)
        o, lse = gpu_fwd(q, k, v, True, 0.0, num_splits=splits)
        for i in range(nq):
            cnt = mask[i].sum()
            want = mask[i] / cnt if cnt else np.zeros(nk)
            got = o[0, i, 0, :nk].double().numpy()
            tol = 1e-7 if dtype == "fp32" else 2.0 ** -9
            assert np.abs(got - want).max() <= tol, (name, i, got, want)
            assert np.all(o[0, i, 0, nk:].float().numpy() == 0)
            if cnt:
                assert abs(float(lse[0, 0, i]) - math.log(cnt)) <= 1e-6
            else:
                assert float(lse[0, 0, i]) == -math.inf


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_split_workspace_contents_do_not_matter_and_runs_repeat(dtype):
    """Workspace filled with NaN first; two calls give bitwise equal results."""
    Nq, Nk, d = 33, 2000, 128
    q, k, v = rand_inputs(1, Nq, 8, 2, d, dtype, seed=44, Nk=Nk)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    need = fa.fa_splitkv_workspace_size(1, 8, 2, Nq, Nk, d, 5)
    ws = torch.full((need // 4,), float("nan"), device="cuda")
    outs = []
    for _ in range(2):
        o = torch.full_like(qd, float("nan"))
        l = torch.full((1, 8, Nq), float("nan"), device="cuda")
        fa.fwd(qd, kd, vd, causal=True, out=o, lse=l, num_splits=5, workspace=ws.view(torch.uint8))
        torch.cuda.synchronize()
        outs.append((o.cpu(), l.cpu()))
    (o1, l1), (o2, l2) = outs
    iv = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(o1.view(iv), o2.view(iv)) and torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    compare(q, k, v, True, 1 / math.sqrt(d), o1, l1, label="nan workspace")


def test_split_agrees_with_unsplit():
    """Split and unsplit results of the same call agree to within the bf16
    output rounding (they differ only in how the key ranges are merged)."""
    q, k, v = rand_inputs(1, 700, 4, 4, 128, "bf16", seed=8)
    o1, l1 = gpu_fwd(q, k, v, True, 0.0884)
    o4, l4 = gpu_fwd(q, k, v, True, 0.0884, num_splits=4)
    assert (o1.float() - o4.float()).abs().max() <= 2 * 2.0 ** -8
    assert ((l1 - l4).abs() / l1.abs().clamp(min=1)).max() <= 1e-5


@pytest.mark.parametrize("name", list(W.SPLIT_WORKLOADS))
def test_split_workload(name):
    """The split-key workloads at full size, launched as the benchmark launches them."""
    w = W.SPLIT_WORKLOADS[name]
    say(f"case split workload {name} splits={fa.fa_splitkv_num_splits(w.B, w.Hq, w.Hkv, w.N, w.Nkv, w.d, w.splits)}")
    q, k, v = W.gen_inputs(w)
    o, lse = gpu_fwd(q, k, v, w.causal, w.scale, num_splits=w.splits)
    compare(q, k, v, w.causal, w.scale, o, lse, rows=W.sample_rows(w), label=name, exact_bounds=True,
            num_splits=w.splits)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads_nq", [(1, 1, 1), (4, 1, 1), (8, 1, 2), (32, 8, 1), (16, 1, 4), (8, 2, 16),
                                      (13, 1, 5), (4, 4, 3)],
                         ids=lambda t: f"Hq{t[0]}Hkv{t[1]}Nq{t[2]}")
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_decode_shapes(heads_nq, causal, d, splits):
    """Few query rows per K/V head (one or two packed 32-row blocks; 13*5 = 65
    rows crosses over to the prefill kernel), long ragged key sequences."""
    Hq, Hkv, Nq = heads_nq
    Nk = 1000 + 37 * Nq
    say(f"case decode Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} d={d} splits={splits}")
    q, k, v = rand_inputs(2, Nq, Hq, Hkv, d, "bf16", seed=Hq * 100 + Nq + d + splits, Nk=Nk)
    o, lse = gpu_fwd(q, k, v, causal, 1 / math.sqrt(d), num_splits=splits)
    compare(q, k, v, causal, 1 / math.sqrt(d), o, lse, label=f"decode Hq={Hq} Hkv={Hkv} Nq={Nq}", num_splits=splits)


def test_decode_rows_without_keys():
    """More query rows than keys in the decoding kernel: rows i < Nq - Nk see
    nothing under the bottom-right alignment and must come out zero."""
    q, k, v = rand_inputs(1, 12, 4, 1, 128, "bf16", seed=5, Nk=7)
    for splits in (1, 2):
        o, lse = gpu_fwd(q, k, v, True, 0.1, num_splits=splits)
        compare(q, k, v, True, 0.1, o, lse, label=f"decode empty rows splits={splits}", num_splits=splits)
        assert torch.all(o[0, :5].float() == 0) and torch.all(torch.isneginf(lse[0, :, :5]))
