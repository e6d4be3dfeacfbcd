"""HIP path vs the fp64 oracle on small shapes: several tiles, ragged tails,
MHA / MQA / GQA, both head dims, both dtypes, causal and not, edge cases."""
import math

import numpy as np
import pytest
import torch

import exact_attention_93_amd as fa
from tests.gpu_util import compare, gpu_fwd, rand_inputs, say

pytestmark = pytest.mark.gpu

NS = [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 255, 300]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", NS)
def test_small_gqa(N, causal, d, dtype):
    B, Hq, Hkv = 2, 8, 2
    say(f"case small_gqa N={N} causal={causal} d={d} dtype={dtype}")
    q, k, v = rand_inputs(B, N, Hq, Hkv, d, dtype, seed=N * 7 + d + causal)
    o, lse = gpu_fwd(q, k, v, causal, 1 / math.sqrt(d))
    compare(q, k, v, causal, 1 / math.sqrt(d), o, lse, label=f"N={N}", num_splits=1)


@pytest.mark.parametrize("heads", [(1, 1), (4, 1), (3, 3), (6, 2)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_head_layouts(heads, causal, dtype):
    Hq, Hkv = heads
    say(f"case heads={heads} causal={causal} dtype={dtype}")
    for B, N, d in [(1, 200, 128), (3, 77, 64)]:
        q, k, v = rand_inputs(B, N, Hq, Hkv, d, dtype, seed=B * 100 + N + Hq)
        o, lse = gpu_fwd(q, k, v, causal, 1 / math.sqrt(d))
        compare(q, k, v, causal, 1 / math.sqrt(d), o, lse, label=f"B={B} N={N} d={d}", num_splits=1)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.5, 3e-3])
def test_scales(scale, dtype):
    say(f"case scale={scale} dtype={dtype}")
    q, k, v = rand_inputs(1, 150, 4, 4, 64, dtype, seed=5, q_std=2.0)
    for causal in (False, True):
        o, lse = gpu_fwd(q, k, v, causal, scale)
        compare(q, k, v, causal, scale, o, lse, label=f"scale={scale} causal={causal}", num_splits=1)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_peaked_logits_rescale(dtype):
    # large |q| makes the running maximum jump often: exercises the rescale
    say(f"case peaked dtype={dtype}")
    q, k, v = rand_inputs(1, 700, 2, 1, 128, dtype, seed=9, q_std=8.0)
    for causal in (False, True):
        o, lse = gpu_fwd(q, k, v, causal, 1 / math.sqrt(128))
        compare(q, k, v, causal, 1 / math.sqrt(128), o, lse, label=f"peaked causal={causal}", num_splits=1)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_worked_example(dtype):
    """The second page's section 8 example embedded at d = 64: scores
    (sqrt2, 1/sqrt2, 1/sqrt2) and v[:, 0] = (1, 0, 1) give O[:, 0] = 0.752."""
    say(f"case worked_example dtype={dtype}")
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    q = torch.zeros(1, 3, 1, 64)
    q[..., 0] = 1
    q[..., 1] = 1
    k = torch.zeros(1, 3, 1, 64)
    k[0, 0, 0, :2] = 1
    k[0, 1, 0, 0] = 1
    k[0, 2, 0, 1] = 1
    v = torch.zeros(1, 3, 1, 64)
    v[0, :, 0, 0] = torch.tensor([1.0, 0.0, 1.0])
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    o, lse = gpu_fwd(q, k, v, False, 1 / math.sqrt(2))
    tol = 1e-5 if dtype == "fp32" else 1e-2
    assert abs(o[0, :, 0, 0].float() - 0.751745).max() < tol
    if dtype == "fp32":   # the page's three decimals
        assert abs(round(float(o[0, 0, 0, 0]), 3) - 0.752) < 1e-9
    else:                 # 0.752 is not a bf16 value: within one bf16 ulp (2^-8 at 0.75)
        assert abs(float(o[0, 0, 0, 0]) - 0.752) <= 2 ** -8
    compare(q, k, v, False, 1 / math.sqrt(2), o, lse, label="worked example", num_splits=1)


def test_properties_bf16():
    """Rows of P sum to one, outputs in the convex hull of V, shift invariance."""
    B, N, Hq, Hkv, d = 1, 333, 4, 2, 64
    q, k, v = rand_inputs(B, N, Hq, Hkv, d, "bf16", seed=77)
    v1 = v.clone()
    v1[..., 5] = 1.0
    for causal in (False, True):
        o, lse = gpu_fwd(q, k, v1, causal, 0.125)
        assert (o[..., 5].float() - 1.0).abs().max() <= 2 ** -8, "ones column"
        vf = v1.float()
        g = Hq // Hkv
        for h in range(Hq):
            for i in (0, 1, 50, N - 1):
                vis = vf[0, : (i + 1 if causal else N), h // g]
                assert torch.all(o[0, i, h].float() >= vis.min(0).values - 1e-2)
                assert torch.all(o[0, i, h].float() <= vis.max(0).values + 1e-2)
        # shift: k[..., 63] = 1 and q[..., 63] = c_i / scale (exact in bf16)
        qa, ka = q.clone(), k.clone()
        qa[..., 63] = 0
        ka[..., 63] = 1
        o0, l0 = gpu_fwd(qa, ka, v1, causal, 0.125)
        c = torch.randint(-8, 9, (B, N, Hq)).float() * 0.5
        qs = qa.clone()
        qs[..., 63] = (c / 0.125).to(torch.bfloat16)
        o1, l1 = gpu_fwd(qs, ka, v1, causal, 0.125)
        assert (o1.float() - o0.float()).abs().max() <= 1e-2
        assert ((l1 - l0) - c.permute(0, 2, 1)).abs().max() <= 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_deterministic_and_every_output_written(dtype):
    q, k, v = rand_inputs(2, 257, 4, 2, 128, dtype, seed=3)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for causal in (False, True):
        o1 = torch.full_like(qd, float("nan"))
        l1 = torch.full((2, 4, 257), float("nan"), device="cuda")
        fa.fwd(qd, kd, vd, causal=causal, out=o1, lse=l1)
        o2 = torch.full_like(qd, float("nan"))
        l2 = torch.full((2, 4, 257), float("nan"), device="cuda")
        fa.fwd(qd, kd, vd, causal=causal, out=o2, lse=l2)
        torch.cuda.synchronize()
        assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all(), "unwritten output"
        assert torch.equal(o1.view(torch.int16) if dtype == "bf16" else o1.view(torch.int32),
                           o2.view(torch.int16) if dtype == "bf16" else o2.view(torch.int32))
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_causal_row_equals_prefix_attention():
    q, k, v = rand_inputs(1, 300, 2, 2, 64, "bf16", seed=12)
    o, lse = gpu_fwd(q, k, v, True, 0.125)
    for i in (0, 64, 127, 128, 299):
        op, lp = gpu_fwd(q[:, : i + 1].contiguous(), k[:, : i + 1].contiguous(), v[:, : i + 1].contiguous(), False, 0.125)
        assert (o[0, i].float() - op[0, i].float()).abs().max() <= 1e-2
        assert (lse[0, :, i] - lp[0, :, i]).abs().max() <= 1e-4 * max(1.0, float(lse[0, :, i].abs().max()))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_scores_growing_past_the_reference(dtype, causal):
    """Scores that climb steeply with the key index: every new tile's maximum
    sits far (hundreds, base 2) above the running reference, so the kernels
    must move the reference and rescale on every tile: q = (1, small...),
    k_j = (j/8 rounded to the input type, small...), so the scores rise by
    about 8*scale per 64 keys (46 and 460 in base 2 for the two scales); the
    oracle reads the same rounded values."""
    say(f"case growing scores dtype={dtype} causal={causal}")
    N, d = 333, 64
    q, k, v = rand_inputs(1, N, 2, 1, d, dtype, seed=21)
    dt = q.dtype
    q = (q.float() * 0.01).to(dt)
    k = (k.float() * 0.01).to(dt)
    q[..., 0] = 1.0
    k[..., 0] = (torch.arange(N, dtype=torch.float32) / 8.0).view(1, N, 1).to(dt)
    for scale in (4.0, 40.0):
        o, lse = gpu_fwd(q, k, v, causal, scale)
        compare(q, k, v, causal, scale, o, lse, label=f"growing scale={scale}", num_splits=1)
