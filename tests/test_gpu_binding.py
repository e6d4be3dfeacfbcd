"""The Python binding rejects caller-supplied outputs and workspaces that do
not fit what the kernels write, before anything is launched (the buffers
keep their contents)."""
import pytest
import torch

import exact_attention_93_amd as fa
from tests.gpu_util import rand_inputs, say

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def inputs(N=70, Nk=None, dtype="bf16"):
    return tuple(t.cuda() for t in rand_inputs(1, N, 4, 2, 64, dtype, seed=3, Nk=Nk))


def filled(shape, dtype):
    return torch.full(shape, SENTINEL, dtype=dtype, device="cuda")


def untouched(*ts):
    torch.cuda.synchronize()
    return all(bool((t.float() == SENTINEL).all()) for t in ts)


@pytest.mark.parametrize("bad", ["shape", "dtype", "strided", "lse_shape", "lse_dtype", "host"])
def test_fwd_rejects_bad_outputs(bad):
    say(f"case binding fwd {bad}")
    q, k, v = inputs()
    out, lse = filled(q.shape, q.dtype), filled((1, 4, 70), torch.float32)
    if bad == "shape":
        out = filled((1, 69, 4, 64), q.dtype)
    elif bad == "dtype":
        out = filled(q.shape, torch.float32)
    elif bad == "strided":
        out = filled((1, 4, 70, 64), q.dtype).transpose(1, 2)
    elif bad == "lse_shape":
        lse = filled((1, 70, 4), torch.float32)
    elif bad == "lse_dtype":
        lse = filled((1, 4, 70), torch.bfloat16)
    elif bad == "host":
        out = torch.full(q.shape, SENTINEL, dtype=q.dtype)
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, causal=True, out=out, lse=lse)
    assert untouched(lse) and (bad == "host" or untouched(out))


def test_split_rejects_small_or_host_workspace():
    say("case binding split workspace")
    q, k, v = inputs(N=3, Nk=900)
    need = fa.fa_splitkv_workspace_size(1, 4, 2, 3, 900, 64, 4)
    assert need > 0
    out, lse = filled(q.shape, q.dtype), filled((1, 4, 3), torch.float32)
    for ws in (torch.empty(need - 1, dtype=torch.uint8, device="cuda"), torch.empty(need, dtype=torch.uint8)):
        with pytest.raises(ValueError):
            fa.fwd(q, k, v, causal=True, out=out, lse=lse, num_splits=4, workspace=ws)
    assert untouched(out, lse)
    fa.fwd(q, k, v, causal=True, out=out, lse=lse, num_splits=4,
           workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    assert not untouched(out)


def test_bwd_rejects_bad_gradients():
    say("case binding bwd")
    q, k, v = inputs()
    o, lse = fa.fwd(q, k, v, causal=True)
    do = torch.randn_like(q)
    dq, dk = filled(q.shape, q.dtype), filled(k.shape, k.dtype)
    for kw in (dict(dq=filled(k.shape, q.dtype)), dict(dk=filled(q.shape, k.dtype)),
               dict(dv=filled(k.shape, torch.float32)),
               dict(workspace=torch.empty(fa.fa_bwd_workspace_size(1, 4, 70) - 1, dtype=torch.uint8,
                                          device="cuda"))):
        args = dict(dq=dq, dk=dk)
        args.update(kw)
        with pytest.raises(ValueError):
            fa.bwd(q, k, v, o, lse, do, causal=True, **args)
    assert untouched(dq, dk)


def test_fp8_and_blocksparse_reject_bad_outputs():
    say("case binding fp8 / blocksparse")
    q, k, v = inputs(N=130)
    codes = [t.to(torch.float8_e4m3fn) for t in (q, k, v)]
    qd = torch.ones(1, 4, device="cuda")
    kd = torch.ones(1, 2, device="cuda")
    with pytest.raises(ValueError):
        fa.fwd_fp8(codes[0], codes[1], codes[2], qd, kd, kd.clone(), out=filled((1, 130, 4, 64), torch.float32))
    q128, k128, v128 = (torch.randn(1, 130, h, 128, device="cuda").to(torch.bfloat16) for h in (4, 2, 2))
    with pytest.raises(ValueError):
        fa.fwd_fp8(*(t.to(torch.float8_e4m3fn) for t in (q128, k128, v128)), qd, kd, kd.clone(),
                   lse=filled((1, 4, 129), torch.float32))
    mask = torch.ones(4, 2, 3, dtype=torch.uint8, device="cuda")
    lse = filled((4, 130), torch.float32)
    with pytest.raises(ValueError):
        fa.fwd_blocksparse(q, k, v, mask, lse=lse)
    assert untouched(lse)


def _hip_runtime():
    """The HIP runtime library this process (and libfa.so) uses."""
    import ctypes
    path = next(ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln)
    hip = ctypes.CDLL(path)
    hip.hipSetDevice.restype = ctypes.c_int
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    return hip


def test_stale_runtime_error_does_not_fail_a_launch():
    """An earlier failed HIP call elsewhere in the process (here a rejected
    device index) leaves HIP's last-error state set; the entry points still
    report their own launches as successful."""
    say("case binding stale runtime error")
    q, k, v = inputs()
    hip = _hip_runtime()
    for call in (lambda: fa.fwd(q, k, v, causal=True),
                 lambda: fa.fwd(q, k, v, num_splits=3),
                 lambda: fa.bwd(q, k, v, *fa.fwd(q, k, v, causal=True), torch.randn_like(q), causal=True)):
        assert hip.hipSetDevice(9999) != 0          # rejected by the runtime, nothing else happens
        call()
    torch.cuda.synchronize()
