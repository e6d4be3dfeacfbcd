"""The C ABI on the CPU: the library loads, exports what include/fa.h
declares, and rejects invalid arguments before any HIP call (so these calls
are safe without a GPU: none of them reaches a launch)."""
import ctypes
import os
import re
import subprocess

import pytest

import exact_attention_93_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH if hasattr(fa, "LIB_PATH") else fa._build.LIB_PATH):
        pytest.fail("libfa.so is not built; run __graft_entry__.build()")
    return fa.load_library()


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(fa.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa._build.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(fa_\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name, val in fa.STATUS.items():
        assert re.search(rf"\b{name}\s*=\s*{val}\b", text), name


def test_version_and_strerror(lib):
    assert fa.fa_version() == 100
    for st in range(9):
        assert fa.fa_strerror(st)
    assert "unknown" in fa.fa_strerror(99)


# Fake, well-separated, 16-byte aligned "device" addresses: every call below
# fails validation, so nothing is ever dereferenced or launched.
Q, K, V, O, L = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
GOOD = dict(B=1, Hq=4, Hkv=2, N=16, d=64, scale=0.125, causal=1)


def call(entry, q=Q, k=K, v=V, o=O, lse=L, **kw):
    a = dict(GOOD)
    a.update(kw)
    return entry(q, k, v, o, lse, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], None)


@pytest.mark.parametrize("entry", [fa.fa_fwd, fa.fa_fwd_f32], ids=["bf16", "f32"])
def test_invalid_arguments(lib, entry):
    S = fa.STATUS
    assert call(entry, q=None) == S["FA_ERR_NULL"]
    assert call(entry, lse=None) == S["FA_ERR_NULL"]
    assert call(entry, o=0) == S["FA_ERR_NULL"]
    for bad in (dict(B=0), dict(Hq=0), dict(Hkv=0), dict(N=0), dict(N=-5)):
        assert call(entry, **bad) == S["FA_ERR_SHAPE"], bad
    assert call(entry, N=1 << 20, Hq=32, Hkv=32, d=128) == S["FA_ERR_SHAPE"]
    assert call(entry, Hq=6, Hkv=4) == S["FA_ERR_HEADS"]
    for d in (0, 32, 96, 256):
        assert call(entry, d=d) == S["FA_ERR_HEADDIM"], d
    assert call(entry, q=Q + 8) == S["FA_ERR_ALIGN"]
    assert call(entry, o=O + 2) == S["FA_ERR_ALIGN"]
    assert call(entry, lse=L + 2) == S["FA_ERR_ALIGN"]
    for sc in (float("nan"), float("inf"), -float("inf"), 1e-45):
        assert call(entry, scale=sc) == S["FA_ERR_SCALE"], sc
    assert call(entry, o=Q) == S["FA_ERR_ALIAS"]
    assert call(entry, lse=K + 64) == S["FA_ERR_ALIAS"]
    assert call(entry, lse=O + 16) == S["FA_ERR_ALIAS"]


def test_python_wrapper_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd(x, x, x)
