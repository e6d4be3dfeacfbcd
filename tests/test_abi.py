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
    assert fa.fa_version() == 200
    for st in range(12):
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
    bad_d = (0, 32, 96, 512) if entry is fa.fa_fwd else (0, 32, 96, 256, 512)   # bf16 takes d = 256
    for d in bad_d:
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


W = 0x60000000   # fake workspace address
SGOOD = dict(B=2, Hq=4, Hkv=2, Nq=16, Nk=300, d=64, scale=0.125, causal=1, ns=3)


def scall(entry, q=Q, k=K, v=V, o=O, lse=L, ws=W, ws_bytes=1 << 24, **kw):
    a = dict(SGOOD)
    a.update(kw)
    return entry(q, k, v, o, lse, a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                 a["ns"], ws, ws_bytes, None)


@pytest.mark.parametrize("entry", [fa.fa_fwd_splitkv, fa.fa_fwd_splitkv_f32], ids=["bf16", "f32"])
def test_invalid_arguments_split(lib, entry):
    S = fa.STATUS
    assert scall(entry, q=None) == S["FA_ERR_NULL"]
    for bad in (dict(Nq=0), dict(Nk=0), dict(Nk=-1), dict(B=0)):
        assert scall(entry, **bad) == S["FA_ERR_SHAPE"], bad
    assert scall(entry, Nk=1 << 20, Hkv=32, Hq=32, d=128) == S["FA_ERR_SHAPE"]
    assert scall(entry, Nq=1 << 20, Hkv=1, Hq=32, d=128) == S["FA_ERR_SHAPE"]
    assert scall(entry, Hq=3) == S["FA_ERR_HEADS"]
    assert scall(entry, d=512) == S["FA_ERR_HEADDIM"]
    if entry is fa.fa_fwd_splitkv_f32:
        assert scall(entry, d=256) == S["FA_ERR_HEADDIM"]
    else:   # d = 256 passes the head-dim check; keep another argument invalid so nothing launches
        assert scall(entry, d=256, q=Q + 8) == S["FA_ERR_ALIGN"]
    for ns in (-1, 257, 1 << 30):
        assert scall(entry, ns=ns) == S["FA_ERR_SPLITS"], ns
    need = fa.fa_splitkv_workspace_size(2, 4, 2, 16, 300, 64, 3)
    assert scall(entry, ws=None) == S["FA_ERR_WORKSPACE"]
    assert scall(entry, ws_bytes=need - 1) == S["FA_ERR_WORKSPACE"]
    assert scall(entry, ws=W + 8) == S["FA_ERR_WORKSPACE"]
    assert scall(entry, ws=O) == S["FA_ERR_ALIAS"]          # workspace on the output
    assert scall(entry, ws=K - 64) == S["FA_ERR_ALIAS"]     # workspace running into k
    assert scall(entry, lse=W) == S["FA_ERR_ALIAS"]
    # one range needs no workspace, so a NULL one is not an error; keep an
    # earlier argument invalid so that nothing is launched
    assert scall(entry, ns=1, ws=None, ws_bytes=0, q=Q + 8) == S["FA_ERR_ALIGN"]
    assert scall(entry, ns=1, ws=None, ws_bytes=0, scale=float("nan")) == S["FA_ERR_SCALE"]


def test_split_shape_helpers(lib):
    n = fa.fa_splitkv_num_splits
    w = fa.fa_splitkv_workspace_size
    # ranges are whole 64-key quanta, none empty: 300 keys = 5 quanta
    assert n(1, 1, 1, 1, 300, 64, 1) == 1
    assert n(1, 1, 1, 1, 300, 64, 2) == 2      # 3 + 2 quanta
    assert n(1, 1, 1, 1, 300, 64, 4) == 3      # 2 + 2 + 1 quanta
    assert n(1, 1, 1, 1, 300, 64, 5) == 5
    assert n(1, 1, 1, 1, 300, 64, 200) == 5
    assert n(1, 1, 1, 1, 64, 64, 8) == 1
    assert n(1, 1, 1, 1, 65, 64, 8) == 2
    assert w(1, 1, 1, 1, 300, 64, 1) == 0
    assert w(2, 4, 2, 16, 300, 64, 3) == 3 * 2 * 4 * 16 * 65 * 4
    assert w(1, 32, 8, 1, 32768, 128, 64) == 64 * 32 * 129 * 4
    # the library's choice: decode with few heads splits, a big prefill does not
    assert n(1, 32, 8, 1, 32768, 128, 0) > 8
    assert n(2, 32, 32, 4096, 4096, 128, 0) == 1
    assert n(1, 1, 1, 1, 100, 64, 0) == 1     # too short to split
    assert n(1, 3, 2, 1, 100, 64, 0) == -fa.STATUS["FA_ERR_SHAPE"]
    assert n(1, 4, 2, 1, 100, 96, 0) == -fa.STATUS["FA_ERR_HEADDIM"]
    assert n(1, 4, 2, 1, 100, 64, -2) == -fa.STATUS["FA_ERR_SPLITS"]
    assert w(1, 3, 2, 1, 100, 64, 4) == 0


def bcall(q=Q, k=K, v=V, o=O, lse=L, do=0x70000000, dq=0x80000000, dk=0x90000000, dv=0xA0000000,
          ws=W, ws_bytes=1 << 24, **kw):
    a = dict(B=2, Hq=4, Hkv=2, Nq=16, Nk=300, d=64, scale=0.125, causal=1)
    a.update(kw)
    return fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                     a["scale"], a["causal"], ws, ws_bytes, None)


def test_invalid_arguments_bwd(lib):
    S = fa.STATUS
    for name in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"):
        assert bcall(**{name: None}) == S["FA_ERR_NULL"], name
    for bad in (dict(B=0), dict(Nq=0), dict(Nk=0), dict(Hkv=0)):
        assert bcall(**bad) == S["FA_ERR_SHAPE"], bad
    assert bcall(Nk=1 << 20, Hkv=32, Hq=32, d=128) == S["FA_ERR_SHAPE"]
    assert bcall(Hq=3) == S["FA_ERR_HEADS"]
    assert bcall(d=96) == S["FA_ERR_HEADDIM"]
    assert bcall(d=256) == S["FA_ERR_HEADDIM"]
    assert bcall(dk=0x90000008) == S["FA_ERR_ALIGN"]
    assert bcall(lse=L + 2) == S["FA_ERR_ALIGN"]
    assert bcall(scale=float("inf")) == S["FA_ERR_SCALE"]
    assert bcall(ws=None) == S["FA_ERR_WORKSPACE"]
    assert bcall(ws_bytes=fa.fa_bwd_workspace_size(2, 4, 16) - 4) == S["FA_ERR_WORKSPACE"]
    assert bcall(dq=Q) == S["FA_ERR_ALIAS"]
    assert bcall(dv=0x90000000 + 64) == S["FA_ERR_ALIAS"]       # dv overlaps dk
    assert bcall(ws=L) == S["FA_ERR_ALIAS"]                      # workspace on lse
    assert fa.fa_bwd_workspace_size(2, 4, 16) == 2 * (2 * 4 * 16 * 4)   # delta and lse in base 2
    assert fa.fa_bwd_workspace_size(0, 4, 16) == 0


def test_invalid_arguments_fp8(lib):
    S = fa.STATUS
    QD, KD, VD = 0xB0000000, 0xB0001000, 0xB0002000

    def fcall(q=Q, k=K, v=V, qd=QD, kd=KD, vd=VD, o=O, lse=L, **kw):
        a = dict(B=1, Hq=4, Hkv=2, N=16, d=128, scale=0.1, causal=1)
        a.update(kw)
        return fa.fa_fwd_fp8(q, k, v, qd, kd, vd, o, lse, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["scale"],
                             a["causal"], None)
    assert fcall(qd=None) == S["FA_ERR_NULL"]
    assert fcall(v=None) == S["FA_ERR_NULL"]
    assert fcall(d=64) == S["FA_ERR_HEADDIM"]
    assert fcall(kd=KD + 2) == S["FA_ERR_ALIGN"]
    assert fcall(q=Q + 4) == S["FA_ERR_ALIGN"]
    assert fcall(N=0) == S["FA_ERR_SHAPE"]
    assert fcall(Hq=3) == S["FA_ERR_HEADS"]
    assert fcall(scale=float("nan")) == S["FA_ERR_SCALE"]
    assert fcall(o=Q + 1024) == S["FA_ERR_ALIAS"]      # bf16 output running over the fp8 q


def test_invalid_arguments_blocksparse(lib):
    S = fa.STATUS
    MK = 0xC0000000

    def mcall(q=Q, k=K, v=V, o=O, lse=L, mask=MK, **kw):
        a = dict(B=1, Hq=4, Hkv=2, N=300, d=128, scale=0.1, causal=1)
        a.update(kw)
        return fa.fa_fwd_blocksparse(q, k, v, o, lse, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["scale"],
                                     a["causal"], mask, None)
    assert mcall(mask=None) == S["FA_ERR_NULL"]
    assert mcall(q=None) == S["FA_ERR_NULL"]
    assert mcall(N=65537) == S["FA_ERR_SHAPE"]
    assert mcall(d=96) == S["FA_ERR_HEADDIM"]
    assert mcall(Hq=3) == S["FA_ERR_HEADS"]
    assert mcall(o=O + 2) == S["FA_ERR_ALIGN"]
    assert mcall(lse=Q) == S["FA_ERR_ALIAS"]


def test_invalid_arguments_fp8_block(lib):
    S = fa.STATUS
    QE, KE, VE = 0xB0000000, 0xB0001000, 0xB0002000

    def fcall(q=Q, k=K, v=V, qe=QE, ke=KE, ve=VE, o=O, lse=L, **kw):
        a = dict(B=1, Hq=4, Hkv=2, N=16, d=128, scale=0.1, causal=1)
        a.update(kw)
        return fa.fa_fwd_fp8_block(q, k, v, qe, ke, ve, o, lse, a["B"], a["Hq"], a["Hkv"], a["N"], a["d"],
                                   a["scale"], a["causal"], None)
    assert fcall(ve=None) == S["FA_ERR_NULL"]
    assert fcall(k=None) == S["FA_ERR_NULL"]
    assert fcall(d=64) == S["FA_ERR_HEADDIM"]
    assert fcall(q=Q + 4) == S["FA_ERR_ALIGN"]
    assert fcall(N=0) == S["FA_ERR_SHAPE"]
    assert fcall(Hq=3) == S["FA_ERR_HEADS"]
    assert fcall(scale=float("inf")) == S["FA_ERR_SCALE"]
    assert fcall(qe=O + 8) == S["FA_ERR_ALIAS"]        # exponents inside the output
    assert fcall(ke=L) == S["FA_ERR_ALIAS"]            # exponents on lse


def test_invalid_arguments_quantize_fp8(lib):
    S = fa.STATUS
    X, C, E, SG = 0x10000000, 0x20000000, 0x30000000, 0x40000000

    def qcall(x=X, c=C, e=E, sg=SG, B=1, N=100, H=2, d=128):
        return fa.fa_quantize_fp8(x, c, e, B, N, H, d, sg, None)
    assert qcall(x=None) == S["FA_ERR_NULL"]
    assert qcall(e=None) == S["FA_ERR_NULL"]
    assert qcall(N=0) == S["FA_ERR_SHAPE"]
    assert qcall(N=(1 << 29) // 256) == S["FA_ERR_SHAPE"]
    assert qcall(d=64) == S["FA_ERR_HEADDIM"]
    assert qcall(x=X + 8) == S["FA_ERR_ALIGN"]
    assert qcall(c=C + 4) == S["FA_ERR_ALIGN"]
    assert qcall(sg=SG + 1) == S["FA_ERR_ALIGN"]
    assert qcall(c=X + 64) == S["FA_ERR_ALIAS"]       # codes over the input
    assert qcall(e=C + 16) == S["FA_ERR_ALIAS"]       # exponents over the codes
