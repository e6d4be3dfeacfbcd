"""The d = 256 forward's matrix products are inline assembly (fa_fwd_bf16.hip
says why), so the wait states the hardware needs around them are explicit
s_nop statements tied to their registers, and each run of products ends with
a statement that waits out the gap and claims its destinations.  This test
compiles the forward for gfx950, in both LDS layouts, and checks every d = 256
kernel on every control-flow path (tests/asm_hazards.py):

- S^T (VGPR destination) untouched for 11 wait states after its product, the
  O^T accumulator (AGPR destination) for 32;
- no vector write of a product's operands fewer than 2 wait states before it.

A copy of the source without the claim of O^T after the P V products must
fail the first check: the compiler copies the accumulator past the loop's
closing barrier, which another wavefront may already wait at."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from exact_attention_93_amd import _build
from tests.asm_hazards import dest_hazards, kernels, source_hazards

SRC = os.path.join(_build.CSRC, "fa_fwd_bf16.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
D256 = "fwd_bf16_kernelILi256E"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")


def _asm(src, out, single_stage):
    cmd = [HIPCC, *_build.HIPCC_FLAGS, "-I", os.path.join(_build.ROOT, "include"), "-I", _build.CSRC,
           f"-DFA_SINGLE_STAGE={int(single_stage)}", "--cuda-device-only", "-S", src, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return open(out).read()


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    tmp = tmp_path_factory.mktemp("asm")
    src = open(SRC).read()
    # the planted mistake: no claim of O^T after the P V products
    m = re.search(r"( *pv_ring\(vs\);\n)((?: *//[^\n]*\n)*) *sync_acc\(\);\n", src)
    assert m is not None and src.count("pv_ring(vs);") == 1
    planted = tmp / "fa_fwd_bf16_planted.hip"
    planted.write_text(src[:m.start()] + m.group(1) + src[m.end():])
    jobs = {"main": (SRC, False), "single_stage": (SRC, True), "planted": (str(planted), False)}
    with ThreadPoolExecutor(max_workers=3) as ex:
        futs = {k: ex.submit(_asm, s, str(tmp / f"{k}.s"), ss) for k, (s, ss) in jobs.items()}
        return {k: f.result() for k, f in futs.items()}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("layout", ["main", "single_stage"])
def test_d256_products_keep_their_gaps(listings, layout):
    ks = kernels(listings[layout], D256)
    assert len(ks) == 6, sorted(ks)     # causal x (split, block mask, plain)
    for name, code in ks.items():
        assert sum(ln.startswith("v_mfma") for ln in code) > 0, name
        dh = dest_hazards(code)
        sh = source_hazards(code)
        assert not dh, f"{name}: {len(dh)} early accesses to a product's destination, e.g. {dh[:2]}"
        assert not sh, f"{name}: {len(sh)} late writes of a product's operands, e.g. {sh[:2]}"


@pytest.mark.timeout(600)
def test_the_scan_catches_a_missing_claim(listings):
    ks = kernels(listings["planted"], D256)
    assert len(ks) == 6
    early = {name: dest_hazards(code) for name, code in ks.items()}
    assert any(early.values()), "the copy without the O^T claim shows no hazard"
    # what it finds is the accumulator copied while the products still write it
    name, hits = next((n, h) for n, h in early.items() if h)
    assert any(o.startswith("v_accvgpr") for _, o, _ in hits), hits[:3]


# The scans themselves, on short listings whose answer is known.
MF_S = "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], 0"           # S^T into v[0:15]
MF_S2 = "v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], a[4:7], v[0:15]"     # accumulates into it
MF_O = "v_mfma_f32_32x32x16_bf16 a[32:47], v[16:19], v[20:23], a[32:47]"  # O^T into a[32:47]


def test_scan_destination_rules():
    assert dest_hazards([MF_S, "v_mov_b32_e32 v40, v3"])                     # read at once
    assert not dest_hazards([MF_S, "s_nop 10", "v_mov_b32_e32 v40, v3"])     # 11 wait states
    assert dest_hazards([MF_S, "s_nop 9", "v_mov_b32_e32 v40, v3"])
    assert not dest_hazards([MF_S, MF_S2])                                   # same accumulator
    assert dest_hazards([MF_S, "v_mfma_f32_32x32x16_bf16 v[40:55], v[0:3], a[4:7], 0"])  # S^T as operand
    assert dest_hazards([MF_O, "s_nop 15", "v_accvgpr_mov_b32 a100, a47"])  # O^T needs 32
    assert not dest_hazards([MF_O, "s_nop 15", "s_nop 15", "v_accvgpr_mov_b32 a100, a47"])
    # a branch that skips the gap
    code = [MF_O, "s_cbranch_scc1 .LBB0_1", "s_nop 15", "s_nop 15", ".LBB0_1:", "v_accvgpr_mov_b32 a100, a47"]
    assert dest_hazards(code)
    code = [MF_O, "s_nop 15", "s_nop 15", "s_cbranch_scc1 .LBB0_1", ".LBB0_1:", "v_accvgpr_mov_b32 a100, a47"]
    assert not dest_hazards(code)


def test_scan_source_rules():
    assert source_hazards(["v_accvgpr_write_b32 a1, v9", MF_S])              # Q^T written at once
    assert source_hazards(["v_cvt_pk_bf16_f32 v17, v1, v2", "s_nop 0", MF_S])  # one wait state
    assert not source_hazards(["v_cvt_pk_bf16_f32 v17, v1, v2", "s_nop 1", MF_S])
    assert source_hazards(["v_accvgpr_mov_b32 a40, a200", MF_O])             # the accumulator moved in
    assert not source_hazards(["v_mov_b32_e32 v40, v1", MF_S])               # not an operand
    # a write that reaches the product only through a branch
    code = ["v_accvgpr_write_b32 a1, v9", "s_branch .LBB0_2", "s_nop 15", ".LBB0_2:", MF_S]
    assert source_hazards(code)
    code = ["v_accvgpr_write_b32 a1, v9", "s_branch .LBB0_3", ".LBB0_2:", MF_S, ".LBB0_3:", "s_nop 0"]
    assert not source_hazards(code)
