"""The block-scaled e4m3 quantiser of oracle/fp8.py against facts fixed
outside it (CPU only): the e4m3 format as torch implements it, the Hadamard
matrix as scipy builds it, orthogonality, brute-force exponents, and planted
mistakes that these checks must catch."""
import importlib.util
import os

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import fp8 as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_decode_landmarks():
    # 1.0, the largest finite value, the smallest normal and subnormal, NaN
    assert F.e4m3_decode(np.uint8(0x38)) == 1.0
    assert F.e4m3_decode(np.uint8(0x7E)) == 448.0
    assert F.e4m3_decode(np.uint8(0x08)) == 2.0 ** -6
    assert F.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9
    assert F.e4m3_decode(np.uint8(0xB8)) == -1.0
    assert np.isnan(F.e4m3_decode(np.uint8(0x7F))) and np.isnan(F.e4m3_decode(np.uint8(0xFF)))


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    back = F.e4m3_encode(F.e4m3_decode(codes))
    # -0 keeps its sign bit; every other code comes back as itself
    assert np.array_equal(back, codes)


def test_encode_ties_go_to_even():
    # 1.0625 lies halfway between 1.0 (0x38, mantissa 000) and 1.125 (0x39)
    assert F.e4m3_encode(1.0625) == 0x38
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3a): even is 0x3a
    assert F.e4m3_encode(1.1875) == 0x3A
    # halfway between the two smallest subnormals 2^-9 and 2^-8 -> 2^-8 (even)
    assert F.e4m3_encode(1.5 * 2.0 ** -9) == 0x02
    assert F.e4m3_encode(-1.0625) == 0xB8


def test_encode_matches_torch_on_random_values():
    g = np.random.default_rng(5)
    x = np.concatenate([g.standard_normal(20000) * s for s in (1e-3, 0.1, 1.0, 30.0)])
    x = np.clip(x, -448, 448).astype(np.float32)
    ours = F.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_rejects_values_beyond_the_format():
    with pytest.raises(ValueError):
        F.e4m3_encode(449.0)
    with pytest.raises(ValueError):
        F.e4m3_encode(np.inf)


def test_butterfly_is_the_hadamard_product():
    # small integers: every butterfly sum is exact in float32, so the result
    # must equal x @ H exactly, H from scipy
    g = np.random.default_rng(1)
    for d in (2, 8, 64, 128):
        x = g.integers(-50, 51, size=(5, d)).astype(np.float32)
        H = scipy.linalg.hadamard(d).astype(np.float64)
        assert np.array_equal(F.hadamard_butterfly_f32(x).astype(np.float64), x.astype(np.float64) @ H)


def test_butterfly_float32_rounding_stays_within_float32_error():
    g = np.random.default_rng(2)
    x = g.standard_normal((200, 128)).astype(np.float32)
    exact = x.astype(np.float64) @ scipy.linalg.hadamard(128).astype(np.float64)
    y = F.hadamard_butterfly_f32(x).astype(np.float64)
    # 7 stages of additions, each with relative error <= 2^-24 of a partial sum
    # bounded by sum |x|
    bound = 7 * 2.0 ** -24 * np.abs(x).astype(np.float64).sum(axis=1, keepdims=True)
    assert np.all(np.abs(y - exact) <= bound)


def test_rotation_multiplies_scores_by_d():
    g = np.random.default_rng(3)
    d = 128
    s = np.where(g.random(d) < 0.5, -1.0, 1.0)
    q = g.integers(-20, 21, size=(7, d)).astype(np.float32)
    k = g.integers(-20, 21, size=(9, d)).astype(np.float32)
    qr = F.hadamard_butterfly_f32(q * s.astype(np.float32)).astype(np.float64)
    kr = F.hadamard_butterfly_f32(k * s.astype(np.float32)).astype(np.float64)
    assert np.array_equal(qr @ kr.T, d * (q.astype(np.float64) @ k.astype(np.float64).T))
    # and the normalised transform is orthogonal
    R = np.diag(s) @ scipy.linalg.hadamard(d) / np.sqrt(d)
    assert np.allclose(R @ R.T, np.eye(d), atol=1e-12)


def test_rotation_spreads_an_outlier_coordinate():
    d = 128
    x = np.zeros((1, d), dtype=np.float32)
    x[0, 5] = 100.0
    s = np.ones(d, dtype=np.float32)
    y = F.hadamard_butterfly_f32(x * s)
    assert np.all(np.abs(y) == 100.0)      # one coordinate spread evenly over all d


@pytest.mark.parametrize("amax", [0.0, 1e-30, 2.0 ** -20, 0.3, 1.0, 447.9, 448.0, 448.0001, 896.0, 1e6])
def test_block_exponent_is_the_smallest_that_fits(amax):
    e = F.block_exponent(amax)
    if amax == 0.0:
        assert e == -127
        return
    assert amax / 2.0 ** e <= 448.0
    assert e == -127 or amax / 2.0 ** (e - 1) > 448.0


def test_quantize_blocks_against_brute_force():
    g = np.random.default_rng(4)
    B, N, H, d = 2, 150, 3, 16          # a ragged last block of 22 rows
    x = (g.standard_normal((B, N, H, d)) * np.exp(g.standard_normal((B, 1, H, 1)))).astype(np.float32)
    signs = np.where(g.random(d) < 0.5, -1, 1).astype(np.int8)
    for sg in (None, signs):
        codes, exps = F.quantize_blocks(x, sg)
        assert exps.shape == (B, H, 3)
        y = x.astype(np.float64)
        if sg is not None:
            y = (x * sg.astype(np.float32)).astype(np.float64) @ scipy.linalg.hadamard(d)
        for b in range(B):
            for h in range(H):
                for r in range(3):
                    blk = y[b, 64 * r:64 * (r + 1), h]
                    e = int(exps[b, h, r])
                    # smallest power-of-two scale that keeps the block inside e4m3
                    assert np.abs(blk).max() / 2.0 ** e <= 448.0 < np.abs(blk).max() / 2.0 ** (e - 1)
                    deq = F.e4m3_decode(codes[b, 64 * r:64 * (r + 1), h]) * 2.0 ** e
                    # nearest code: error at most half a step of the e4m3 grid
                    # (2^-4 relative for normal values, 2^-10 * 2^e below)
                    step = np.maximum(np.abs(blk) * 2.0 ** -4, 2.0 ** -10 * 2.0 ** e)
                    assert np.all(np.abs(deq - blk) <= step * (1 + 1e-6))
        deq = F.dequantize_blocks(codes, exps)
        assert deq.shape == x.shape


MUTATIONS = [
    ("decode exponent bias", "2.0 ** (e - 7.0)", "2.0 ** (e - 8.0)"),
    ("decode subnormal scale", "m / 8.0 * 2.0 ** -6", "m / 8.0 * 2.0 ** -7"),
    ("ties away from zero", "((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))", "(d_hi == d_lo)"),
    ("butterfly sign", "y[..., i + h] = a - b", "y[..., i + h] = b - a"),
    ("butterfly pairing", "b = y[..., i + h].copy()", "b = y[..., (i + 2 * h) % d].copy()"),
    ("exponent off by one", "return max(e, -127)", "return max(e + 1, -127)"),
    ("signs ignored", "y = hadamard_butterfly_f32(x * s)", "y = hadamard_butterfly_f32(x)"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistakes_are_caught(name, old, new, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "fp8.py")).read()
    assert src.count(old) == 1, name
    path = tmp_path / "fp8_mut.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("fp8_mut", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    checks = [test_decode_matches_torch_for_every_code, test_encode_ties_go_to_even,
              test_butterfly_is_the_hadamard_product, test_quantize_blocks_against_brute_force,
              test_rotation_multiplies_scores_by_d]
    caught = False
    for chk in checks:
        try:
            chk.__globals__["F"] = mod
            chk()
        except (AssertionError, ValueError):
            caught = True
        finally:
            chk.__globals__["F"] = F
        if caught:
            break
    assert caught, f"planted mistake '{name}' went unnoticed"
