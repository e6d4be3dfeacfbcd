"""Block-scaled e4m3 quantisation with incoherent processing, written out plainly.

TEST INFRASTRUCTURE ONLY: imported by the test suite, never by the GPU
library, and it imports nothing from it.

The second page ("FlashAttention：IO 感知的精确注意力", section 10, lever 3
of FlashAttention-3, and section 12.2) names two precision measures for FP8
attention: quantisation with one scale per block rather than per tensor, and
"incoherent processing", a rotation or permutation that spreads outlier
values over many coordinates before they are quantised.  It gives no block
shape, scale format or rotation.  The readings taken here:

* a block is 64 consecutive rows (sequence positions) of one head, all d
  coordinates;
* a block's scale is a power of two 2^e (the block-scale format the gfx950
  scaled fp8 products take), e the smallest integer with
  max|x| / 2^e <= 448 (the largest finite e4m3 value); a block of zeros
  gets e = -127;
* each element is stored as the e4m3 (OCP E4M3FN) code nearest to x / 2^e,
  ties to the even code;
* the rotation is x -> (x * s) H, with s a vector of d random signs (an
  input) and H the d x d Sylvester-Hadamard matrix, H[i, j] =
  (-1)^popcount(i & j).  H / sqrt(d) and diag(s) are orthogonal, so rotating
  both q and k multiplies every score q.k by exactly d:
  ((q s) H)((k s) H)^T = d q k^T.  It is computed in float32 by the
  radix-2 butterfly network, stage by stage (h = 1, 2, 4, ..., d/2; each
  stage replaces the pair at positions i, i + h, i & h == 0, by (a + b,
  a - b)), the rounding order the GPU uses too, so that both sides reach
  the same float32 values and therefore the same codes.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 64          # rows per quantisation block


def e4m3_decode(codes) -> np.ndarray:
    """Real values (float64) of e4m3 codes (uint8), from the format's
    definition: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
    exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


_POS_CODES = np.arange(0x7F, dtype=np.int64)          # 0x00 .. 0x7e: every finite value >= 0
_POS_VALUES = e4m3_decode(_POS_CODES)                  # increasing


def e4m3_encode(x) -> np.ndarray:
    """The e4m3 code nearest to each value (|x| <= 448), ties to the code
    with an even mantissa: a search over the 127 finite non-negative codes.
    The sign goes to bit 7 (zero keeps code 0x00 or 0x80 with its sign)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(~np.isfinite(a)) or np.any(a > E4M3_MAX):
        raise ValueError("e4m3_encode: value outside the finite e4m3 range")
    hi = np.searchsorted(_POS_VALUES, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def hadamard_butterfly_f32(x) -> np.ndarray:
    """y = x H along the last axis (length a power of two), H the Sylvester
    Hadamard matrix, in float32: the radix-2 butterfly stages in order
    h = 1, 2, 4, ..., each pair (i, i + h) with i & h == 0 becoming
    (x_i + x_{i+h}, x_i - x_{i+h})."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    h = 1
    while h < d:
        idx = np.arange(d)
        i = idx[(idx & h) == 0]
        a = y[..., i].copy()
        b = y[..., i + h].copy()
        y[..., i] = a + b
        y[..., i + h] = a - b
        h *= 2
    return y


def block_exponent(amax: float) -> int:
    """Smallest integer e with amax / 2^e <= 448 (-127 for amax == 0)."""
    if amax == 0.0:
        return -127
    e = int(np.ceil(np.log2(amax / E4M3_MAX)))
    # settle the boundary exactly (log2 is not exact near powers of two)
    while amax / 2.0 ** e > E4M3_MAX:
        e += 1
    while e > -127 and amax / 2.0 ** (e - 1) <= E4M3_MAX:
        e -= 1
    return max(e, -127)


def quantize_blocks(x, signs=None, block: int = BLOCK):
    """Block-scaled e4m3 quantisation of a [B, N, H, d] tensor (float32
    values; bf16 inputs are widened exactly before this is called).

    With `signs` (d values of +-1): the rows are first rotated,
    y = (x * signs) H (hadamard_butterfly_f32); otherwise y = x.  For each
    (b, h) and block of `block` rows (the last one ragged): e =
    block_exponent(max |y|), codes = e4m3_encode(y / 2^e).

    Returns (codes uint8 [B, N, H, d], exps int8 [B, H, ceil(N / block)])."""
    x = np.asarray(x, dtype=np.float32)
    B, N, H, d = x.shape
    if signs is not None:
        s = np.asarray(signs, dtype=np.float32).reshape(d)
        y = hadamard_butterfly_f32(x * s)
    else:
        y = x
    nb = (N + block - 1) // block
    codes = np.zeros((B, N, H, d), dtype=np.uint8)
    exps = np.zeros((B, H, nb), dtype=np.int8)
    for b in range(B):
        for h in range(H):
            for r in range(nb):
                blk = y[b, r * block:(r + 1) * block, h].astype(np.float64)
                e = block_exponent(float(np.abs(blk).max()))
                exps[b, h, r] = e
                codes[b, r * block:(r + 1) * block, h] = e4m3_encode(blk / 2.0 ** e)
    return codes, exps


def dequantize_blocks(codes, exps, block: int = BLOCK) -> np.ndarray:
    """The real values code * 2^e (float64) of a block-quantised tensor."""
    codes = np.asarray(codes)
    B, N, H, d = codes.shape
    e = np.repeat(np.asarray(exps, dtype=np.float64), block, axis=2)[:, :, :N]   # [B, H, N]
    return e4m3_decode(codes) * (2.0 ** e).transpose(0, 2, 1)[..., None]
