"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This module draws inputs and picks sample rows; it holds no attention
arithmetic.  Both the GPU path and the CPU oracle consume what it produces,
so the two always see bit-identical input values.

Recipe (one CPU generator per workload, seeded with ``seed``): q, k, v are
drawn in that order with ``torch.randn`` in float32, q is multiplied by
``q_std`` (4.0 for the peaked long-context case), and the result is rounded
to bf16 (round to nearest even) unless the workload is fp32.  Layout is
[B, N, H, d] contiguous for every tensor (q with the query length, k and v
with the key length).
"""
from __future__ import annotations

import math
import random
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str          # "fp32", "bf16" or "fp8"
    causal: bool
    q_std: float
    seed: int
    Nk: int = 0         # key length; 0 = the query length N
    splits: int = 1     # key ranges (0 = the library's choice)
    mask: str = ""      # block mask pattern ("butterfly"), or dense

    @property
    def Nkv(self) -> int:
        return self.Nk or self.N

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def pairs(self) -> float:
        """(query, key) pairs per head the FLOP count credits.

        Equal lengths: N^2, halved when causal (the conventional count).
        Unequal lengths: the exact number of visible pairs (bottom-right
        causal alignment)."""
        Nq, Nk = self.N, self.Nkv
        if Nq == Nk:
            return Nq * Nq / 2 if self.causal else float(Nq * Nq)
        if not self.causal:
            return float(Nq * Nk)
        off = Nk - Nq
        lo = max(0, -off)                        # first row that sees a key
        full = max(lo, min(Nq, Nk - off))        # rows from here on see all Nk keys (off >= 0 case)
        tri = sum(range(lo + off + 1, full + off + 1)) if full > lo else 0
        return float(tri + (Nq - full) * Nk)

    @property
    def flops(self) -> float:
        """4*d FLOPs per credited (query, key) pair per head and batch entry
        (with a block mask: the pairs it keeps)."""
        if self.mask:
            return 4.0 * self.B * self.d * mask_kept_pairs(self.block_mask(), self.N, self.causal)
        return 4.0 * self.B * self.Hq * self.pairs * self.d

    def block_mask(self):
        if self.mask == "butterfly":
            return butterfly_mask(self.Hq, self.N)
        raise ValueError(self.mask)

    @property
    def io_bytes(self) -> int:
        """Bytes the forward must move at least once: q, k, v read, o and lse written
        (fp8: one-byte inputs, bf16 output)."""
        s_in = {"fp32": 4, "fp8": 1, "fp8blk": 1}.get(self.dtype, 2)
        s_out = 4 if self.dtype == "fp32" else 2
        return ((self.Hq * self.N * (s_in + s_out) + 2 * self.Hkv * self.Nkv * s_in) * self.B * self.d
                + 4 * self.B * self.Hq * self.N)


# The five workloads: a tiny fp32 single head, bf16 MHA at d=64, the headline
# causal d=128 case, a long-context case with peaked logits, and causal GQA.
WORKLOADS = {
    "single_head_fp32_N256_d64": Workload("single_head_fp32_N256_d64", 1, 1, 1, 256, 64, "fp32", False, 1.0, 1001),
    "mha_bf16_B4_H16_N2048_d64": Workload("mha_bf16_B4_H16_N2048_d64", 4, 16, 16, 2048, 64, "bf16", False, 1.0, 1002),
    "causal_bf16_B2_H32_N4096_d128": Workload("causal_bf16_B2_H32_N4096_d128", 2, 32, 32, 4096, 128, "bf16", True, 1.0, 1003),
    "causal_bf16_B1_H32_N16384_d128_qstd4": Workload("causal_bf16_B1_H32_N16384_d128_qstd4", 1, 32, 32, 16384, 128, "bf16", True, 4.0, 1004),
    "gqa_causal_bf16_B1_Hq32_Hkv8_N32768_d128": Workload("gqa_causal_bf16_B1_Hq32_Hkv8_N32768_d128", 1, 32, 8, 32768, 128, "bf16", True, 1.0, 1005),
}
ORDER = list(WORKLOADS)
HEADLINE = "causal_bf16_B2_H32_N4096_d128"

# Split-key workloads (query length != key length), on the head shape of the
# grouped-query case: one decoding step (one query row per head against a
# 32K-key cache; the query sees every key under the bottom-right causal
# alignment) and a chunked prefill (1024 new queries against 16K keys).
SPLIT_WORKLOADS = {
    "decode_bf16_B1_Hq32_Hkv8_Nk32768_d128": Workload(
        "decode_bf16_B1_Hq32_Hkv8_Nk32768_d128", 1, 32, 8, 1, 128, "bf16", True, 1.0, 1006, Nk=32768, splits=0),
    "chunk_causal_bf16_B1_H32_Nq1024_Nk16384_d128": Workload(
        "chunk_causal_bf16_B1_H32_Nq1024_Nk16384_d128", 1, 32, 32, 1024, 128, "bf16", True, 1.0, 1007,
        Nk=16384, splits=0),
}
# fp8 (e4m3) inputs with one dequantisation factor per (batch, head), on the
# headline shape.
FP8_WORKLOADS = {
    "causal_fp8_B2_H32_N4096_d128": Workload(
        "causal_fp8_B2_H32_N4096_d128", 2, 32, 32, 4096, 128, "fp8", True, 1.0, 1008),
    # the same shape with block-scaled e4m3 inputs: the seeded bf16 draws of
    # gen_inputs, with q and k rotated by random_signs(128, seed)
    "causal_fp8blk_B2_H32_N4096_d128": Workload(
        "causal_fp8blk_B2_H32_N4096_d128", 2, 32, 32, 4096, 128, "fp8blk", True, 1.0, 1011),
}
# Head dimension 256 (the FLOP count of the headline case, half the heads).
D256_WORKLOADS = {
    "causal_bf16_B2_H16_N4096_d256": Workload(
        "causal_bf16_B2_H16_N4096_d256", 2, 16, 16, 4096, 256, "bf16", True, 1.0, 1009),
}
# Block-sparse: a butterfly pattern over 128 x 128 blocks (the sparsity form
# the first page names for block-sparse FlashAttention): block row a keeps
# key block c iff a == c or a xor c is a power of two; 8 of 128 blocks at
# N = 16384, the FLOPs of the headline case.
SPARSE_WORKLOADS = {
    "butterfly_bf16_B1_H32_N16384_d128": Workload(
        "butterfly_bf16_B1_H32_N16384_d128", 1, 32, 32, 16384, 128, "bf16", False, 1.0, 1010, mask="butterfly"),
}
# fp32 inputs and outputs at scale (the accuracy path): the headline shape,
# and a split call of 256 new queries against a 64K-key context.
FP32_WORKLOADS = {
    "causal_fp32_B2_H32_N4096_d128": Workload(
        "causal_fp32_B2_H32_N4096_d128", 2, 32, 32, 4096, 128, "fp32", True, 1.0, 1012),
    "chunk_causal_fp32_B1_H8_Nq256_Nk65536_d128": Workload(
        "chunk_causal_fp32_B1_H8_Nq256_Nk65536_d128", 1, 8, 8, 256, 128, "fp32", True, 1.0, 1013,
        Nk=65536, splits=0),
}
ALL_WORKLOADS = {**WORKLOADS, **SPLIT_WORKLOADS, **FP8_WORKLOADS, **D256_WORKLOADS, **SPARSE_WORKLOADS,
                 **FP32_WORKLOADS}
MASK_BLOCK = (128, 64)      # query rows x keys per block-mask entry of the GPU library


def butterfly_mask(Hq: int, N: int) -> torch.Tensor:
    """uint8 block mask [Hq, ceil(N/128), ceil(N/64)] of the butterfly pattern
    over 128 x 128 blocks (each 128-key block is two 64-key mask columns)."""
    nb = -(-N // 128)
    a = torch.arange(nb)[:, None]
    c = torch.arange(nb)[None, :]
    x = a ^ c
    keep = (x == 0) | ((x & (x - 1)) == 0)
    m = keep.repeat_interleave(2, dim=1)[:, : -(-N // 64)]
    return m.to(torch.uint8).unsqueeze(0).expand(Hq, -1, -1).contiguous()


def random_block_mask(Hq: int, N: int, density: float, seed: int) -> torch.Tensor:
    """uint8 block mask [Hq, ceil(N/128), ceil(N/64)] with entries kept with
    probability `density` (seeded)."""
    g = torch.Generator().manual_seed(seed)
    shape = (Hq, -(-N // 128), -(-N // 64))
    return (torch.rand(shape, generator=g) < density).to(torch.uint8).contiguous()


def mask_kept_pairs(mask: torch.Tensor, N: int, causal: bool) -> float:
    """(query, key) pairs a block mask keeps, summed over heads (causal rule included)."""
    if not causal:   # block extents times kept entries
        rows = torch.clamp(N - 128 * torch.arange(mask.shape[1]), max=128).to(torch.float64)
        keys = torch.clamp(N - 64 * torch.arange(mask.shape[2]), max=64).to(torch.float64)
        return float((mask.to(torch.float64) * rows[None, :, None] * keys[None, None, :]).sum())
    m = mask.to(torch.bool).repeat_interleave(128, dim=1)[:, :N].repeat_interleave(64, dim=2)[:, :, :N]
    m = m & torch.ones(N, N, dtype=torch.bool).tril()
    return float(m.sum())


def make(B, Hq, Hkv, N, d, dtype="bf16", causal=False, q_std=1.0, seed=0, name="custom", Nk=0,
         splits=1) -> Workload:
    return Workload(name, B, Hq, Hkv, N, d, dtype, causal, q_std, seed, Nk, splits)


def gen_inputs(w: Workload):
    """(q, k, v) on the host, drawn as described in the module docstring."""
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    q = torch.randn((w.B, w.N, w.Hq, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.Nkv, w.Hkv, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.Nkv, w.Hkv, w.d), generator=g, dtype=torch.float32)
    if w.q_std != 1.0:
        q = q * w.q_std
    if w.dtype in ("bf16", "fp8blk"):     # fp8blk: the bf16 values its quantiser starts from
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    elif w.dtype != "fp32":
        raise ValueError(w.dtype)
    return q.contiguous(), k.contiguous(), v.contiguous()


def quantize_fp8(x: torch.Tensor):
    """Per-(batch, head) e4m3 quantisation of a float [B, N, H, d] tensor.

    descale = amax / 440 over each (b, h) slice (a little headroom below the
    format's 448), codes = round-to-nearest-even e4m3 of x / descale.  Returns
    (codes as torch.float8_e4m3fn [B, N, H, d], descale float32 [B, H])."""
    amax = x.abs().amax(dim=(1, 3)).clamp(min=1e-12)          # [B, H]
    descale = (amax / 440.0).to(torch.float32)
    codes = (x / descale[:, None, :, None]).to(torch.float8_e4m3fn)
    return codes.contiguous(), descale.contiguous()


def gen_inputs_fp8(w: Workload):
    """fp8 workload inputs: the same seeded randn draws as gen_inputs, then
    quantize_fp8 on each of q, k, v.  Returns (q8, k8, v8, q_descale,
    k_descale, v_descale)."""
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    q = torch.randn((w.B, w.N, w.Hq, w.d), generator=g, dtype=torch.float32) * w.q_std
    k = torch.randn((w.B, w.Nkv, w.Hkv, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.Nkv, w.Hkv, w.d), generator=g, dtype=torch.float32)
    (q8, qd), (k8, kd), (v8, vd) = quantize_fp8(q), quantize_fp8(k), quantize_fp8(v)
    return q8, k8, v8, qd, kd, vd


def dequantize_fp8(codes: torch.Tensor, descale: torch.Tensor) -> torch.Tensor:
    """The real values code * descale as float32 [B, N, H, d] (the e4m3 code
    widens exactly; the product is rounded once to float32)."""
    return (codes.to(torch.float32) * descale[:, None, :, None]).contiguous()


QUANT_BLOCK = 64    # rows per block of the block-scaled fp8 format


def random_signs(d: int, seed: int) -> torch.Tensor:
    """d random signs (+1 / -1, int8) for the rotation of the block-scaled fp8
    path, from a CPU generator seeded with ``seed``."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randint(0, 2, (d,), generator=g, dtype=torch.int8) * 2 - 1).contiguous()


def random_block_codes(B: int, N: int, H: int, d: int, seed: int, exp_range=(-3, 3)):
    """Seeded block-scaled fp8 inputs: e4m3 codes of randn values (uint8
    [B, N, H, d]) and one exponent per 64 rows of a head (int8
    [B, H, ceil(N / 64)], uniform in exp_range).  The real values are
    code * 2^exp."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    codes = torch.randn((B, N, H, d), generator=g).to(torch.float8_e4m3fn).view(torch.uint8)
    nb = (N + QUANT_BLOCK - 1) // QUANT_BLOCK
    exps = torch.randint(exp_range[0], exp_range[1] + 1, (B, H, nb), generator=g, dtype=torch.int8)
    return codes.contiguous(), exps.contiguous()


def outlier_inputs(B: int, N: int, Hq: int, Hkv: int, d: int, seed: int, channels: int = 2,
                   channel_gain: float = 30.0, shared_channels: bool = True, rare: float = 0.0,
                   growth: float = 0.0):
    """bf16 q, k, v [B, N, H, d]: randn values with the structure that makes
    low-precision attention hard, each part optional:
    * outlier channels: ``channels`` of the d coordinates of q and k
      multiplied by ``channel_gain`` in every row, the same coordinates in q
      and k when ``shared_channels``, else drawn separately;
    * rare outliers: each element of q, k and v gains an extra
      N(0, 10^2) draw with probability ``rare``;
    * growth along the sequence: 64-row block r of q, k and v multiplied by
      2^(growth * (r - last block)), so the first blocks are the smallest."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((B, N, Hq, d), generator=g)
    k = torch.randn((B, N, Hkv, d), generator=g)
    v = torch.randn((B, N, Hkv, d), generator=g)
    if channels:
        cq = torch.randperm(d, generator=g)[:channels]
        ck = cq if shared_channels else torch.randperm(d, generator=g)[:channels]
        q[..., cq] *= channel_gain
        k[..., ck] *= channel_gain
    if rare:
        q, k, v = (t + (torch.rand(t.shape, generator=g) < rare) * torch.randn(t.shape, generator=g) * 10
                   for t in (q, k, v))
    if growth:
        nb = (N + QUANT_BLOCK - 1) // QUANT_BLOCK
        f = torch.repeat_interleave(2.0 ** (growth * (torch.arange(nb) - (nb - 1))), QUANT_BLOCK)[:N]
        q, k, v = (t * f[None, :, None, None] for t in (q, k, v))
    return tuple(t.to(torch.bfloat16).contiguous() for t in (q, k, v))


def sample_rows(w: Workload, per_head: int = 512, seed: int | None = None):
    """Query rows to check, as (b, h, i) triples.

    Per (b, h): rows 0, 1, 2, 3, N-2, N-1, then uniform draws without
    replacement until ``per_head`` rows (all rows when N <= per_head), from
    ``random.Random(seed * 1_000_003 + b * Hq + h)``.
    """
    seed = w.seed if seed is None else seed
    out = []
    for b in range(w.B):
        for h in range(w.Hq):
            if w.N <= per_head:
                rows = list(range(w.N))
            else:
                fixed = [0, 1, 2, 3, w.N - 2, w.N - 1]
                rng = random.Random(seed * 1_000_003 + b * w.Hq + h)
                rest = [i for i in rng.sample(range(4, w.N - 2), per_head - len(fixed))]
                rows = sorted(set(fixed + rest))
            out.extend((b, h, i) for i in rows)
    return out
