"""Helpers for the GPU parity tests: run the HIP path, run the oracle on the
same host values, compare at the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import exact_attention_93_amd as fa
import oracle
from tests.fwd_bound import fwd_intervals

# bf16 I/O with fp32 accumulation: max |o - ref| <= 1e-2 and mean <= 1e-3.
# fp32 I/O: max |o - ref| <= 1e-5.  LSE: |lse - ref| <= 1e-4 * max(1, |ref|).
TOL = {"bf16": (1e-2, 1e-3), "fp32": (1e-5, 1e-6)}
LSE_REL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_fwd(q, k, v, causal, scale, num_splits=1):
    """q, k, v: host tensors.  Returns host (o, lse) from libfa.so."""
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def compare(q, k, v, causal, scale, o, lse, rows=None, kind=None, label="", exact_bounds=False,
            block_mask=None, num_splits=None):
    """Compare GPU outputs o [B,N,Hq,d], lse [B,Hq,N] with the oracle on rows.

    Every element and log-sum-exp must lie in its interval derived from the
    forward's arithmetic (tests/fwd_bound.py; num_splits as passed to the
    library, None when unknown, which takes the bound that covers a merge of
    key ranges).  Besides, exact_bounds=True applies the stated bounds
    verbatim (the named workloads).  Otherwise (small shapes, where few keys
    per row leave |O| near 1) the bf16 mean bound also admits the output
    format's own mean rounding error, ulp(ref)/4, on top of 1e-3.
    """
    kind = kind or ("fp32" if q.dtype == torch.float32 else "bf16")
    if block_mask is None:
        ro, rl = oracle.attention(q, k, v, scale, causal, rows=rows)
    else:   # 128 query rows x 64 keys per mask entry, as the GPU library reads it
        ro, rl = oracle.attention(q, k, v, scale, causal, rows=rows, block_mask=block_mask, block=(128, 64))
    B, N, Hq, d = q.shape
    if rows is None:
        go = o.float().numpy().transpose(0, 2, 1, 3).reshape(-1, d).astype(np.float64)
        gl = lse.numpy().reshape(-1).astype(np.float64)
    else:
        r = np.asarray(rows)
        go = o.float().numpy()[r[:, 0], r[:, 2], r[:, 1]].astype(np.float64)
        gl = lse.numpy()[r[:, 0], r[:, 1], r[:, 2]].astype(np.float64)
    check_intervals(q, k, v, causal, scale, go, gl, rows, kind, label, block_mask, num_splits)
    # rows that see no key: O exactly 0 and lse exactly -inf on both sides
    empty = np.isneginf(rl)
    if empty.any():
        say(f"[parity] {label}: {int(empty.sum())} row(s) without visible keys")
        assert np.all(np.isneginf(gl[empty])), "a row without keys must have lse = -inf"
        assert np.all(go[empty] == 0.0), "a row without keys must have a zero output"
    gl = np.where(empty, 0.0, gl)
    rl = np.where(empty, 0.0, rl)
    err = np.abs(go - ro)
    lerr = np.abs(gl - rl) / np.maximum(1.0, np.abs(rl))
    mx, mean, lmx = float(err.max()), float(err.mean()), float(lerr.max())
    at = np.unravel_index(int(np.argmax(err)), err.shape)
    say(f"[parity] {label} kind={kind} rows={len(rl)} max|dO|={mx:.3e} (ref {ro[at]:.5f} got {go[at]:.5f} "
        f"at row {at[0]} col {at[1]}) mean|dO|={mean:.3e} max rel dLSE={lmx:.3e}")
    tmax, tmean = TOL[kind]
    if kind == "fp32" and not exact_bounds:
        # Off the unit-variance workload the fp32 rounding of the scores
        # themselves can exceed 1e-5 (peaked logits): the bound becomes twice
        # the error of a plain fp32 evaluation of the same definition.
        pe = plain_fp32_error(q, k, v, causal, scale, ro, rows, block_mask)
        tmax, tmean = max(tmax, 2 * pe[0]), max(tmean, 2 * pe[1])
        say(f"[parity] {label}: plain fp32 evaluation error max {pe[0]:.3e} mean {pe[1]:.3e}")
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl)), "non-finite output"
    if kind == "bf16":
        # An element whose exact value has |ref| >= 4 is held to half a bf16
        # ulp of ref plus 1e-3 instead (the output format alone can miss 1e-2
        # there); every other element to the 1e-2 bound.  Counted and reported.
        big = np.abs(ro) >= 4.0
        half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ro), 1e-30))) - 8)
        limited = big & (err > tmax) & (err <= half_ulp + 1e-3)
        if limited.any():
            say(f"[parity] {label}: {int(limited.sum())} rounding-limited element(s) with |ref| >= 4")
        err = np.where(limited, 0.0, err)
        mx = float(err.max())
    assert mx <= tmax, f"max |dO| {mx} > {tmax}"
    if kind == "bf16" and not exact_bounds:
        tmean = tmean + float(np.mean(np.exp2(np.floor(np.log2(np.maximum(np.abs(ro), 2.0 ** -126))) - 7) / 4))
    assert mean <= tmean, f"mean |dO| {mean} > {tmean}"
    assert lmx <= LSE_REL, f"LSE error {lmx} > {LSE_REL}"
    return mx, mean, lmx


def key_ranges(q, k, num_splits):
    """(merged, keys per range at most) of a forward call with this
    num_splits: whether it merges several key ranges, and a bound on the
    length of each (None: unknown, taken as a merge of ranges of any
    length).  The library cuts the keys into ranges of a multiple of 64,
    never more ranges than requested, so a range holds at most
    ceil(ceil(Nk / 64) / nsplit) * 64 keys."""
    if num_splits is None:
        return True, None
    if num_splits == 1:
        return False, None
    B, Nq, Hq, d = q.shape
    Nk = k.shape[1]
    nsplit = fa.fa_splitkv_num_splits(B, Hq, k.shape[2], Nq, Nk, d, num_splits)
    if nsplit <= 1:
        return False, None
    return True, -(-(-(-Nk // 64)) // nsplit) * 64


def check_intervals(q, k, v, causal, scale, go, gl, rows, kind, label, block_mask=None, num_splits=None):
    """Every output element go [R, d] and log-sum-exp gl [R] (fp64, in the
    order of rows; None = every row) inside its interval from
    tests/fwd_bound.py."""
    B, N, Hq, d = q.shape
    if rows is None:
        rows = np.array([(b, h, i) for b in range(B) for h in range(Hq) for i in range(N)], dtype=np.int32)
    split, range_keys = key_ranges(q, k, num_splits)
    lo, hi, llo, lhi = fwd_intervals(q, k, v, scale, causal, rows, kind, block_mask=block_mask, split=split,
                                     range_keys=range_keys)
    assert np.all(np.isfinite(lo)) and np.all(np.isfinite(hi)) and np.all(lo <= hi), \
        f"{label}: the derived intervals degenerate (the bound does not hold at this size)"
    bad = (go < lo) | (go > hi)
    radius = (hi - lo) / 2
    say(f"[parity] {label}: derived intervals ({'with' if split else 'without'} a merge) median half-width "
        f"{np.median(radius):.2e} max {radius.max():.2e}")
    if bad.any():
        r, x = np.argwhere(bad)[0]
        raise AssertionError(f"{label}: {int(bad.sum())} output element(s) outside their derived interval, first "
                             f"row {tuple(np.asarray(rows)[r])} col {x}: {go[r, x]!r} not in [{lo[r, x]!r}, {hi[r, x]!r}]")
    fin = np.isfinite(llo)
    assert np.array_equal(fin, np.isfinite(gl)), f"{label}: rows without keys differ from the derived ones"
    lbad = (gl[fin] < llo[fin]) | (gl[fin] > lhi[fin])
    if lbad.any():
        i = np.nonzero(fin)[0][np.argmax(lbad)]
        raise AssertionError(f"{label}: {int(lbad.sum())} lse value(s) outside their derived interval, first "
                             f"row {tuple(np.asarray(rows)[i])}: {gl[i]!r} not in [{llo[i]!r}, {lhi[i]!r}]")


def plain_fp32_error(q, k, v, causal, scale, ro, rows, block_mask=None):
    """Error of softmax(scale Q K^T) V evaluated in float32 on the CPU (torch),
    against the fp64 oracle values ro; (max, mean)."""
    B, N, Hq, d = q.shape
    Nk = k.shape[1]
    g = Hq // k.shape[2]
    qt = q.float().permute(0, 2, 1, 3)
    kt = k.float().repeat_interleave(g, dim=2).permute(0, 2, 3, 1).contiguous()
    vt = v.float().repeat_interleave(g, dim=2).permute(0, 2, 1, 3).contiguous()
    s = torch.matmul(qt, kt) * np.float32(scale)
    if causal:   # bottom-right alignment: key j kept iff j - i <= Nk - N
        s = s.masked_fill(~torch.ones(N, Nk, dtype=torch.bool).tril(Nk - N), float("-inf"))
    if block_mask is not None:
        keep = torch.as_tensor(block_mask).to(torch.bool).repeat_interleave(128, dim=1)[:, :N]
        keep = keep.repeat_interleave(64, dim=2)[:, :, :Nk]
        s = s.masked_fill(~keep[None], float("-inf"))
    o = torch.nan_to_num(torch.matmul(torch.softmax(s, dim=-1), vt), nan=0.0)   # [B, Hq, N, d]
    if rows is None:
        o = o.reshape(-1, d)
    else:
        r = np.asarray(rows)
        o = o[r[:, 0], r[:, 1], r[:, 2]]
    e = np.abs(o.double().numpy() - ro)
    return float(e.max()), float(e.mean())


def rand_inputs(B, N, Hq, Hkv, d, dtype, seed, q_std=1.0, Nk=None):
    Nk = N if Nk is None else Nk
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, N, Hq, d), generator=g) * q_std
    k = torch.randn((B, Nk, Hkv, d), generator=g)
    v = torch.randn((B, Nk, Hkv, d), generator=g)
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    return q.to(dt).contiguous(), k.to(dt).contiguous(), v.to(dt).contiguous()
