#!/usr/bin/env python3
"""Benchmark of the exact attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of fa_fwd (the whole hot path) over the headline workload:
causal attention, B=2, H=32, N=4096, d=128, bf16 inputs and output, fp32
accumulation, synthetic inputs already resident in HBM.  W untimed warm-up
steps, continued until at least WARMUP_FLOOR_S seconds of back-to-back steps
have run (the number actually run is reported), then exactly K steps between
a synchronisation on each side, timed with one pair of events on the stream
the kernel runs on (one before the first step, one after the last; the spread
of single steps comes from a separate pass afterwards).  One JSON line is
printed.

value = conventional FLOPs (4*B*H*N^2*d, halved for causal) / mean step time.
roofline: achieved = the same FLOPs per launch / mean launch duration, against
the dense bf16 matrix-core peak of MI355X (2.5 PFLOP/s, i.e. 2516.6 TFLOP/s
at 2.4 GHz); traffic = HBM bytes per launch from the committed rocprofv3
counter summary, used only while the kernel sources still hash to the value
recorded there (else null).
cpu_baseline: the fp64 CPU oracle, timed on this host's cores over a bounded
sample of the same workload's query rows, in the same unit.

--pass bwd times the backward instead (one fa_bwd call per step, the
forward's o and lse computed once before timing, dO seeded randn), with the
conventional backward count of 2.5x the forward FLOPs.

--workload picks another named workload.  The split-key ones (unequal query
and key lengths) run fa_fwd_splitkv, whose step is two launches (the
split forward and the merge) with the workspace allocated before timing; a
workload whose FLOPs per algorithmic byte fall below the machine balance
(2.5 PFLOP/s / 8 TB/s) is reported in GB/s of algorithmic bytes against the
HBM peak instead.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s at N=4096,d=128 causal bf16; % of dense bf16 MFMA peak"
# MI355X dense matrix-core peaks (published "2.5 PFLOP/s" bf16 and "5 PFLOP/s"
# fp8, written out exactly: 256 CUs x 2048 bf16 FMA per clock x 2 x 2.4 GHz).
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP8_TFLOPS = 5033.2
PEAK_FP32_TFLOPS = 157.3        # dense fp32 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak bandwidth (published)
# Untimed back-to-back steps run for at least this long before the timed
# region, whatever --warmup asks for: the GPU's clock needs tens of
# milliseconds of load to settle (the headline step takes ~350 us on the first
# launches and ~272 us from about the hundredth on).  The steps actually run
# are reported in the JSON line.
WARMUP_FLOOR_S = 0.5
PROFILES = os.path.join(ROOT, "profiles")


def kernel_sources(w, bwd: bool):
    """The sources a workload's launches depend on: the kernels it runs, the
    shared internal header, the C-ABI layer and the public header."""
    if bwd:
        kern = ["fa_bwd_bf16.hip"]
    elif w.dtype in ("fp8", "fp8blk"):
        kern = ["fa_fwd_fp8.hip"]
    elif w.dtype == "fp32":
        kern = ["fa_fwd_f32.hip", "fa_combine.hip"]
    elif w.N * (w.Hq // w.Hkv) <= 64:          # the decoding kernel's shapes
        kern = ["fa_decode_bf16.hip", "fa_combine.hip"]
    else:
        kern = ["fa_fwd_bf16.hip", "fa_combine.hip"]
    return kern + ["fa_internal.h", "fa_api.cpp"]


def kernel_source_hash(names) -> str:
    """sha256 over the named sources and the public header."""
    from exact_attention_93_amd import _build
    h = hashlib.sha256()
    for path in [os.path.join(_build.CSRC, n) for n in names] + [os.path.join(ROOT, "include", "fa.h")]:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_file(w, bwd: bool):
    """The committed counter summary for this workload, if one is kept."""
    from exact_attention_93_amd import workloads as W
    if bwd:   # both kernels of the step (dq, then dk/dv)
        return os.path.join(PROFILES, f"fa_bwd_bf16_{w.name}_traffic.txt")
    if w.name.startswith("decode_"):
        return os.path.join(PROFILES, f"fa_decode_bf16_{w.name}_traffic.txt")
    kern = {"fp8": "fwd_fp8", "fp8blk": "fwd_fp8", "fp32": "fwd_f32"}.get(w.dtype, "fwd_bf16")
    return os.path.join(PROFILES, f"fa_{kern}_{w.name}_traffic.txt")


def read_traffic(path, src_hash):
    """HBM bytes per launch from a committed counter summary taken with the
    same sources (hash), or None."""
    if path is None or not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != src_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def visible_keys(w, i):
    """Keys query row i sees (bottom-right causal alignment), as an array."""
    import numpy as np
    if not w.causal:
        return np.full(len(i), w.Nkv)
    return np.clip(i + (w.Nkv - w.N) + 1, 0, w.Nkv)


def cpu_baseline(w, seconds: float, hbm: bool):
    """Time the fp64 oracle on the workload's sampled query rows."""
    import numpy as np
    import oracle
    from exact_attention_93_amd import workloads as W

    scale = w.scale
    if w.dtype == "fp8":
        q8, k8, v8, qd, kd, vd = W.gen_inputs_fp8(w)
        q, k, v = W.dequantize_fp8(q8, qd), W.dequantize_fp8(k8, kd), W.dequantize_fp8(v8, vd)
    elif w.dtype == "fp8blk":
        # the oracle's block quantiser (q and k rotated), then the real values
        import torch
        from oracle import fp8 as F
        qb, kb, vb = W.gen_inputs(w)
        signs = W.random_signs(w.d, w.seed).numpy()
        deq = lambda x, sg: torch.from_numpy(F.dequantize_blocks(*F.quantize_blocks(x.float().numpy(), sg))
                                             .astype(np.float32))
        q, k, v = deq(qb, signs), deq(kb, signs), deq(vb, None)
        scale = w.scale / w.d
    else:
        q, k, v = W.gen_inputs(w)
    bb, hh, ii = np.meshgrid(np.arange(w.B), np.arange(w.Hq), np.arange(w.N), indexing="ij")
    rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)   # every query row
    threads = oracle.host_threads()
    # calibrate on 1024 evenly strided rows, then size the sample to about
    # `seconds` (every row when the whole workload fits)
    mk = {}
    if w.mask:
        mk = {"block_mask": w.block_mask(), "block": (128, 64)}
    probe = rows[np.linspace(0, len(rows) - 1, min(1024, len(rows))).astype(int)]
    t0 = time.perf_counter()
    oracle.attention(q, k, v, scale, w.causal, rows=probe, threads=threads, **mk)
    dt = max(time.perf_counter() - t0, 1e-3)
    n = int(min(len(rows), max(len(probe), len(probe) * seconds / dt)))
    pick = rows[np.linspace(0, len(rows) - 1, n).astype(int)]
    t0 = time.perf_counter()
    oracle.attention(q, k, v, scale, w.causal, rows=pick, threads=threads, **mk)
    dt = time.perf_counter() - t0
    sample = (f"all {n} query rows of {w.name}" if n == len(rows) else
              f"{n} of the {len(rows)} query rows of {w.name}, evenly strided over (b, h, i)")

    def work(sel):
        """The sample's work in the metric's unit: bytes (its share of the
        workload's algorithmic bytes) or FLOPs (4*d per visible key)."""
        if hbm:
            return w.io_bytes * len(sel) / len(rows)
        if w.mask:   # kept keys of each sampled row (non-causal block masks)
            m = mk["block_mask"].numpy().astype(np.float64)
            keys = np.minimum(w.N - 64 * np.arange(m.shape[2]), 64).astype(np.float64)
            vis = m[sel[:, 1], sel[:, 2] // 128] @ keys
        else:
            vis = visible_keys(w, sel[:, 2])
        return float(4.0 * w.d * vis.sum())

    # The same oracle on one thread, over every `threads`-th row of the sample.
    one = pick[::threads]
    t0 = time.perf_counter()
    oracle.attention(q, k, v, scale, w.causal, rows=one, threads=1, **mk)
    dt1 = time.perf_counter() - t0
    scale_unit, unit = (1e9, "GB/s") if hbm else (1e12, "TFLOP/s")
    what = ("bytes counted as the sample's share of the workload's algorithmic bytes" if hbm
            else "FLOPs counted as 4*d per visible key")
    return {
        "value": work(pick) / dt / scale_unit, "unit": unit, "cores": threads, "kind": "oracle",
        "sample": sample + f"; fp64 3-pass oracle, {dt:.1f} s wall; {what}",
        "single_thread": {"value": work(one) / dt1 / scale_unit, "unit": unit, "cores": 1,
                          "sample": f"{len(one)} of those rows (every {threads}th), {dt1:.1f} s wall"},
    }


def cpu_baseline_bwd(w, seconds: float, do):
    """Time the fp64 backward oracle on whole (batch, K/V head) groups."""
    import oracle
    from exact_attention_93_amd import workloads as W

    q, k, v = W.gen_inputs(w)
    threads = oracle.host_threads()
    groups = [(b, hk) for b in range(w.B) for hk in range(w.Hkv)]
    t0 = time.perf_counter()
    oracle.attention_bwd(q, k, v, do, w.scale, w.causal, groups=groups[:1], threads=threads)
    dt = max(time.perf_counter() - t0, 1e-3)
    n = int(min(len(groups), max(1, seconds / dt)))
    pick = groups[:: max(1, len(groups) // n)][:n]
    t0 = time.perf_counter()
    oracle.attention_bwd(q, k, v, do, w.scale, w.causal, groups=pick, threads=threads)
    dt = time.perf_counter() - t0
    flops = 2.5 * w.flops * len(pick) / len(groups)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(pick)} of the {len(groups)} (batch, K/V head) groups of {w.name} (every gradient "
                      f"element of those heads); fp64 backward oracle, {dt:.1f} s wall; FLOPs counted as the "
                      "groups' share of 2.5x the forward count"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline case)")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward (default) or the backward")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time for cpu_baseline (0: skip)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain copy of this many MiB (counter calibration runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the benchmark runs on one GPU only; --gpus must be 1 "
              "(the forward would shard by (batch, head) with no exchange)", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_93_amd as fa
    from exact_attention_93_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    fa.load_library()   # fails loudly if libfa.so is missing

    w = W.ALL_WORKLOADS[args.workload or W.HEADLINE]
    dev = torch.device("cuda:0")
    fp8 = w.dtype in ("fp8", "fp8blk")
    fp8blk = w.dtype == "fp8blk"
    if fp8blk:
        # block-scaled e4m3 inputs from the library's own quantiser (q and k rotated)
        qb, kb, vb = (t.to(dev) for t in W.gen_inputs(w))
        signs = W.random_signs(w.d, w.seed).to(dev)
        (q, qd), (k, kd) = fa.quantize_fp8(qb, signs), fa.quantize_fp8(kb, signs)
        v, vd = fa.quantize_fp8(vb, None)
        o = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=dev)
    elif fp8:
        q, k, v, qd, kd, vd = (t.to(dev) for t in W.gen_inputs_fp8(w))
        o = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=dev)
    else:
        q, k, v = (t.to(dev) for t in W.gen_inputs(w))
        o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    splits = fa.fa_splitkv_num_splits(w.B, w.Hq, w.Hkv, w.N, w.Nkv, w.d, w.splits)
    if splits < 1:
        raise SystemExit(f"bench.py: invalid split arguments for {w.name}")
    ws_bytes = fa.fa_splitkv_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.Nkv, w.d, w.splits)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev) if ws_bytes else None
    fp32 = w.dtype == "fp32"
    peak_mfma = PEAK_FP8_TFLOPS if fp8 else PEAK_FP32_TFLOPS if fp32 else PEAK_BF16_TFLOPS
    hbm_bound = w.flops / w.io_bytes < peak_mfma / PEAK_HBM_GBS * 1e3

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        print(f"# calibration copy: {args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB written per neg kernel",
              file=sys.stderr, flush=True)

    bwd = args.which == "bwd"
    if bwd:
        if w.dtype != "bf16":
            raise SystemExit("bench.py: the backward runs on bf16 workloads only")
        g = torch.Generator(device="cpu").manual_seed(w.seed + 50)
        do_host = torch.randn(tuple(q.shape), generator=g).to(torch.bfloat16)
        do = do_host.to(dev)
        fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream,
               num_splits=w.splits, workspace=ws)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.Hq, w.N), dtype=torch.uint8, device=dev)
        hbm_bound = False

    sparse = bool(w.mask)
    if sparse:
        bmask = w.block_mask().to(dev)

    # One call through the Python binding validates the arguments; the timed
    # steps then call the C entry point directly with the same, pre-marshalled
    # arguments (one ctypes call per step), so that the host keeps ahead of
    # short steps such as the decode step.
    lib = fa.load_library()
    sp = stream.cuda_stream
    ptr = lambda t: t.data_ptr()
    if sparse:
        fa.fwd_blocksparse(q, k, v, bmask, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)
        entry, cargs = lib.fa_fwd_blocksparse, (ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), w.B, w.Hq, w.Hkv, w.N,
                                                w.d, w.scale, int(w.causal), ptr(bmask), sp)
    elif fp8blk:
        fa.fwd_fp8_block(q, k, v, qd, kd, vd, causal=w.causal, scale=w.scale / w.d, out=o, lse=lse, stream=stream)
        entry, cargs = lib.fa_fwd_fp8_block, (ptr(q), ptr(k), ptr(v), ptr(qd), ptr(kd), ptr(vd), ptr(o), ptr(lse),
                                              w.B, w.Hq, w.Hkv, w.N, w.d, w.scale / w.d, int(w.causal), sp)
    elif fp8:
        fa.fwd_fp8(q, k, v, qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)
        entry, cargs = lib.fa_fwd_fp8, (ptr(q), ptr(k), ptr(v), ptr(qd), ptr(kd), ptr(vd), ptr(o), ptr(lse),
                                        w.B, w.Hq, w.Hkv, w.N, w.d, w.scale, int(w.causal), sp)
    elif bwd:
        fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=bws,
               stream=stream)
        entry, cargs = lib.fa_bwd, (ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), ptr(do), ptr(dq), ptr(dk), ptr(dv),
                                    w.B, w.Hq, w.Hkv, w.N, w.Nkv, w.d, w.scale, int(w.causal), ptr(bws),
                                    bws.numel(), sp)
    else:
        fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream,
               num_splits=w.splits, workspace=ws)
        f32 = q.dtype == torch.float32
        if w.Nkv == w.N and w.splits == 1:
            entry = lib.fa_fwd_f32 if f32 else lib.fa_fwd
            cargs = (ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), w.B, w.Hq, w.Hkv, w.N, w.d, w.scale,
                     int(w.causal), sp)
        else:
            entry = lib.fa_fwd_splitkv_f32 if f32 else lib.fa_fwd_splitkv
            cargs = (ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), w.B, w.Hq, w.Hkv, w.N, w.Nkv, w.d, w.scale,
                     int(w.causal), w.splits, ptr(ws) if ws is not None else 0,
                     ws.numel() if ws is not None else 0, sp)

    def step():
        if entry(*cargs) != 0:
            raise SystemExit(f"bench.py: {entry.__name__} failed")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Warm-up floor: keep the GPU loaded (at most two chunks of steps in
    # flight, so it never idles between them) until WARMUP_FLOOR_S has passed.
    warm_steps, chunk = args.warmup, 16
    t_w = time.perf_counter()
    pending = []
    while time.perf_counter() - t_w < WARMUP_FLOOR_S:
        for _ in range(chunk):
            step()
        warm_steps += chunk
        ev_w = torch.cuda.Event()
        ev_w.record(stream)
        pending.append(ev_w)
        if len(pending) > 2:
            pending.pop(0).synchronize()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_w

    # Timed region: K steps between one pair of events on the launch stream
    # (an event recorded between steps costs the GPU a few microseconds, which
    # would distort short steps).  One untimed lead step goes first, so that
    # the start event is reached by a busy GPU with the timed steps already
    # queued behind it: recorded on an idle GPU, the event would also time
    # the host's latency to the first launch (~0.1 ms, 2% of 20 headline steps).
    K = args.steps
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step()
    e_start.record(stream)
    for _ in range(K):
        step()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = e_start.elapsed_time(e_end)
    ms_per_step = total_ms / K
    mean_launch_ms = ms_per_step
    # Spread of single steps, from a separate untimed pass with an event
    # before each step (these spans include the events' own cost).
    n_spread = min(K, 50)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_spread + 1)]
    for i in range(n_spread):
        ev[i].record(stream)
        step()
    ev[n_spread].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(n_spread)]   # ms per step
    outs = (dq, dk, dv) if bwd else (o, lse)
    if not all(torch.isfinite(t.float()).all() for t in outs):
        print("bench.py: non-finite output", file=sys.stderr)
        sys.exit(1)

    flops = 2.5 * w.flops if bwd else w.flops
    if hbm_bound:
        unit, peak, work = "GB/s", PEAK_HBM_GBS, w.io_bytes / 1e9
    else:
        unit, peak, work = "TFLOP/s", peak_mfma, flops / 1e12
    value = work / (ms_per_step * 1e-3)
    achieved = work / (mean_launch_ms * 1e-3)
    headline = w.name == W.HEADLINE and not bwd
    src_hash = kernel_source_hash(kernel_sources(w, bwd))
    traffic = read_traffic(traffic_file(w, bwd), src_hash)
    if bwd:
        metric = f"attn bwd TFLOP/s (2.5x forward FLOPs) on {w.name}; % of dense bf16 MFMA peak"
    elif fp8blk:
        metric = (f"attn fwd TFLOP/s on {w.name} (e4m3 inputs with one power-of-two scale per 64 rows, q and k "
                  "Hadamard-rotated; bf16 output); % of dense fp8 MFMA peak")
    elif fp8:
        metric = f"attn fwd TFLOP/s on {w.name} (e4m3 inputs, bf16 output); % of dense fp8 MFMA peak"
    elif sparse:
        metric = (f"attn fwd TFLOP/s on {w.name} (FLOPs of the kept blocks only); "
                  "% of dense bf16 MFMA peak")
    elif fp32:
        metric = f"attn fwd {unit} on {w.name} (fp32 in and out)" + (
            "; % of HBM peak" if hbm_bound else "; % of dense fp32 MFMA peak")
    else:
        metric = METRIC if headline else (
            f"attn fwd {unit} on {w.name}" + ("; % of HBM peak" if hbm_bound else "; % of dense bf16 MFMA peak"))
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_done": {"steps": warm_steps, "floor_s": WARMUP_FLOOR_S,
                        "seconds_beyond_requested": round(warm_s, 3)},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded randn, bf16 round-to-nearest-even)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "io_dtype": w.dtype, "accumulate": "fp32", "layout": "BNHD",
                   "flops_per_step": flops, "pct_of_peak": round(100 * value / peak, 2)},
        "roofline": {"bound": "hbm" if hbm_bound else "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic},
        "timing": {"mean_launch_us": round(mean_launch_ms * 1e3, 2),
                   "min_step_us_with_events": round(min(per) * 1e3, 2),
                   "max_step_us_with_events": round(max(per) * 1e3, 2),
                   "with_events_from": f"a separate pass of {n_spread} steps with an event before each step "
                                       "(each event adds GPU time, so these can exceed the mean)",
                   "host_wall_s": round(wall, 4),
                   "host_wall_covers": f"the lead step and the {K} timed steps, from a synchronised GPU to the end",
                   "kernel_source_hash": src_hash},
    }
    if w.Nkv != w.N or splits > 1:
        out["config"].update({"Nk": w.Nkv, "splits": splits, "algorithmic_bytes_per_step": w.io_bytes})
    if fp32:
        out["dtype"] = "f32"
        out["data"] = "synthetic (seeded randn, fp32)"
    if bwd:
        out["config"]["pass"] = "bwd"
    if sparse:
        out["config"].update({"block_mask": w.mask, "mask_block": [128, 64],
                              "kept_fraction": round(w.flops / (4.0 * w.B * w.Hq * w.N * w.N * w.d), 4)})
    if fp8:
        out["dtype"] = "fp8-e4m3"
        out["data"] = "synthetic (seeded randn, e4m3 round-to-nearest-even with one scale per (batch, head))"
        out["config"].update({"io_dtype": "e4m3 in, bf16 out", "descale": "per (batch, head)"})
    if fp8blk:
        out["data"] = ("synthetic (seeded randn in bf16, quantised on the GPU by fa_quantize_fp8: q and k "
                       "rotated by a seeded random-sign Hadamard transform, one power-of-two scale per 64 rows)")
        out["config"].update({"descale": "per 64-row block (power of two)", "rotation": "q, k: random-sign Hadamard",
                              "scale_passed": w.scale / w.d})
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = (cpu_baseline_bwd(w, args.cpu_seconds, do_host) if bwd
                               else cpu_baseline(w, args.cpu_seconds, hbm_bound))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
