#!/usr/bin/env python3
"""Throughput of the SQA attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--variant HQ,HKV] [--causal 0|1] [--no-cpu-baseline]
                    [--no-compare] [--no-backward] [--no-configs]

A step is one sqa_attn_fwd call over the whole workload (default: B=1,
N=32768, d=64, SQA H_q=8 / H_kv=4, bf16, encoder-style), with inputs already
resident in HBM. FLOPs are counted as 4*B*N^2*H_q*d, halved for causal.
Warm-up is at least W calls and at least 0.5 s of GPU time; the K timed calls
are bracketed by device synchronisations, with a HIP event between
consecutive calls on the launch stream, so the line carries the mean (the
headline, = total / K), the median and the minimum of the per-call times.
While the timed calls run, a thread samples the GPU's graphics clock
(amdsmi GPU metrics), and the roofline is also stated against the peak at
that measured clock (256 CUs x 4096 bf16 FLOP per clock).
Prints ONE JSON line. The line also carries:
  * roofline: the attention kernel's achieved TFLOP/s against the MI355X
    dense bf16 MFMA peak (2516.6 TFLOP/s = 256 CU x 4096 FLOP/clk x 2.4 GHz);
  * cpu_baseline: the fp64 oracle timed on this host's cores on a bounded
    sample of the same workload (sampled query rows, every head);
  * comparison: MHA / GQA-4 / MQA at the same shape (H_q = 16) and the
    measured speedup of the SQA variant over MHA;
  * backward: one sqa_attn_bwd call per step on the same workload (the
    forward's o and lse, a seeded N(0,1) upstream gradient), with FLOPs
    counted as 2.5x the forward's (the five matrix products of the textbook
    backward) and, separately, the FLOPs the kernels execute (3.5x: the dK/dV
    and dQ kernels both recompute S and dP);
  * configs: every workload the target names, each variant timed the same
    way (median and minimum over its calls, TFLOP/s, tokens/s, fraction of
    the nominal and of the clock-adjusted peak, speedup over the (16,16)
    baseline of the same shape next to H/H_q): the SQAT-m attention core
    (fp32, N=1024), the SQAT-m layer (B=16, N=1024), 32k (8,4) / MHA /
    GQA-4 / MQA, 131k (8,8) / (4,4) / (16,16) under both masks, and 200k
    (4,4) / (16,16) with 1 % of the keys scaled by 8.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # dense MFMA, published MI355X figure
PEAK_F32_TFLOPS = 157.3
METRIC = "SQA fwd TFLOP/s + tokens/s at N=32k-200k; % of MI355X bf16 MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_traffic.json")


def counted_flops(B, Hq, N, d, causal):
    f = 4.0 * B * N * N * Hq * d
    return f / 2 if causal else f


KERNELS = {64: ("attn_fwd_bf16_d64_kernel", "attn_fwd_bf16_d64.hip"),
           128: ("attn_fwd_bf16_d128_kernel", "attn_fwd_bf16_d128.hip")}


def kernel_name(d: int) -> str:
    return KERNELS[d][0] if d in KERNELS else f"attn_fwd_bf16_kernel<{d}>"


def kernel_source(d: int) -> str:
    name = KERNELS[d][1] if d in KERNELS else "attn_fwd_bf16.hip"
    return os.path.join(ROOT, "sparse_query_attention_sqa_amd", "csrc", name)


def kernel_source_hash(d: int = 64) -> str:
    with open(kernel_source(d), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic(workload: str, variant, causal: int, d: int):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, only if
    it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    key = f"{workload}:{variant[0]},{variant[1]}:c{causal}"
    e = t.get("entries", {}).get(key)
    if not e or e.get("kernel_sha256_16") != kernel_source_hash(d):
        return None
    return e.get("hbm_bytes_per_launch")


# --num-splits: key-range splits of the forward (None: the library's choice)
NUM_SPLITS = None


def resolved_splits(sqa, B, Hq, Hkv, N, d, causal, T=0):
    if NUM_SPLITS is not None:
        return NUM_SPLITS
    return sqa.sqa_attn_fwd_num_splits(B, Hq, Hkv, N, d, causal=bool(causal), T=T)


def bwd_splits(sqa, B, Hq, Hkv, N, d, causal, T=0):
    """Range splits of the timed backward: --num-splits where the backward
    allows it (encoder-style), else the library's choice."""
    if NUM_SPLITS is not None and not causal:
        return NUM_SPLITS
    return sqa.sqa_attn_bwd_num_splits(B, Hq, Hkv, N, d, causal=bool(causal), T=T)


class ClockSampler:
    """Reads the graphics clock (MHz, mean over the XCDs) from amdsmi's GPU
    metrics in a thread while a kernel runs back to back. The firmware
    refreshes that table about once per second, so a clock reading needs a
    window of a few seconds: only refreshes that arrive more than
    SETTLE_S after the window opened (and so describe a loaded interval)
    count. Reports None where amdsmi is unavailable."""

    SETTLE_S = 1.1

    def __init__(self, period_s: float = 0.02):
        self.period = period_s
        self.samples = []
        self._stop = None
        self._thread = None
        self._handle = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            self._amdsmi = amdsmi
            self._handle = handles[0] if handles else None
            if self._handle is not None and self._read() is None:
                self._handle = None
        except Exception:
            self._handle = None

    def _read(self):
        """(refresh stamp, MHz) or None."""
        try:
            m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
            stamp = m.get("system_clock_counter", m.get("firmware_timestamp"))
            xs = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
            if xs:
                return stamp, sum(xs) / len(xs)
            c = m.get("current_gfxclk")
            if isinstance(c, (int, float)) and 0 < c < 10000:
                return stamp, float(c)
            return None
        except Exception:
            return None

    def start(self):
        import threading
        self.samples = []
        if self._handle is None:
            return
        self._stop = threading.Event()
        t0 = time.perf_counter()

        def run():
            seen = set()
            while not self._stop.is_set():
                r = self._read()
                if r is not None and r[0] not in seen:
                    seen.add(r[0])
                    self.samples.append((time.perf_counter() - t0, r[1]))
                self._stop.wait(self.period)
        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            self._thread = None
        xs = [c for t, c in self.samples if t >= self.SETTLE_S]
        if not xs:
            return None
        return {"mean_mhz": round(sum(xs) / len(xs), 1), "min_mhz": round(min(xs), 1),
                "max_mhz": round(max(xs), 1), "refreshes": len(xs)}


CLOCK = None  # ClockSampler, created in main()
MIN_WARMUP_S = 0.5
CLOCK_WINDOW_S = 2.6
# A HIP event recorded between two calls adds about 2.5 us to the interval
# it closes (measured on the SQAT-m layer: 32.2 us per call with an event
# after every call, 29.6 with one after every ten, 29.6 around 100 calls).
# Calls shorter than this are therefore timed in groups between events.
MIN_INTERVAL_MS = 0.25


def measure(torch, fn, steps, warmup, min_warmup_s=None, clock_window_s=None):
    """Warm up (at least ``warmup`` calls and ``min_warmup_s`` of GPU time,
    each call synchronised so the queue never runs ahead; with a clock
    window, the warm-up lasts at least that long and the graphics clock is
    sampled meanwhile: the clock of this kernel under sustained load), then
    time exactly ``steps`` calls bracketed by synchronisations, with a HIP
    event on the launch stream between consecutive calls -- or, for calls
    shorter than MIN_INTERVAL_MS (estimated from 5 calls between two events;
    not under --profile), between consecutive groups of about MIN_INTERVAL_MS
    of calls, each group's time divided by its number of calls. Returns the mean (total /
    steps), median and minimum per-call times in ms, the calls per timed
    interval, the wall time of the timed calls and the clock."""
    stream = torch.cuda.current_stream()
    if min_warmup_s is None or MIN_WARMUP_S == 0.0:
        min_warmup_s = MIN_WARMUP_S
    if clock_window_s is None:
        clock_window_s = CLOCK_WINDOW_S
    window = clock_window_s if (clock_window_s and CLOCK is not None and CLOCK._handle is not None) else 0.0
    if window:
        CLOCK.start()
    done, t0 = 0, time.perf_counter()
    while done < warmup or time.perf_counter() - t0 < max(min_warmup_s, window):
        fn()
        torch.cuda.synchronize()
        done += 1
    clk = CLOCK.stop() if window else None
    group = 1
    if MIN_WARMUP_S > 0.0:  # --profile: exactly warmup + steps calls, one event after each
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(5):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        est = e0.elapsed_time(e1) / 5
        group = max(1, min(steps, math.ceil(MIN_INTERVAL_MS / max(est, 1e-6))))
    nint = max(1, steps // group)
    sizes = [steps // nint + (1 if i < steps % nint else 0) for i in range(nint)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nint + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record(stream)
    for i, sz in enumerate(sizes):
        for _ in range(sz):
            fn()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = sorted(evs[i].elapsed_time(evs[i + 1]) / sizes[i] for i in range(nint))
    total = evs[0].elapsed_time(evs[nint])
    n = len(per)
    median = per[n // 2] if n % 2 else 0.5 * (per[n // 2 - 1] + per[n // 2])
    return {"mean_ms": total / steps, "median_ms": median, "min_ms": per[0], "calls_per_interval": group,
            "wall_s": wall, "warmup_calls": done, "clock": clk}


def clock_peak_tflops(clk):
    """bf16 dense MFMA peak at the measured mean graphics clock."""
    if not clk:
        return None
    return 256 * 4096 * clk["mean_mhz"] * 1e6 / 1e12


def time_variant(sqa, torch, q, k, v, scale, causal, steps, warmup):
    out = torch.empty_like(q)
    fn = lambda: sqa.sqa_attn_fwd(q, k, v, scale=scale, causal=causal, out=out, num_splits=NUM_SPLITS)
    m = measure(torch, fn, steps, warmup)
    return m, out


def cpu_baseline(w, variant, causal, rows_count, arrays):
    import numpy as np

    from oracle import attention as oracle_attention
    from synth import sample_rows, select_variant
    Hq, Hkv = variant
    q, k, v = select_variant(*arrays, Hq, Hkv)
    rows = sample_rows(w.N, rows_count)
    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        host_cores = os.cpu_count() or 1
    threads = max(1, min(16, host_cores))
    t0 = time.perf_counter()
    oracle_attention(q, k, v, scale=w.scale, causal=bool(causal), rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    if causal:
        flops = float(np.sum(4.0 * (rows + 1) * w.d)) * w.B * Hq
    else:
        flops = 4.0 * len(rows) * w.N * w.d * w.B * Hq
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "host_cores": host_cores,
            "kind": "oracle",
            "sample": f"{len(rows)} seeded query rows x {w.B * Hq} heads of {w.name} "
                      f"({Hq},{Hkv}) causal={causal}, full key range; fp64 numpy, "
                      f"{dt:.2f} s wall"}


def bench_backward(sqa, torch, q, k, v, w, causal, steps, warmup):
    """Time sqa_attn_bwd; inputs, o, lse and the upstream gradient are resident."""
    from synth import draw_upstream
    o, lse = sqa.sqa_attn_fwd(q, k, v, scale=w.scale, causal=bool(causal), return_lse=True)
    do = torch.from_numpy(draw_upstream(tuple(q.shape), "bf16", seed=55)).to("cuda").to(torch.bfloat16)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    ns = bwd_splits(sqa, B, Hq, Hkv, N, d, causal)
    ws = torch.empty(max(1, sqa.sqa_attn_bwd_split_workspace_bytes(B, Hq, Hkv, N, d, ns)), dtype=torch.uint8,
                     device="cuda")

    def fn():
        sqa.sqa_attn_bwd(q, k, v, o, do, lse, scale=w.scale, causal=bool(causal), dq=dq, dk=dk, dv=dv,
                         workspace=ws, num_splits=ns)

    ms = _timed(torch, fn, steps, warmup)
    fwd = counted_flops(B, Hq, N, d, causal)
    counted = 2.5 * fwd
    tflops = counted / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "counted_flop": counted, "tflops_counted": round(tflops, 2),
            "frac_of_peak_counted": round(tflops / PEAK_BF16_TFLOPS, 4),
            "executed_flop": 3.5 * fwd,
            "tflops_executed": round(3.5 * fwd / (ms * 1e-3) / 1e12, 2),
            "kernels": ["bwd_rowterms_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"],
            "num_splits": ns,
            "tokens_per_s": round(B * N / (ms * 1e-3), 1)}


# v_exp_f32: one wave64 instruction (64 exps) per 10.85 cycles per SIMD --
# the rate the issue probe measures (bench.py --probe,
# profiles/issue_probe_forward_mix_d64.md) -- on 1024 SIMDs at 2.4 GHz
PEAK_EXP_PER_S = 1024 * 64 / 10.85 * 2.4e9
HBM_BYTES_PER_S = 8.0e12


def layer_bound(B, N, D, Hq, Hkv, d, measured_ms):
    """Lower bound on the SQA layer's time as the sum, over its three
    kernels, of each kernel's largest single-resource time: the QKV+RoPE and
    output-projection GEMMs by their HBM bytes (inputs read once, outputs
    written once) or bf16 MFMA FLOPs, the causal d = 16 attention by its HBM
    bytes, its MFMA FLOPs or its exponentials at the measured v_exp_f32 rate."""
    e = 2  # bf16
    x = B * N * D * e
    qkv = B * N * (Hq + 2 * Hkv) * d * e
    o = B * N * Hq * d * e
    wts = (D * (Hq + 2 * Hkv) * d + Hq * d * D) * e
    gemm1_flop = 2.0 * B * N * D * (Hq + 2 * Hkv) * d
    gemm2_flop = 2.0 * B * N * Hq * d * D
    attn_flop = counted_flops(B, Hq, N, d, True)
    exps = B * Hq * N * (N + 1) / 2.0
    t1 = max((x + qkv + D * (Hq + 2 * Hkv) * d * e) / HBM_BYTES_PER_S, gemm1_flop / (PEAK_BF16_TFLOPS * 1e12))
    t2 = max((qkv + o) / HBM_BYTES_PER_S, attn_flop / (PEAK_BF16_TFLOPS * 1e12), exps / PEAK_EXP_PER_S)
    t3 = max((o + x + Hq * d * D * e) / HBM_BYTES_PER_S, gemm2_flop / (PEAK_BF16_TFLOPS * 1e12))
    bound_us = (t1 + t2 + t3) * 1e6
    return {"bound": "hbm+exp (sum over kernels)", "bound_us": round(bound_us, 2),
            "bound_parts_us": {"qkv_rope_gemm": round(t1 * 1e6, 2), "attention": round(t2 * 1e6, 2),
                               "out_proj_gemm": round(t3 * 1e6, 2)},
            "algorithmic_bytes": x + 2 * qkv + 2 * o + x + wts,
            "frac_of_bound": round(bound_us / (measured_ms * 1e3), 4)}


def _timed(torch, fn, steps, warmup):
    return measure(torch, fn, steps, warmup, clock_window_s=0)["mean_ms"]


def _common(args, ms, w, extra):
    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "data": "synthetic"}
    line.update(extra)
    return line


def bench_layer(sqa, torch, w, args):
    """SQAT-m attention layer: projections + RoPE + causal SQA + output projection."""
    from synth import draw_layer
    Hq, Hkv = w.variants[0]
    d = w.d_model // w.H
    x, wq, wk, wv, wo = draw_layer(w.B, w.N, w.d_model, w.H, Hq, Hkv, seed=0)
    dev = lambda a: torch.from_numpy(a).to("cuda").to(torch.bfloat16).contiguous()
    tx, tq, tk, tv, to = (dev(a) for a in (x, wq, wk, wv, wo))
    out = torch.empty_like(tx)
    ws = torch.empty(sqa.sqa_layer_workspace_bytes(w.B, w.N, w.d_model, w.H, Hq, Hkv),
                     dtype=torch.uint8, device="cuda")
    fn = lambda: sqa.sqa_layer_fwd(tx, tq, tk, tv, to, H=w.H, H_q=Hq, H_kv=Hkv, rope_base=w.rope_base,
                                   scale=w.scale, causal=True, out=out, workspace=ws)
    m = measure(torch, fn, args.steps, args.warmup)
    ms = m["mean_ms"]
    attn = counted_flops(w.B, Hq, w.N, d, True)
    gemm = 2.0 * w.B * w.N * w.d_model * (Hq + 2 * Hkv) * d + 2.0 * w.B * w.N * Hq * d * w.d_model
    tflops = (attn + gemm) / (ms * 1e-3) / 1e12
    lb = layer_bound(w.B, w.N, w.d_model, Hq, Hkv, d, ms)
    return _common(args, ms, w, {
        "value": round(tflops, 3), "unit": "TFLOP/s", "dtype": "bf16",
        "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1),
        "config": {"workload": w.name, "B": w.B, "N": w.N, "D": w.d_model, "H": w.H, "H_q": Hq,
                   "H_kv": Hkv, "d": d, "causal": 1, "flop_attention": attn, "flop_gemm": gemm},
        "roofline": {"bound": "hbm+exp", "achieved": round(ms * 1e3, 3), "peak": lb["bound_us"], "unit": "us",
                     "frac": lb["frac_of_bound"], "traffic": None, "parts_us": lb["bound_parts_us"],
                     "median_ms": round(m["median_ms"], 5), "min_ms": round(m["min_ms"], 5),
                     "kernel": "whole layer: time against the sum of each kernel's single-resource bound"},
        "cpu_baseline": None, "comparison": None})


def bench_block(sqa, torch, w, args):
    """SQAT-m block: RMSNorm, SQA layer, residual, RMSNorm, SwiGLU, residual.
    One block call per step for the selected variant; the other variants of
    the workload (MHA / GQA / MQA) go in `comparison`."""
    from synth import draw_block
    variant = tuple(int(x) for x in args.variant.split(",")) if args.variant else w.variants[0]
    d = w.d_model // w.H
    dev = lambda a: torch.from_numpy(a).to("cuda").to(torch.bfloat16).contiguous()

    def flops(hq, hkv):
        attn = counted_flops(w.B, hq, w.N, d, True)
        proj = 2.0 * w.B * w.N * w.d_model * (hq + 2 * hkv) * d + 2.0 * w.B * w.N * hq * d * w.d_model
        ffn = 3 * 2.0 * w.B * w.N * w.d_model * w.d_ff
        return attn, proj, ffn

    def run(var):
        hq, hkv = var
        arrs = [dev(a) for a in draw_block(w.B, w.N, w.d_model, w.H, hq, hkv, w.d_ff, seed=0)]
        out = torch.empty_like(arrs[0])
        ws = torch.empty(sqa.sqa_block_workspace_bytes(w.B, w.N, w.d_model, w.H, hq, hkv, w.d_ff),
                         dtype=torch.uint8, device="cuda")
        fn = lambda: sqa.sqa_block_fwd(*arrs, H=w.H, H_q=hq, H_kv=hkv, rope_base=w.rope_base,
                                       scale=w.scale, causal=True, out=out, workspace=ws)
        ms = _timed(torch, fn, args.steps, args.warmup)
        del arrs, out, ws
        torch.cuda.empty_cache()
        return ms

    ms = run(variant)
    attn, proj, ffn = flops(*variant)
    tflops = (attn + proj + ffn) / (ms * 1e-3) / 1e12
    comparison = None
    if not args.no_compare:
        comparison = {}
        for var in w.variants:
            if var == variant:
                continue
            cms = run(var)
            comparison[f"{var[0]},{var[1]}"] = {"ms": round(cms, 4)}
        if "16,16" in comparison:
            comparison["time_ratio_vs_mha"] = round(ms / comparison["16,16"]["ms"], 4)
    return _common(args, ms, w, {
        "value": round(tflops, 3), "unit": "TFLOP/s", "dtype": "bf16",
        "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1),
        "config": {"workload": w.name, "B": w.B, "N": w.N, "D": w.d_model, "H": w.H,
                   "H_q": variant[0], "H_kv": variant[1], "d": d, "F": w.d_ff, "causal": 1,
                   "flop_attention": attn, "flop_projections": proj, "flop_ffn": ffn},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "whole block (small GEMMs, d=16 attention)"},
        "cpu_baseline": None, "comparison": comparison})


def bench_f32(sqa, torch, w, args):
    """SQAT-m attention core in fp32 (VALU-bound correctness workload)."""
    from synth import draw_qkv, select_variant
    Hq, Hkv = w.variants[0]
    causal = w.causal[0] if args.causal is None else args.causal
    q, k, v = select_variant(*draw_qkv(w.B, w.H, w.N, w.d, "f32", seed=0), Hq, Hkv)
    dev = lambda a: torch.from_numpy(a).to("cuda").contiguous()
    tq, tk, tv = dev(q), dev(k), dev(v)
    out = torch.empty_like(tq)
    fn = lambda: sqa.sqa_attn_fwd(tq, tk, tv, scale=w.scale, causal=bool(causal), out=out)
    ms = _timed(torch, fn, args.steps, args.warmup)
    flops = counted_flops(w.B, Hq, w.N, w.d, causal)
    tflops = flops / (ms * 1e-3) / 1e12
    return _common(args, ms, w, {
        "value": round(tflops, 4), "unit": "TFLOP/s", "dtype": "f32",
        "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1),
        "config": {"workload": w.name, "B": w.B, "N": w.N, "H": w.H, "H_q": Hq, "H_kv": Hkv,
                   "d": w.d, "causal": int(causal), "scale": w.scale},
        "roofline": {"bound": "alu", "achieved": round(tflops, 4), "peak": PEAK_F32_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_F32_TFLOPS, 5), "traffic": None,
                     "kernel": "attn_fwd_f32_kernel<16>"},
        "cpu_baseline": None, "comparison": None})


def bench_varlen(sqa, torch, w, args):
    """Packed batch of sequences of mixed lengths (sqa_attn_fwd_varlen); FLOPs
    are the sum over sequences of 4*len^2*H_q*d (halved for causal)."""
    import numpy as np

    from synth import draw_varlen, varlen_lengths
    variant = tuple(int(x) for x in args.variant.split(",")) if args.variant else w.variants[0]
    causal = w.causal[0] if args.causal is None else args.causal
    lens = varlen_lengths(w.N, w.varlen)
    q_all, k_all, v_all, cu = draw_varlen(lens, w.H, w.H, w.d, "bf16", seed=0)
    tcu = torch.from_numpy(cu).to("cuda")
    maxlen = int(lens.max())
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(torch.bfloat16).contiguous()

    def flops(hq):
        f = float(np.sum(4.0 * lens.astype(np.float64) ** 2)) * hq * w.d
        return f / 2 if causal else f

    def run(var):
        hq, hkv = var
        q, k, v = dev(q_all[:hq]), dev(k_all[:hkv]), dev(v_all[:hkv])
        out = torch.empty_like(q)
        fn = lambda: sqa.sqa_attn_fwd_varlen(q, k, v, tcu, maxlen, scale=w.scale, causal=bool(causal), out=out,
                                             num_splits=NUM_SPLITS)
        ms = _timed(torch, fn, args.steps, args.warmup)
        del q, k, v, out
        torch.cuda.empty_cache()
        return ms

    ms = run(variant)
    tflops = flops(variant[0]) / (ms * 1e-3) / 1e12
    backward = None
    if not args.no_backward and w.d in (64, 128):
        from synth import draw_upstream
        hq, hkv = variant
        q, k, v = dev(q_all[:hq]), dev(k_all[:hkv]), dev(v_all[:hkv])
        o, lse = sqa.sqa_attn_fwd_varlen(q, k, v, tcu, maxlen, scale=w.scale, causal=bool(causal), return_lse=True)
        do = dev(draw_upstream(tuple(q.shape), "bf16", seed=55))
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ns = bwd_splits(sqa, w.varlen, hq, hkv, maxlen, w.d, causal, T=w.N)
        ws = torch.empty(sqa.sqa_attn_bwd_varlen_split_workspace_bytes(w.varlen, hq, hkv, w.N, w.d, ns),
                         dtype=torch.uint8, device="cuda")
        fn = lambda: sqa.sqa_attn_bwd_varlen(q, k, v, o, do, lse, tcu, maxlen, scale=w.scale, causal=bool(causal),
                                             dq=dq, dk=dk, dv=dv, workspace=ws, num_splits=ns)
        bms = _timed(torch, fn, args.steps, args.warmup)
        counted = 2.5 * flops(hq)
        backward = {"ms": round(bms, 4), "counted_flop": counted, "num_splits": ns,
                    "tflops_counted": round(counted / (bms * 1e-3) / 1e12, 2),
                    "frac_of_peak_counted": round(counted / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del q, k, v, o, lse, do, dq, dk, dv, ws
        torch.cuda.empty_cache()
    comparison = None
    if not args.no_compare:
        comparison = {}
        for var in w.variants:
            if var != variant:
                cms = run(var)
                comparison[f"{var[0]},{var[1]}"] = {"ms": round(cms, 4),
                                                    "tflops": round(flops(var[0]) / (cms * 1e-3) / 1e12, 2)}
        if "16,16" in comparison:
            comparison["speedup_vs_mha"] = round(comparison["16,16"]["ms"] / ms, 3)
    kernel = kernel_name(w.d)
    return _common(args, ms, w, {
        "value": round(tflops, 3), "unit": "TFLOP/s", "dtype": "bf16",
        "tokens_per_s": round(w.N / (ms * 1e-3), 1),
        "config": {"workload": w.name, "T": w.N, "sequences": lens.tolist(), "H": w.H,
                   "H_q": variant[0], "H_kv": variant[1], "d": w.d, "causal": int(causal),
                   "num_splits": resolved_splits(sqa, w.varlen, variant[0], variant[1], maxlen, w.d, causal,
                                                 T=w.N)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": kernel, "per_launch_flop": flops(variant[0])},
        "cpu_baseline": None, "comparison": comparison, "backward": backward})


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long32k_bf16")
    ap.add_argument("--variant", default=None, help="H_q,H_kv (default: the workload's first)")
    ap.add_argument("--causal", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="for runs under a profiler: warm up with exactly --warmup calls (no minimum time, no "
                         "clock window), so that the trace holds only the calls asked for")
    ap.add_argument("--probe", action="store_true",
                    help="only run the issue-rate probes (libsqa_probe.so) and the 32k (8,4) forward; "
                         "print their JSON object")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the sweep over every target workload (the configs object)")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only sqa_attn_bwd (for profiling) and print its object")
    ap.add_argument("--cpu-rows", type=int, default=65536)
    ap.add_argument("--num-splits", type=int, default=None,
                    help="key-range splits of the d=64 forward (default: the library's choice)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times) and exit; "
                         "used to scale rocprofv3 FETCH_SIZE/WRITE_SIZE")
    args = ap.parse_args()
    global NUM_SPLITS, CLOCK
    NUM_SPLITS = args.num_splits

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs on one GPU; the forward needs no collective)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_query_attention_sqa_amd as sqa
    from synth import WORKLOADS, draw_qkv, select_variant

    if not os.path.exists(sqa.lib_path()):
        from sparse_query_attention_sqa_amd import _build
        _build.build()
    sqa.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.profile:
        global MIN_WARMUP_S, CLOCK_WINDOW_S
        MIN_WARMUP_S = 0.0
        CLOCK_WINDOW_S = 0.0
        CLOCK = None
    else:
        CLOCK = ClockSampler()

    if args.probe:
        print(json.dumps({"probes": run_probes(torch, sqa)}), flush=True)
        return

    if args.copy_calib:
        n = args.copy_calib * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_per_launch": n}), flush=True)
        return

    w = WORKLOADS[args.workload]
    if w.block:
        print(json.dumps(bench_block(sqa, torch, w, args)), flush=True)
        return
    if w.layer:
        print(json.dumps(bench_layer(sqa, torch, w, args)), flush=True)
        return
    if w.dtype != "bf16":
        print(json.dumps(bench_f32(sqa, torch, w, args)), flush=True)
        return
    if w.varlen:
        print(json.dumps(bench_varlen(sqa, torch, w, args)), flush=True)
        return
    variant = tuple(int(x) for x in args.variant.split(",")) if args.variant else w.variants[0]
    causal = w.causal[0] if args.causal is None else args.causal
    Hq, Hkv = variant

    q_all, k_all, v_all = draw_qkv(w.B, w.H, w.N, w.d, w.dtype, seed=0, peaky=w.peaky)

    def dev(a):
        return torch.from_numpy(a).to("cuda").to(torch.bfloat16).contiguous()

    def run(var, steps, warmup):
        q, k, v = (dev(a) for a in select_variant(q_all, k_all, v_all, *var))
        m, _ = time_variant(sqa, torch, q, k, v, w.scale, bool(causal), steps, warmup)
        del q, k, v
        torch.cuda.empty_cache()
        return m

    if args.backward_only:
        q, k, v = (dev(a) for a in select_variant(q_all, k_all, v_all, *variant))
        print(json.dumps({"backward": bench_backward(sqa, torch, q, k, v, w, causal, args.steps,
                                                     args.warmup)}), flush=True)
        return

    # the headline: exactly --steps timed calls after the warm-up
    m = run(variant, args.steps, args.warmup)
    ms = m["mean_ms"]
    flops = counted_flops(w.B, Hq, w.N, w.d, causal)
    tflops = flops / (ms * 1e-3) / 1e12
    tokens = w.B * w.N / (ms * 1e-3)

    comparison = None
    if not args.no_compare:
        comparison = {}
        for var in [(16, 16), (16, 4), (16, 1)] + [v for v in w.variants if v != variant]:
            key = f"{var[0]},{var[1]}"
            if key in comparison or var == variant or var[0] > w.H:
                continue
            cm = run(var, args.steps, args.warmup)
            cms = cm["mean_ms"]
            comparison[key] = {"ms": round(cms, 4), "median_ms": round(cm["median_ms"], 4),
                               "tflops": round(counted_flops(w.B, var[0], w.N, w.d, causal) / (cms * 1e-3) / 1e12, 2)}
        if "16,16" in comparison:
            comparison["speedup_vs_mha"] = round(comparison["16,16"]["ms"] / ms, 3)
            comparison["expected_H_over_Hq"] = w.H / Hq

    backward = None
    if not args.no_backward and w.d in (64, 128):
        q, k, v = (dev(a) for a in select_variant(q_all, k_all, v_all, *variant))
        backward = bench_backward(sqa, torch, q, k, v, w, causal, args.steps, args.warmup)
        del q, k, v
        torch.cuda.empty_cache()
    del q_all, k_all, v_all

    traffic = stored_traffic(w.name, variant, causal, w.d)
    cpk = clock_peak_tflops(m["clock"])
    roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic,
                "traffic_source": "profiles/attn_fwd_bf16_traffic.json (rocprofv3 FETCH_SIZE/WRITE_SIZE of this "
                                  "kernel source, scaled by a 1 GiB copy); null if the source changed since",
                "kernel": kernel_name(w.d),
                "per_launch_flop": flops,
                "median_ms": round(m["median_ms"], 5), "min_ms": round(m["min_ms"], 5),
                "tflops_median": round(flops / (m["median_ms"] * 1e-3) / 1e12, 2),
                "tflops_min_time": round(flops / (m["min_ms"] * 1e-3) / 1e12, 2),
                "clock": m["clock"],
                "peak_at_clock": round(cpk, 1) if cpk else None,
                "frac_at_clock": round(tflops / cpk, 4) if cpk else None}

    configs = None
    if not args.no_configs and w.name == "long32k_bf16":
        configs = run_configs(sqa, torch, args)

    cpu = None
    if not args.no_cpu_baseline:
        qa, ka, va = draw_qkv(w.B, w.H, w.N, w.d, w.dtype, seed=0, peaky=w.peaky)
        cpu = cpu_baseline(w, variant, causal, args.cpu_rows, (qa, ka, va))

    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "tokens_per_s": round(tokens, 1),
        "config": {"workload": w.name, "B": w.B, "N": w.N, "H": w.H, "H_q": Hq, "H_kv": Hkv,
                   "d": w.d, "causal": int(causal), "scale": w.scale, "peaky_keys": w.peaky,
                   "num_splits": resolved_splits(sqa, w.B, Hq, Hkv, w.N, w.d, causal),
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "comparison": comparison,
        "backward": backward,
        "configs": configs,
        "warmup_calls": m["warmup_calls"],
        "wall_s_timed_region": round(m["wall_s"], 4),
    }
    print(json.dumps(line), flush=True)


# ------------------------------------------------------------ issue probes
PROBE_KINDS = {0: "mfma_only", 1: "forward_mix_registers", 2: "forward_mix_with_lds_reads", 3: "exp_only",
               4: "fma_only"}


def run_probes(torch, sqa):
    """Time the issue-rate probes of libsqa_probe.so (two 4-wave workgroups
    per CU) and the d = 64 forward on the 32k (8,4) workload in the same
    process; rates per launch from HIP events, clock sampled meanwhile."""
    import ctypes
    path = os.path.join(ROOT, "sparse_query_attention_sqa_amd", "libsqa_probe.so")
    lib = ctypes.CDLL(path)
    lib.sqa_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.sqa_probe_run.restype = ctypes.c_int
    lib.sqa_probe_threads.argtypes = [ctypes.c_int]
    lib.sqa_probe_threads.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = 2 * cus
    out = torch.empty(lib.sqa_probe_threads(wgs), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    res = {"workgroups": wgs, "threads_per_workgroup": 256, "cus": cus}
    iters = {0: 4000, 1: 2000, 2: 2000, 3: 40000, 4: 40000}
    for kind, name in PROBE_KINDS.items():
        n = iters[kind]
        fn = lambda: _check_probe(lib.sqa_probe_run(kind, wgs, n, ctypes.c_void_p(out.data_ptr()),
                                                    ctypes.c_void_p(st.cuda_stream)))
        m = measure(torch, fn, 7, 2, min_warmup_s=0.3)
        t = m["median_ms"] * 1e-3
        e = {"iters": n, "median_ms": round(m["median_ms"], 4), "min_ms": round(m["min_ms"], 4),
             "clock_mhz": m["clock"]["mean_mhz"] if m["clock"] else None}
        waves = wgs * 4
        if kind in (0, 1, 2):
            fl = waves * n * 16 * 32768.0
            e["mfma_tflops"] = round(fl / t / 1e12, 2)
            e["frac_of_nominal"] = round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4)
            cpk = clock_peak_tflops(m["clock"])
            e["frac_at_clock"] = round(fl / t / 1e12 / cpk, 4) if cpk else None
        else:
            ops = waves * n * 16.0  # wave64 instructions
            e["wave_instructions_per_s"] = round(ops / t, 1)
            e["lane_ops_per_s"] = round(ops * 64 / t, 1)
            if m["clock"]:
                e["cycles_per_wave_instruction_per_simd"] = round(t * m["clock"]["mean_mhz"] * 1e6 / (ops / (cus * 4)), 3)
        res[name] = e
    base = res["mfma_only"]["mfma_tflops"]
    for name in ("forward_mix_registers", "forward_mix_with_lds_reads"):
        res[name]["frac_of_mfma_only"] = round(res[name]["mfma_tflops"] / base, 4)
    # the forward itself on the 32k (8,4) workload, same process
    from synth import draw_qkv, select_variant
    q, k, v = (torch.from_numpy(a).to("cuda").to(torch.bfloat16).contiguous()
               for a in select_variant(*draw_qkv(1, 16, 32768, 64, "bf16", seed=0), 8, 4))
    o = torch.empty_like(q)
    fn = lambda: sqa.sqa_attn_fwd(q, k, v, scale=0.125, causal=False, out=o, num_splits=1)
    m = measure(torch, fn, 20, 5)
    fl = counted_flops(1, 8, 32768, 64, False)
    tf = fl / (m["median_ms"] * 1e-3) / 1e12
    cpk = clock_peak_tflops(m["clock"])
    mix = res["forward_mix_with_lds_reads"]
    e = {"median_ms": round(m["median_ms"], 4), "tflops": round(tf, 2),
         "frac_of_nominal": round(tf / PEAK_BF16_TFLOPS, 4), "frac_of_mfma_only": round(tf / base, 4),
         "frac_of_forward_mix_with_lds_reads": round(tf / mix["mfma_tflops"], 4),
         "clock_mhz": m["clock"]["mean_mhz"] if m["clock"] else None,
         "frac_at_clock": round(tf / cpk, 4) if cpk else None}
    if cpk and mix.get("frac_at_clock"):
        # per clock cycle: the kernel's MFMA fraction against the probe's
        e["per_clock_vs_forward_mix_with_lds_reads"] = round(e["frac_at_clock"] / mix["frac_at_clock"], 4)
    res["attn_fwd_bf16_d64_kernel_long32k_8_4"] = e
    return res


def _check_probe(code):
    if code != 0:
        raise RuntimeError(f"sqa_probe_run failed with HIP error {code}")


# ------------------------------------------------------------ every config
CONFIG_MIN_TIMED_S = 0.25
CONFIG_MIN_CALLS = 3
CONFIG_MAX_CALLS = 20


def _calls_for(ms_estimate):
    return int(max(CONFIG_MIN_CALLS, min(CONFIG_MAX_CALLS, math.ceil(CONFIG_MIN_TIMED_S * 1e3 / max(ms_estimate, 1e-3)))))


def _entry(m, flops, tokens, peak, calls):
    cpk = clock_peak_tflops(m["clock"])
    med = m["median_ms"]
    tf = flops / (med * 1e-3) / 1e12
    e = {"calls": calls, "calls_per_interval": m["calls_per_interval"], "median_ms": round(med, 5),
         "min_ms": round(m["min_ms"], 5),
         "mean_ms": round(m["mean_ms"], 5), "tflops": round(tf, 2),
         "tflops_min_time": round(flops / (m["min_ms"] * 1e-3) / 1e12, 2),
         "tokens_per_s": round(tokens / (med * 1e-3), 1), "frac": round(tf / peak, 4),
         "clock_mhz": m["clock"]["mean_mhz"] if m["clock"] else None}
    if cpk and peak == PEAK_BF16_TFLOPS:
        e["frac_at_clock"] = round(tf / cpk, 4)
    return e


def _attn_config(sqa, torch, wname, variants, causals):
    """Time every (variant, causal) of a long-sequence workload; speedups are
    t(16,16) / t(variant) of the same mask, next to H / H_q."""
    from synth import WORKLOADS, draw_qkv, select_variant
    w = WORKLOADS[wname]
    qa, ka, va = draw_qkv(w.B, w.H, w.N, w.d, w.dtype, seed=0, peaky=w.peaky)
    out = {}
    for var in variants:
        q, k, v = (torch.from_numpy(a).to("cuda").to(torch.bfloat16).contiguous()
                   for a in select_variant(qa, ka, va, *var))
        o = torch.empty_like(q)
        for causal in causals:
            fn = lambda: sqa.sqa_attn_fwd(q, k, v, scale=w.scale, causal=bool(causal), out=o)
            fl = counted_flops(w.B, var[0], w.N, w.d, causal)
            est = fl / (1.0e15) * 1e3  # ms at 1 PFLOP/s, to size the timed calls
            calls = _calls_for(est)
            m = measure(torch, fn, calls, 2)
            out[f"{var[0]},{var[1]}" + (":causal" if causal else "")] = _entry(m, fl, w.B * w.N, PEAK_BF16_TFLOPS,
                                                                                 calls)
            print(f"[bench] {wname} {var} causal={causal}: {m['median_ms']:.4f} ms", file=sys.stderr, flush=True)
        del q, k, v, o
        torch.cuda.empty_cache()
    del qa, ka, va
    for key, e in out.items():
        causal = key.endswith(":causal")
        base = out.get("16,16" + (":causal" if causal else ""))
        hq = int(key.split(",")[0])
        if base and hq != 16:
            e["speedup_vs_16_16"] = round(base["median_ms"] / e["median_ms"], 3)
            e["H_over_Hq"] = round(w.H / hq, 3)
    return {"workload": wname, "B": w.B, "N": w.N, "d": w.d, "peaky_keys": w.peaky, "variants": out}


def run_configs(sqa, torch, args):
    from synth import WORKLOADS, draw_layer, draw_qkv, select_variant
    res = {}
    # SQAT-m attention core, fp32 (a correctness workload; fp32 vector bound)
    w = WORKLOADS["sqatm_core_f32"]
    q, k, v = (torch.from_numpy(a).to("cuda").contiguous()
               for a in select_variant(*draw_qkv(w.B, w.H, w.N, w.d, "f32", seed=0), 8, 4))
    o = torch.empty_like(q)
    core = {}
    for causal in (0, 1):
        fn = lambda: sqa.sqa_attn_fwd(q, k, v, scale=w.scale, causal=bool(causal), out=o)
        m = measure(torch, fn, 50, 5, min_warmup_s=0.2)
        core["8,4" + (":causal" if causal else "")] = _entry(m, counted_flops(w.B, 8, w.N, w.d, causal), w.B * w.N,
                                                              PEAK_F32_TFLOPS, 50)
    res["C1_sqatm_core_f32"] = {"workload": w.name, "B": w.B, "N": w.N, "d": w.d, "dtype": "f32",
                                "peak": "fp32 vector 157.3 TFLOP/s", "variants": core}
    del q, k, v, o
    # SQAT-m layer: projections + RoPE + causal SQA + output projection
    w = WORKLOADS["sqatm_layer_bf16"]
    d = w.d_model // w.H
    arrs = [torch.from_numpy(a).to("cuda").to(torch.bfloat16).contiguous()
            for a in draw_layer(w.B, w.N, w.d_model, w.H, 8, 4, seed=0)]
    y = torch.empty_like(arrs[0])
    ws = torch.empty(sqa.sqa_layer_workspace_bytes(w.B, w.N, w.d_model, w.H, 8, 4), dtype=torch.uint8, device="cuda")
    fn = lambda: sqa.sqa_layer_fwd(*arrs, H=w.H, H_q=8, H_kv=4, rope_base=w.rope_base, scale=w.scale, causal=True,
                                   out=y, workspace=ws)
    m = measure(torch, fn, 100, 10, min_warmup_s=0.2)
    attn = counted_flops(w.B, 8, w.N, d, True)
    gemm = 2.0 * w.B * w.N * w.d_model * (8 + 2 * 4) * d + 2.0 * w.B * w.N * 8 * d * w.d_model
    e = _entry(m, attn + gemm, w.B * w.N, PEAK_BF16_TFLOPS, 100)
    e.update(layer_bound(w.B, w.N, w.d_model, 8, 4, d, m["median_ms"]))
    res["C2_sqatm_layer_bf16"] = {"workload": w.name, "B": w.B, "N": w.N, "D": w.d_model, "d": d, "causal": 1,
                                  "variants": {"8,4:causal": e}}
    del arrs, y, ws
    torch.cuda.empty_cache()
    res["C3_long32k"] = _attn_config(sqa, torch, "long32k_bf16", [(8, 4), (16, 16), (16, 4), (16, 1)], (0,))
    res["C4_long131k"] = _attn_config(sqa, torch, "long131k_bf16", [(8, 8), (4, 4), (16, 16)], (0, 1))
    res["C5_long200k_peaky"] = _attn_config(sqa, torch, "long200k_peaky_bf16", [(4, 4), (16, 16)], (0,))
    return res


if __name__ == "__main__":
    main()
