#!/usr/bin/env python3
"""Throughput of the SQA attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--variant HQ,HKV] [--causal 0|1] [--no-cpu-baseline]
                    [--no-compare]

A step is one sqa_attn_fwd call over the whole workload (default: B=1,
N=32768, d=64, SQA H_q=8 / H_kv=4, bf16, encoder-style), with inputs already
resident in HBM. FLOPs are counted as 4*B*N^2*H_q*d, halved for causal.
Prints ONE JSON line. The line also carries:
  * roofline: the attention kernel's achieved TFLOP/s against the MI355X
    dense bf16 MFMA peak (2516.6 TFLOP/s = 256 CU x 4096 FLOP/clk x 2.4 GHz),
    timed with HIP events on the stream the kernel runs on;
  * cpu_baseline: the fp64 oracle timed on this host's cores on a bounded
    sample of the same workload (sampled query rows, every head);
  * comparison: MHA / GQA-4 / MQA at the same shape (H_q = 16) and the
    measured speedup of the SQA variant over MHA;
  * backward: one sqa_attn_bwd call per step on the same workload (the
    forward's o and lse, a seeded N(0,1) upstream gradient), with FLOPs
    counted as 2.5x the forward's (the five matrix products of the textbook
    backward) and, separately, the FLOPs the kernels execute (3.5x: the dK/dV
    and dQ kernels both recompute S and dP).
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


def time_variant(sqa, torch, q, k, v, scale, causal, steps, warmup):
    stream = torch.cuda.current_stream()
    out = torch.empty_like(q)
    for _ in range(warmup):
        sqa.sqa_attn_fwd(q, k, v, scale=scale, causal=causal, out=out, num_splits=NUM_SPLITS)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        sqa.sqa_attn_fwd(q, k, v, scale=scale, causal=causal, out=out, num_splits=NUM_SPLITS)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return start.elapsed_time(end) / steps, wall, out


def cpu_baseline(w, variant, causal, rows_count, arrays):
    import numpy as np

    from oracle import attention as oracle_attention
    from synth import sample_rows, select_variant
    Hq, Hkv = variant
    q, k, v = select_variant(*arrays, Hq, Hkv)
    rows = sample_rows(w.N, rows_count)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    threads = max(1, min(16, cores))
    t0 = time.perf_counter()
    oracle_attention(q, k, v, scale=w.scale, causal=bool(causal), rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    if causal:
        flops = float(np.sum(4.0 * (rows + 1) * w.d)) * w.B * Hq
    else:
        flops = 4.0 * len(rows) * w.N * w.d * w.B * Hq
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
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


# v_exp_f32 issues at half rate: 64 lanes / 8 cycles per SIMD, 1024 SIMDs, 2.4 GHz
PEAK_EXP_PER_S = 1024 * 8 * 2.4e9


def _timed(torch, fn, steps, warmup):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


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
    ms = _timed(torch, fn, args.steps, args.warmup)
    attn = counted_flops(w.B, Hq, w.N, d, True)
    gemm = 2.0 * w.B * w.N * w.d_model * (Hq + 2 * Hkv) * d + 2.0 * w.B * w.N * Hq * d * w.d_model
    exps = w.B * Hq * w.N * (w.N + 1) / 2.0
    tflops = (attn + gemm) / (ms * 1e-3) / 1e12
    achieved = exps / (ms * 1e-3) / 1e12
    return _common(args, ms, w, {
        "value": round(tflops, 3), "unit": "TFLOP/s", "dtype": "bf16",
        "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1),
        "config": {"workload": w.name, "B": w.B, "N": w.N, "D": w.d_model, "H": w.H, "H_q": Hq,
                   "H_kv": Hkv, "d": d, "causal": 1, "flop_attention": attn, "flop_gemm": gemm},
        "roofline": {"bound": "alu", "achieved": round(achieved, 3),
                     "peak": round(PEAK_EXP_PER_S / 1e12, 3), "unit": "Texp/s",
                     "frac": round(achieved * 1e12 / PEAK_EXP_PER_S, 4), "traffic": None,
                     "kernel": "whole layer (attention at d=16 is v_exp-bound)"},
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
    ap.add_argument("--backward-only", action="store_true",
                    help="time only sqa_attn_bwd (for profiling) and print its object")
    ap.add_argument("--cpu-rows", type=int, default=65536)
    ap.add_argument("--num-splits", type=int, default=None,
                    help="key-range splits of the d=64 forward (default: the library's choice)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times) and exit; "
                         "used to scale rocprofv3 FETCH_SIZE/WRITE_SIZE")
    args = ap.parse_args()
    global NUM_SPLITS
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

    def run(var):
        q, k, v = (dev(a) for a in select_variant(q_all, k_all, v_all, *var))
        ms, wall, _ = time_variant(sqa, torch, q, k, v, w.scale, bool(causal), args.steps, args.warmup)
        del q, k, v
        torch.cuda.empty_cache()
        return ms, wall

    if args.backward_only:
        q, k, v = (dev(a) for a in select_variant(q_all, k_all, v_all, *variant))
        print(json.dumps({"backward": bench_backward(sqa, torch, q, k, v, w, causal, args.steps,
                                                     args.warmup)}), flush=True)
        return

    ms, wall = run(variant)
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
            cms, _ = run(var)
            comparison[key] = {"ms": round(cms, 4),
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

    traffic = stored_traffic(w.name, variant, causal, w.d)
    roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic,
                "kernel": kernel_name(w.d),
                "per_launch_flop": flops}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, variant, causal, args.cpu_rows, (q_all, k_all, v_all))

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
        "wall_s_timed_region": round(wall, 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
