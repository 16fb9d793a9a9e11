"""Shared helpers for the GPU parity tests: device transfer, oracle threading
and the acceptance checks.

Acceptance (stated tolerance, per workload and variant):
  * fp32 inputs:  max |O - O_ref| <= 1e-4 over every checked element.
  * bf16 inputs:  max |O - O_ref| <= 1e-2 * max |O_ref| over every checked
    element (all heads, all checked rows).
  * per-row gate (stricter in effect where rows differ in magnitude): for the
    rows it is applied to, max_c |O - O_ref| <= max(1e-2 * max_c |O_ref|, 2^-14)
    (2^-14 is the bf16 resolution floor, which only takes over for rows whose
    outputs all but vanish).
  * per-row gate for gradients: a gradient row is a sum of products whose
    terms cancel (each row of dS sums to zero), so its bar is set by the
    sum of the terms' absolute values, the scale of the rounding error any
    computation of it makes: max_c |g - g_ref| <= max(1e-2 * max_c A, 2^-14)
    with A the oracle's absolute-term sums (attention_bwd(absolute=True)).
    The kernels round dS and P to bf16 (relative error at most 2^-8 per
    term), so their error stays below 2^-8 * A ~ 3.9e-3 * A.
  * LSE of bf16 inputs: |LSE - LSE_ref| <= 5e-3. The kernels sum the
    probabilities after rounding them to bf16 (relative error at most 2^-8
    each), so |LSE - LSE_ref| <= ln(1 + 2^-8) ~ 3.9e-3 plus fp32 rounding.
"""
from __future__ import annotations

import os
import sys

import numpy as np

FP32_TOL = 1e-4
BF16_REL = 1e-2
ROW_FLOOR = 2.0 ** -14
LSE_BF16 = 5e-3


def oracle_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.contiguous()


def to_host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def check_global(got: np.ndarray, ref: np.ndarray, dtype: str, label: str = "", floor: float = 0.0):
    """``floor`` adds an absolute term to the bf16 bar, for tensors that can
    vanish identically (a gradient that is exactly zero is only zero up to
    fp32 rounding in the kernel)."""
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    refmax = float(np.max(np.abs(ref))) if ref.size else 0.0
    tol = FP32_TOL if dtype == "f32" else BF16_REL * refmax + floor
    log(f"[parity] {label} max_err={err:.3e} tol={tol:.3e} max|ref|={refmax:.3e}")
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    assert err <= tol, f"{label}: max error {err:.3e} > tolerance {tol:.3e}"
    return err, tol


def check_rows(got: np.ndarray, ref: np.ndarray, label: str = ""):
    """Per-row gate; got/ref [..., R, d] (a row is the last axis)."""
    err = np.max(np.abs(got - ref), axis=-1)
    lim = np.maximum(BF16_REL * np.max(np.abs(ref), axis=-1), ROW_FLOOR)
    worst = float(np.max(err / lim)) if err.size else 0.0
    log(f"[parity] {label} per-row worst err/limit={worst:.3f}")
    assert np.all(err <= lim), f"{label}: per-row gate failed (worst ratio {worst:.3f})"


def check_rows_scaled(got: np.ndarray, ref: np.ndarray, mag: np.ndarray, label: str = ""):
    """Per-row gate against a per-row magnitude: got/ref/mag [..., R, d];
    limit max(1e-2 * max_c mag, 2^-14) per row."""
    err = np.max(np.abs(got - ref), axis=-1)
    lim = np.maximum(BF16_REL * np.max(mag, axis=-1), ROW_FLOOR)
    worst = float(np.max(err / lim)) if err.size else 0.0
    log(f"[parity] {label} per-row worst err/limit={worst:.3f}")
    assert np.all(err <= lim), f"{label}: per-row gate failed (worst ratio {worst:.3f})"
