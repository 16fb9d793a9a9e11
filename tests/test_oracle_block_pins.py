"""Pins for the fp64 block oracle (``oracle.rms_norm``, ``oracle.swiglu``,
``oracle.block``): library routines (torch's rms_norm and silu in float64,
scipy's expit), closed forms (unit RMS rows, scale invariance, a vanishing
gate or output projection), the pre-norm residual structure, and a
pure-Python brute force of a tiny block built on the brute-force layer of the
forward pins.
"""
import math

import numpy as np
import pytest
import torch

from oracle import block, layer, rms_norm, swiglu
from synth import draw_block
from tests.test_oracle_pins import _brute_layer


# ---------------------------------------------------------------- RMSNorm
def test_rms_norm_matches_torch_fp64():
    rng = np.random.default_rng(40)
    x = rng.standard_normal((3, 7, 48)) * 2.5
    w = 1.0 + 0.1 * rng.standard_normal(48)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (48,), torch.from_numpy(w), eps=1e-6).numpy()
    assert np.max(np.abs(rms_norm(x, w, 1e-6) - ref)) <= 1e-12


def test_rms_norm_closed_forms():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((5, 64))
    ones = np.ones(64)
    y = rms_norm(x, ones, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-14)   # unit RMS rows
    assert np.allclose(rms_norm(7.0 * x, ones, eps=0.0), y, atol=1e-14)    # scale invariance
    # a constant row c maps to sign(c) * weight
    w = rng.standard_normal(64)
    assert np.allclose(rms_norm(np.full((1, 64), -3.0), w, eps=0.0)[0], -w, atol=1e-14)


# ---------------------------------------------------------------- SwiGLU
def test_swiglu_matches_torch_silu_fp64():
    rng = np.random.default_rng(42)
    z = rng.standard_normal((4, 9, 32))
    wg, wu, wd = (rng.standard_normal(s) * 0.3 for s in ((32, 40), (32, 40), (40, 32)))
    tz = torch.from_numpy(z)
    ref = ((torch.nn.functional.silu(tz @ torch.from_numpy(wg)) * (tz @ torch.from_numpy(wu)))
           @ torch.from_numpy(wd)).numpy()
    assert np.max(np.abs(swiglu(z, wg, wu, wd) - ref)) <= 1e-12


def test_swiglu_closed_forms():
    from scipy.special import expit
    rng = np.random.default_rng(43)
    z = rng.standard_normal((6, 16))
    wu, wd = rng.standard_normal((16, 8)), rng.standard_normal((8, 16))
    # silu(0) = 0: a zero gate projection kills the feed forward
    assert np.max(np.abs(swiglu(z, np.zeros((16, 8)), wu, wd))) == 0.0
    # identity gate/up/down on one coordinate: silu(a)*b through a one-hot path
    wg1 = np.zeros((16, 1)); wg1[0, 0] = 1.0
    wu1 = np.zeros((16, 1)); wu1[1, 0] = 1.0
    wd1 = np.zeros((1, 16)); wd1[0, 2] = 1.0
    got = swiglu(z, wg1, wu1, wd1)[:, 2]
    ref = z[:, 0] * expit(z[:, 0]) * z[:, 1]
    assert np.max(np.abs(got - ref)) <= 1e-14


# ---------------------------------------------------------------- block
def _blk(seed=44, B=2, N=9, D=32, H=4, Hq=2, Hkv=1, F=40):
    return draw_block(B, N, D, H, Hq, Hkv, F, seed=seed), (H, Hq, Hkv)


def test_block_zero_output_projections_is_identity():
    (x, n1, wq, wk, wv, wo, n2, wg, wu, wd), (H, Hq, Hkv) = _blk()
    y = block(x, n1, wq, wk, wv, np.zeros_like(wo), n2, wg, wu, np.zeros_like(wd), H, Hq, Hkv)
    assert np.array_equal(y, x.astype(np.float64))


def test_block_attention_and_feed_forward_parts():
    (x, n1, wq, wk, wv, wo, n2, wg, wu, wd), (H, Hq, Hkv) = _blk(seed=45)
    x64 = x.astype(np.float64)
    # W_down = 0: only the attention sub-layer remains
    y = block(x, n1, wq, wk, wv, wo, n2, wg, wu, np.zeros_like(wd), H, Hq, Hkv, scale=0.3)
    ref = x64 + layer(rms_norm(x, n1), wq, wk, wv, wo, H, Hq, Hkv, scale=0.3)
    assert np.max(np.abs(y - ref)) <= 1e-12
    # W_O = 0: h = x and only the feed forward remains
    y = block(x, n1, wq, wk, wv, np.zeros_like(wo), n2, wg, wu, wd, H, Hq, Hkv, scale=0.3)
    ref = x64 + swiglu(rms_norm(x, n2), wg, wu, wd)
    assert np.max(np.abs(y - ref)) <= 1e-12


def _brute_block(x, n1, wq, wk, wv, wo, n2, wg, wu, wd, H, Hq, Hkv, eps):
    """Pure-Python loops (math.fsum, math.exp) around the brute-force layer."""
    B, N, D = x.shape
    F = wg.shape[1]

    def norm(a, g):
        out = np.zeros_like(a, dtype=np.float64)
        for b in range(B):
            for t in range(N):
                ms = math.fsum(float(a[b, t, c]) ** 2 for c in range(D)) / D
                r = 1.0 / math.sqrt(ms + eps)
                for c in range(D):
                    out[b, t, c] = float(a[b, t, c]) * r * float(g[c])
        return out

    h = x.astype(np.float64) + _brute_layer(norm(x, n1), wq, wk, wv, wo, H, Hq, Hkv, 10000.0)
    z = norm(h, n2)
    y = h.copy()
    for b in range(B):
        for t in range(N):
            act = []
            for f in range(F):
                gv = math.fsum(z[b, t, c] * float(wg[c, f]) for c in range(D))
                uv = math.fsum(z[b, t, c] * float(wu[c, f]) for c in range(D))
                act.append(gv / (1.0 + math.exp(-gv)) * uv)
            for c in range(D):
                y[b, t, c] += math.fsum(act[f] * float(wd[f, c]) for f in range(F))
    return y


def test_block_matches_bruteforce():
    (x, n1, wq, wk, wv, wo, n2, wg, wu, wd), (H, Hq, Hkv) = _blk(seed=46, B=1, N=5, D=16, F=12)
    d = 16 // H
    y = block(x, n1, wq, wk, wv, wo, n2, wg, wu, wd, H, Hq, Hkv, scale=1.0 / math.sqrt(d), eps=1e-6)
    ref = _brute_block(x, n1, wq, wk, wv, wo, n2, wg, wu, wd, H, Hq, Hkv, 1e-6)
    assert np.max(np.abs(y - ref)) <= 1e-10


def test_block_rejects_wrong_feed_forward_shapes():
    (x, n1, wq, wk, wv, wo, n2, wg, wu, wd), (H, Hq, Hkv) = _blk()
    with pytest.raises(ValueError):
        block(x, n1, wq, wk, wv, wo, n2, wg, wu, wd.T, H, Hq, Hkv)
