"""Pins for the fp64 oracle: each test ties the oracle to something other than
itself -- a pure-Python brute force written from the group definition, a
library routine (torch SDPA in float64, scipy logsumexp), closed forms and
invariants of softmax attention, and the parameter counts printed on the
SQAT-m model card. A dropped term, wrong sign, wrong K/V head, off-by-one
causal mask or transposed operand in the oracle fails at least one of these.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, attention_param_count, kv_head_index, layer, rope
from synth import bf16_round, draw_attn_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- brute force
def _groups(H_q, H_kv):
    """Query heads split into H_kv contiguous groups of equal size; each group
    shares one K/V head ("GQA ..." page, "The idea")."""
    g = H_q // H_kv
    return [list(range(G * g, (G + 1) * g)) for G in range(H_kv)]


def _brute_attention(q, k, v, scale, causal):
    """Pure-Python loops, math.exp and math.fsum; tiny inputs only."""
    B, H_q, N, d = q.shape
    H_kv = k.shape[1]
    groups = _groups(H_q, H_kv)
    out = np.zeros((B, H_q, N, d))
    for b in range(B):
        for G, members in enumerate(groups):
            for i in members:
                for t in range(N):
                    keys = range(t + 1) if causal else range(N)
                    s = [scale * math.fsum(float(q[b, i, t, c]) * float(k[b, G, u, c])
                                           for c in range(d)) for u in keys]
                    mx = max(s)
                    w = [math.exp(x - mx) for x in s]
                    tot = math.fsum(w)
                    for c in range(d):
                        out[b, i, t, c] = math.fsum(wu * float(v[b, G, u, c])
                                                    for wu, u in zip(w, keys)) / tot
    return out


@pytest.mark.parametrize("B,H_q,H_kv,N,d", [
    (1, 2, 1, 1, 4), (1, 2, 2, 2, 4), (2, 4, 2, 5, 8), (1, 8, 4, 17, 16),
    (1, 4, 1, 33, 4), (1, 4, 4, 9, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_oracle_matches_bruteforce(B, H_q, H_kv, N, d, causal):
    q, k, v = draw_attn_case(B, H_q, H_kv, N, d, "f32", seed=7)
    scale = 1.0 / math.sqrt(d)
    ref = _brute_attention(q, k, v, scale, causal)
    got = attention(q, k, v, scale=scale, causal=causal)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_bruteforce_catches_planted_mistakes():
    """The brute force must disagree with plausible oracle mistakes."""
    q, k, v = draw_attn_case(1, 4, 2, 9, 4, "f32", seed=3)
    ref = _brute_attention(q, k, v, 0.5, True)
    # wrong K/V head (i % H_kv instead of the contiguous group)
    kk = np.ascontiguousarray(k[:, [0, 1, 0, 1]])
    vv = np.ascontiguousarray(v[:, [0, 1, 0, 1]])
    wrong = attention(q, kk, vv, scale=0.5, causal=True)
    assert np.max(np.abs(wrong - ref)) > 1e-3
    # causal mask off by one (diagonal excluded) -> compare against a shifted mask
    assert np.max(np.abs(attention(q, k, v, scale=0.5, causal=False) - ref)) > 1e-3
    # dropped scale
    assert np.max(np.abs(attention(q, k, v, scale=1.0, causal=True) - ref)) > 1e-3


# ------------------------------------------------------------- library routine
@pytest.mark.parametrize("H_q,H_kv", [(4, 4), (8, 4), (8, 1), (16, 4), (4, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_oracle_matches_torch_sdpa_fp64(H_q, H_kv, causal):
    """MHA is torch's SDPA directly; grouped variants are SDPA with each K/V
    head repeated for the g query heads of its group."""
    B, N, d = 2, 70, 16
    q, k, v = draw_attn_case(B, H_q, H_kv, N, d, "bf16", seed=11)
    g = H_q // H_kv
    tq = torch.from_numpy(q).double()
    tk = torch.from_numpy(k).double().repeat_interleave(g, dim=1)
    tv = torch.from_numpy(v).double().repeat_interleave(g, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=0.3).numpy()
    got = attention(q, k, v, scale=0.3, causal=causal)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_lse_matches_scipy_logsumexp():
    from scipy.special import logsumexp
    q, k, v = draw_attn_case(1, 4, 2, 40, 8, "f32", seed=5)
    _, lse = attention(q, k, v, scale=0.4, causal=True, return_lse=True)
    for i in range(4):
        j = i // 2
        s = 0.4 * (q[0, i].astype(np.float64) @ k[0, j].astype(np.float64).T)
        for t in range(40):
            assert abs(lse[0, i, t] - logsumexp(s[t, :t + 1])) <= 1e-12


# ------------------------------------------------------------------ invariants
def test_constant_values_give_constant_output():
    q, k, _ = draw_attn_case(1, 8, 4, 50, 16, "bf16", seed=1)
    v = np.ones((1, 4, 50, 16))
    for causal in (False, True):
        o = attention(q, k, v, causal=causal)
        assert np.max(np.abs(o - 1.0)) <= 1e-14


def test_identity_values_expose_probability_matrix():
    N, d = 12, 16
    q, k, _ = draw_attn_case(1, 2, 1, N, d, "f32", seed=2)
    v = np.zeros((1, 1, N, d))
    v[0, 0, np.arange(N), np.arange(N)] = 1.0          # V[u, c] = delta_uc
    for causal in (False, True):
        p = attention(q, k, v, scale=0.7, causal=causal)[0, :, :, :N]
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-14
        if causal:
            assert np.all(np.triu(p, 1) == 0)
            assert np.all(np.diagonal(p, axis1=1, axis2=2) > 0)


def test_identical_keys_give_mean_of_values():
    N, d = 37, 8
    q, k, v = draw_attn_case(1, 4, 2, N, d, "f32", seed=4)
    k[:] = k[:, :, :1, :]                               # every key equal per head
    o = attention(q, k, v, causal=False)
    for i in range(4):
        assert np.allclose(o[0, i], v[0, i // 2].astype(np.float64).mean(0), atol=1e-14)
    oc = attention(q, k, v, causal=True)
    for i in range(4):
        vv = v[0, i // 2].astype(np.float64)
        prefix = np.cumsum(vv, axis=0) / np.arange(1, N + 1)[:, None]
        assert np.allclose(oc[0, i], prefix, atol=1e-13)


def test_zero_scale_is_uniform_attention():
    q, k, v = draw_attn_case(1, 2, 1, 20, 4, "f32", seed=6)
    o = attention(q, k, v, scale=0.0, causal=True)
    vv = v[0, 0].astype(np.float64)
    prefix = np.cumsum(vv, axis=0) / np.arange(1, 21)[:, None]
    assert np.allclose(o[0, 0], prefix, atol=1e-14)


def test_causal_edges():
    q, k, v = draw_attn_case(1, 4, 2, 30, 8, "f32", seed=8)
    oc = attention(q, k, v, causal=True)
    on = attention(q, k, v, causal=False)
    for i in range(4):
        assert np.allclose(oc[0, i, 0], v[0, i // 2, 0], atol=0)
    assert np.allclose(oc[:, :, -1], on[:, :, -1], atol=1e-14)


def test_single_token_returns_value():
    q, k, v = draw_attn_case(3, 4, 2, 1, 8, "f32", seed=9)
    for causal in (False, True):
        o = attention(q, k, v, causal=causal)
        assert np.allclose(o[:, 0::2, 0], v[:, :, 0], atol=0)
        assert np.allclose(o[:, 1::2, 0], v[:, :, 0], atol=0)


def test_permutation_equivariance_noncausal():
    rng = np.random.default_rng(0)
    q, k, v = draw_attn_case(1, 4, 2, 25, 8, "f32", seed=10)
    o = attention(q, k, v)
    pq = rng.permutation(25)
    assert np.allclose(attention(q[:, :, pq], k, v), o[:, :, pq], atol=1e-14)
    pk = rng.permutation(25)
    assert np.allclose(attention(q, k[:, :, pk], v[:, :, pk]), o, atol=1e-14)


def test_key_shift_invariance():
    q, k, v = draw_attn_case(1, 4, 2, 31, 8, "f32", seed=12)
    w = np.random.default_rng(3).standard_normal(8)
    for causal in (False, True):
        a = attention(q, k, v, causal=causal)
        b = attention(q, k + w, v, causal=causal)
        assert np.max(np.abs(a - b)) <= 1e-12


def test_linear_in_values():
    q, k, v = draw_attn_case(1, 4, 2, 23, 8, "f32", seed=13)
    v = v.astype(np.float64)
    v2 = np.random.default_rng(4).standard_normal(v.shape)
    a, b = 0.7, -1.9
    for causal in (False, True):
        lhs = attention(q, k, a * v + b * v2, causal=causal)
        rhs = a * attention(q, k, v, causal=causal) + b * attention(q, k, v2, causal=causal)
        assert np.max(np.abs(lhs - rhs)) <= 1e-12


def test_head_independence_and_mapping():
    """Head i of SQA equals single-head attention on (Q_i, K_kv(i), V_kv(i))."""
    q, k, v = draw_attn_case(2, 8, 4, 19, 8, "bf16", seed=14)
    o = attention(q, k, v, causal=True)
    for b in range(2):
        for i in range(8):
            j = kv_head_index(i, 8, 4)
            single = attention(q[b:b + 1, i:i + 1], k[b:b + 1, j:j + 1],
                               v[b:b + 1, j:j + 1], causal=True)
            assert np.array_equal(single[0, 0], o[b, i])


def test_kv_mapping_special_cases():
    # GQA-1 is MQA, GQA-H is MHA ("GQA ..." page, "The idea"); contiguous groups
    assert [kv_head_index(i, 16, 1) for i in range(16)] == [0] * 16
    assert [kv_head_index(i, 16, 16) for i in range(16)] == list(range(16))
    for H_q, H_kv in [(8, 4), (16, 4), (8, 2), (16, 8)]:
        g = H_q // H_kv
        assert [kv_head_index(i, H_q, H_kv) for i in range(H_q)] == [i // g for i in range(H_q)]
        groups = _groups(H_q, H_kv)
        for G, members in enumerate(groups):
            assert all(kv_head_index(i, H_q, H_kv) == G for i in members)


def test_rows_subset_and_threads_consistent():
    q, k, v = draw_attn_case(1, 4, 2, 300, 16, "bf16", seed=15)
    full = attention(q, k, v, causal=True)
    rows = np.array([0, 1, 63, 64, 150, 299])
    sub = attention(q, k, v, causal=True, rows=rows, chunk_elems=600, threads=3)
    assert np.array_equal(sub, full[:, :, rows])


def test_mqa_reduces_to_repeated_single_head():
    q, k, v = draw_attn_case(1, 4, 1, 15, 8, "f32", seed=16)
    o = attention(q, k, v, causal=False)
    for i in range(4):
        assert np.array_equal(o[0, i], attention(q[:, i:i + 1], k, v)[0, 0])


# -------------------------------------------------------------------- RoPE
def test_rope_explicit_values():
    d = 16
    x = np.zeros((2, d))
    x[:, 0] = 1.0                                       # e_0 at positions 0 and 1
    y = rope(x, 10000.0)
    assert np.allclose(y[0], x[0], atol=0)              # identity at t = 0
    # theta_0 = 1: the pair (0, d/2) rotates by one radian at t = 1
    assert abs(y[1, 0] - math.cos(1.0)) < 1e-15
    assert abs(y[1, d // 2] - math.sin(1.0)) < 1e-15
    assert np.count_nonzero(y[1]) == 2
    # last pair: theta = base^(-2(h-1)/d)
    x2 = np.zeros((4, d))
    x2[:, d // 2 - 1] = 1.0
    y2 = rope(x2, 10000.0)
    th = 10000.0 ** (-2.0 * (d // 2 - 1) / d)
    assert abs(y2[3, d // 2 - 1] - math.cos(3 * th)) < 1e-15
    assert abs(y2[3, d - 1] - math.sin(3 * th)) < 1e-15


def test_rope_is_complex_rotation():
    """Independent form: pair c is the complex number x_c + i x_{c+d/2},
    multiplied by exp(i t theta_c)."""
    rng = np.random.default_rng(5)
    N, d, base = 9, 16, 500.0
    x = rng.standard_normal((N, d))
    y = rope(x, base)
    for t in range(N):
        for c in range(d // 2):
            z = complex(x[t, c], x[t, c + d // 2]) * cmath.exp(1j * t * base ** (-2 * c / d))
            assert abs(y[t, c] - z.real) < 1e-13 and abs(y[t, c + d // 2] - z.imag) < 1e-13


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(6)
    N, d = 40, 16
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    rq = rope(np.tile(q, (N, 1)), 10000.0)
    rk = rope(np.tile(k, (N, 1)), 10000.0)
    assert np.allclose(np.linalg.norm(rq, axis=1), np.linalg.norm(q), atol=1e-12)
    for t, s in [(5, 2), (17, 17), (39, 0), (3, 30)]:
        lhs = rq[t] @ rk[s]
        if t >= s:
            rhs = rq[t - s] @ k
        else:
            rhs = q @ rk[s - t]
        assert abs(lhs - rhs) < 1e-11


def test_rope_rotate_half_equals_interleaved_under_column_permutation():
    """Interleaved pairs (2c, 2c+1) give the same layer output once the W_Q/W_K
    columns are permuted; so the pairing choice cannot change Y's values."""
    rng = np.random.default_rng(7)
    B, N, D, H, Hq, Hkv = 1, 11, 32, 2, 2, 1
    d = D // H
    x = bf16_round(rng.standard_normal((B, N, D)).astype(np.float32))
    wq = rng.standard_normal((D, Hq * d)) * 0.1
    wk = rng.standard_normal((D, Hkv * d)) * 0.1
    wv = rng.standard_normal((D, Hkv * d)) * 0.1
    wo = rng.standard_normal((Hq * d, D)) * 0.1
    y = layer(x, wq, wk, wv, wo, H, Hq, Hkv, rope_base=100.0)

    def interleaved_rope(z):
        t = np.arange(z.shape[-2])[:, None]
        th = 100.0 ** (-2.0 * np.arange(d // 2) / d)
        c, s = np.cos(t * th), np.sin(t * th)
        a, b = z[..., 0::2], z[..., 1::2]
        out = np.empty_like(z)
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = a * s + b * c
        return out

    # per head, interleaved slot 2c holds rotate-half column c, 2c+1 holds c+d/2
    perm_head = np.empty(d, dtype=int)
    perm_head[0::2] = np.arange(d // 2)
    perm_head[1::2] = np.arange(d // 2) + d // 2

    def permute_cols(w, nh):
        return np.concatenate([w[:, h * d + perm_head] for h in range(nh)], axis=1)

    wq2, wk2 = permute_cols(wq, Hq), permute_cols(wk, Hkv)
    xx = x.astype(np.float64)
    qh = interleaved_rope((xx @ wq2).reshape(B, N, Hq, d).transpose(0, 2, 1, 3))
    kh = interleaved_rope((xx @ wk2).reshape(B, N, Hkv, d).transpose(0, 2, 1, 3))
    vh = (xx @ wv).reshape(B, N, Hkv, d).transpose(0, 2, 1, 3)
    o = attention(qh, kh, vh, causal=True)
    y2 = o.transpose(0, 2, 1, 3).reshape(B, N, Hq * d) @ wo
    assert np.max(np.abs(y - y2)) < 1e-12


# -------------------------------------------------------------------- layer
def test_layer_zero_query_projection_closed_form():
    """W_Q = 0: all scores vanish, causal attention becomes a prefix mean and
    RoPE drops out: Y = prefix_mean(X W_V) W_O per head."""
    rng = np.random.default_rng(8)
    B, N, D, H, Hq, Hkv = 2, 13, 64, 4, 2, 1
    d = D // H
    x = rng.standard_normal((B, N, D))
    wq = np.zeros((D, Hq * d))
    wk = rng.standard_normal((D, Hkv * d))
    wv = rng.standard_normal((D, Hkv * d))
    wo = rng.standard_normal((Hq * d, D))
    y = layer(x, wq, wk, wv, wo, H, Hq, Hkv)
    vx = x @ wv                                                     # [B,N,d]
    pm = np.cumsum(vx, axis=1) / np.arange(1, N + 1)[None, :, None]
    o_flat = np.concatenate([pm] * Hq, axis=-1)                     # both heads read kv 0
    assert np.max(np.abs(y - o_flat @ wo)) < 1e-11


def _brute_layer(x, wq, wk, wv, wo, H, Hq, Hkv, base):
    """Pure-Python layer with complex-number RoPE, for tiny shapes."""
    B, N, D = x.shape
    d = D // H
    out = np.zeros((B, N, D))
    groups = _groups(Hq, Hkv)

    def proj(w, b, t, col):
        return math.fsum(float(x[b, t, e]) * float(w[e, col]) for e in range(D))

    def roped(w, b, t, h):
        v = [proj(w, b, t, h * d + c) for c in range(d)]
        r = [0.0] * d
        for c in range(d // 2):
            z = complex(v[c], v[c + d // 2]) * cmath.exp(1j * t * base ** (-2 * c / d))
            r[c], r[c + d // 2] = z.real, z.imag
        return r

    for b in range(B):
        o_flat = [[0.0] * (Hq * d) for _ in range(N)]
        for G, members in enumerate(groups):
            ks = [roped(wk, b, u, G) for u in range(N)]
            vs = [[proj(wv, b, u, G * d + c) for c in range(d)] for u in range(N)]
            for i in members:
                for t in range(N):
                    qv = roped(wq, b, t, i)
                    s = [math.fsum(a * c for a, c in zip(qv, ks[u])) / math.sqrt(d)
                         for u in range(t + 1)]
                    mx = max(s)
                    w = [math.exp(z - mx) for z in s]
                    tot = math.fsum(w)
                    for c in range(d):
                        o_flat[t][i * d + c] = math.fsum(w[u] * vs[u][c] for u in range(t + 1)) / tot
        for t in range(N):
            for e in range(D):
                out[b, t, e] = math.fsum(o_flat[t][f] * float(wo[f, e]) for f in range(Hq * d))
    return out


def test_layer_matches_bruteforce():
    rng = np.random.default_rng(9)
    B, N, D, H, Hq, Hkv = 1, 6, 16, 4, 2, 1
    d = D // H
    x = rng.standard_normal((B, N, D))
    wq = rng.standard_normal((D, Hq * d)) * 0.5
    wk = rng.standard_normal((D, Hkv * d)) * 0.5
    wv = rng.standard_normal((D, Hkv * d)) * 0.5
    wo = rng.standard_normal((Hq * d, D)) * 0.5
    y = layer(x, wq, wk, wv, wo, H, Hq, Hkv, rope_base=10.0)
    ref = _brute_layer(x, wq, wk, wv, wo, H, Hq, Hkv, 10.0)
    assert np.max(np.abs(y - ref)) < 1e-12


def test_layer_rejects_wrong_shapes():
    x = np.zeros((1, 4, 32))
    with pytest.raises(ValueError):
        layer(x, np.zeros((32, 32)), np.zeros((32, 8)), np.zeros((32, 8)), np.zeros((16, 32)),
              4, 2, 1)


# ------------------------------------------------------- printed model sizes
def test_param_counts_match_model_card():
    """Per-layer projection widths H_q*d (Q, O) and H_kv*d (K, V) with d = D/H
    reproduce the differences between the printed SQAT-m model sizes."""
    with open(os.path.join(GOLDEN, "sqatm_param_counts.json")) as f:
        g = json.load(f)
    arch = g["architecture"]
    D, L, H = arch["d_model"], arch["layers"], arch["heads_for_dimension_split"]
    tol = g["difference_tolerance_M"]
    counts = {n: L * attention_param_count(D, H, v["H_q"], v["H_kv"]) / 1e6
              for n, v in g["variants"].items()}
    names = list(counts)
    for a in names:
        for b in names:
            printed = g["variants"][a]["printed_params_M"] - g["variants"][b]["printed_params_M"]
            assert abs((counts[a] - counts[b]) - printed) <= tol + 1e-9, (a, b)
    # exact per-layer figures for the record
    assert attention_param_count(256, 16, 16, 16) == 262144
    assert attention_param_count(256, 16, 8, 4) == 98304
    # a layer that kept W_O at full width would miss the printed SQA size
    wrong = L * (attention_param_count(256, 16, 8, 4) + 128 * 256) / 1e6
    assert abs((counts["MHA"] - wrong) - (12.0 - 10.7)) > tol
