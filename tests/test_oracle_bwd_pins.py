"""Pins for the fp64 backward oracle (``oracle.attention_bwd``).

Each test ties the gradients to something other than the backward code itself:
central finite differences of the (separately pinned) forward oracle, torch
autograd through torch's own float64 attention, and closed forms that follow
from softmax attention (shift invariance, rows of P summing to one, scale 0,
N = 1, linearity). A dropped term, wrong scale, unnormalised P, mask off by
one or missing group sum in the backward fails at least one of them; the last
test plants such mistakes in the oracle and checks that they are caught.
"""
import math

import numpy as np
import pytest
import torch

import oracle.sqa_oracle as so
from oracle import attention, attention_bwd
from synth import draw_attn_case


def _fd_grads(q, k, v, g, scale, causal, h=1e-5):
    """Central differences of L = sum(attention(q, k, v) * g) for every
    element of q, k and v (float64, tiny inputs only)."""
    def loss(qq, kk, vv):
        return float((attention(qq, kk, vv, scale=scale, causal=causal) * g).sum())

    out = []
    for which in range(3):
        base = [q.astype(np.float64).copy(), k.astype(np.float64).copy(), v.astype(np.float64).copy()]
        grad = np.zeros_like(base[which])
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            grad[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        out.append(grad)
    return out


def _check_against_fd(q, k, v, g, scale, causal, tol=1e-7):
    dq, dk, dv = attention_bwd(q, k, v, g, scale=scale, causal=causal)
    fq, fk, fv = _fd_grads(q, k, v, g, scale, causal)
    for got, ref in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.max(np.abs(got - ref)) <= tol * max(1.0, np.max(np.abs(ref)))


# ------------------------------------------------------- finite differences
@pytest.mark.parametrize("H_q,H_kv", [(2, 2), (4, 2), (4, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_finite_differences(H_q, H_kv, causal):
    q, k, v = draw_attn_case(1, H_q, H_kv, 5, 3, "f32", seed=21)
    g = np.random.default_rng(22).standard_normal(q.shape)
    _check_against_fd(q, k, v, g, 0.7, causal)


def test_bwd_matches_finite_differences_negative_scale_batch2():
    q, k, v = draw_attn_case(2, 2, 1, 4, 2, "f32", seed=23)
    g = np.random.default_rng(24).standard_normal(q.shape)
    _check_against_fd(q, k, v, g, -1.3, True)


# ------------------------------------------------------------ torch autograd
@pytest.mark.parametrize("H_q,H_kv", [(4, 4), (8, 4), (8, 1), (4, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_torch_autograd_fp64(H_q, H_kv, causal):
    """torch's float64 SDPA with each K/V head repeated for its group; autograd
    sums the repeated heads' gradients, which is the group sum."""
    B, N, d = 2, 37, 16
    q, k, v = draw_attn_case(B, H_q, H_kv, N, d, "bf16", seed=25)
    gr = np.random.default_rng(26).standard_normal(q.shape)
    grp = H_q // H_kv
    tq = torch.from_numpy(q).double().requires_grad_(True)
    tk = torch.from_numpy(k).double().requires_grad_(True)
    tv = torch.from_numpy(v).double().requires_grad_(True)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(grp, dim=1), tv.repeat_interleave(grp, dim=1),
        is_causal=causal, scale=0.3)
    o.backward(torch.from_numpy(gr))
    dq, dk, dv = attention_bwd(q, k, v, gr, scale=0.3, causal=causal)
    assert np.max(np.abs(dq - tq.grad.numpy())) <= 1e-11
    assert np.max(np.abs(dk - tk.grad.numpy())) <= 1e-11
    assert np.max(np.abs(dv - tv.grad.numpy())) <= 1e-11


# ------------------------------------------------- closed forms, invariants
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_value_grad_column_sums_with_unit_upstream(causal):
    """dO = 1: every row of P sums to 1, so each column of dV_j sums to g*N."""
    H_q, H_kv, N = 8, 2, 23
    q, k, v = draw_attn_case(1, H_q, H_kv, N, 8, "f32", seed=27)
    _, _, dv = attention_bwd(q, k, v, np.ones(q.shape), scale=0.5, causal=causal)
    assert np.allclose(dv.sum(axis=2), (H_q // H_kv) * N, rtol=0, atol=1e-10)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_key_grads_sum_to_zero(causal):
    """Softmax is invariant to adding a constant to a row's scores, so every
    row of dS sums to zero and the key gradients of a head sum to zero."""
    q, k, v = draw_attn_case(1, 4, 2, 19, 8, "f32", seed=28)
    g = np.random.default_rng(29).standard_normal(q.shape)
    _, dk, _ = attention_bwd(q, k, v, g, scale=0.6, causal=causal)
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12 * max(1.0, np.abs(dk).max()) * 19


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_zero_scale_closed_form(causal):
    """scale 0: P is uniform over the visible keys, dQ = dK = 0 and
    dV_u = sum over the group's heads of sum_{t sees u} dO_t / |U_t|."""
    H_q, H_kv, N, d = 4, 2, 11, 4
    q, k, v = draw_attn_case(1, H_q, H_kv, N, d, "f32", seed=30)
    g = np.random.default_rng(31).standard_normal(q.shape)
    dq, dk, dv = attention_bwd(q, k, v, g, scale=0.0, causal=causal)
    assert np.max(np.abs(dq)) == 0.0 and np.max(np.abs(dk)) == 0.0
    ref = np.zeros_like(dv)
    for i in range(H_q):
        j = i // (H_q // H_kv)
        for t in range(N):
            vis = range(t + 1) if causal else range(N)
            for u in vis:
                ref[0, j, u] += g[0, i, t] / len(vis)
    assert np.max(np.abs(dv - ref)) <= 1e-12


def test_bwd_single_token():
    """N = 1: P = [1], so dS = 0 (dQ = dK = 0) and dV = sum of dO over the group."""
    q, k, v = draw_attn_case(2, 6, 2, 1, 8, "f32", seed=32)
    g = np.random.default_rng(33).standard_normal(q.shape)
    dq, dk, dv = attention_bwd(q, k, v, g, scale=0.9, causal=False)
    assert np.max(np.abs(dq)) <= 1e-14 and np.max(np.abs(dk)) <= 1e-14
    ref = g.reshape(2, 2, 3, 1, 8).sum(axis=2)
    assert np.max(np.abs(dv - ref)) <= 1e-14


def test_bwd_linear_in_upstream_and_rows_and_threads():
    q, k, v = draw_attn_case(1, 4, 2, 40, 8, "bf16", seed=34)
    rng = np.random.default_rng(35)
    g1 = rng.standard_normal(q.shape)
    g2 = rng.standard_normal(q.shape)
    a = attention_bwd(q, k, v, g1, scale=0.4, causal=True)
    b = attention_bwd(q, k, v, g2, scale=0.4, causal=True)
    c = attention_bwd(q, k, v, 2.0 * g1 - 3.0 * g2, scale=0.4, causal=True)
    for x, y, z in zip(a, b, c):
        assert np.max(np.abs(z - (2.0 * x - 3.0 * y))) <= 1e-12 * max(1.0, np.abs(z).max())
    rows = np.array([0, 3, 17, 39])
    dq_rows, none_k, none_v = attention_bwd(q, k, v, g1, scale=0.4, causal=True, rows=rows)
    assert none_k is None and none_v is None
    assert np.array_equal(dq_rows, a[0][:, :, rows])
    t = attention_bwd(q, k, v, g1, scale=0.4, causal=True, threads=4, chunk_elems=64)
    for x, y in zip(a, t):
        assert np.max(np.abs(x - y)) <= 1e-13 * max(1.0, np.abs(x).max())


# ------------------------------------------------------- planted mistakes
def _mutant(kind):
    def f(q_rows, t_rows, kj, vj, do_rows, scale, causal, absolute=False, o_rows=None):
        s = (q_rows @ kj.T) * scale
        if causal:
            u = np.arange(kj.shape[0])
            vis = (u[None, :] < t_rows[:, None]) | (u[None, :] == 0) if kind == "mask" \
                else u[None, :] <= t_rows[:, None]
            s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / e.sum(axis=1, keepdims=True)
        dp = do_rows @ vj.T
        if kind == "no_rowsum":
            ds = p * dp
        else:
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq = ds @ kj * (1.0 if kind == "dq_scale" else scale)
        dk_part = ds.T @ q_rows * scale
        dv_part = (e if kind == "unnormalised" else p).T @ do_rows
        return dq, dk_part, dv_part
    return f


@pytest.mark.parametrize("kind", ["no_rowsum", "dq_scale", "unnormalised", "mask"])
def test_finite_differences_catch_planted_mistakes(kind, monkeypatch):
    q, k, v = draw_attn_case(1, 4, 2, 5, 3, "f32", seed=36)
    g = np.random.default_rng(37).standard_normal(q.shape)
    monkeypatch.setattr(so, "_attend_rows_bwd", _mutant(kind))
    with pytest.raises(AssertionError):
        _check_against_fd(q, k, v, g, 0.7, True)


# ---------------------------------------- absolute-term magnitudes (tolerances)
def _abs_terms_brute(q, k, v, g, scale, causal):
    """sum |dS_tu| |K_uc| etc. by explicit loops over every term (tiny N)."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    aq = np.zeros(q.shape)
    ak = np.zeros(k.shape)
    av = np.zeros(v.shape)
    for b in range(B):
        for i in range(Hq):
            j = (i * Hkv) // Hq
            for t in range(N):
                us = [u for u in range(N) if (not causal or u <= t)]
                s = [scale * sum(float(q[b, i, t, c]) * float(k[b, j, u, c]) for c in range(d)) for u in us]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = math.fsum(e)
                p = [x / z for x in e]
                dp = [sum(float(g[b, i, t, c]) * float(v[b, j, u, c]) for c in range(d)) for u in us]
                D = math.fsum(pp * x for pp, x in zip(p, dp))
                for n, u in enumerate(us):
                    ds = p[n] * (dp[n] - D)
                    for c in range(d):
                        aq[b, i, t, c] += abs(scale) * abs(ds) * abs(float(k[b, j, u, c]))
                        ak[b, j, u, c] += abs(scale) * abs(ds) * abs(float(q[b, i, t, c]))
                        av[b, j, u, c] += p[n] * abs(float(g[b, i, t, c]))
    return aq, ak, av


@pytest.mark.parametrize("H_q,H_kv", [(2, 2), (4, 2), (3, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_absolute_terms_match_brute_force(H_q, H_kv, causal):
    q, k, v = draw_attn_case(2, H_q, H_kv, 6, 4, "f32", seed=31)
    g = np.random.default_rng(32).standard_normal(q.shape)
    got = attention_bwd(q, k, v, g, scale=-0.6, causal=causal, absolute=True)
    ref = _abs_terms_brute(q, k, v, g, -0.6, causal)
    for a, r in zip(got, ref):
        assert np.max(np.abs(a - r)) <= 1e-12 * max(1.0, np.max(np.abs(r)))


def test_bwd_absolute_terms_bound_the_gradients():
    q, k, v = draw_attn_case(1, 8, 4, 200, 16, "f32", seed=33)
    g = np.random.default_rng(34).standard_normal(q.shape)
    for causal in (False, True):
        grads = attention_bwd(q, k, v, g, scale=0.25, causal=causal)
        mags = attention_bwd(q, k, v, g, scale=0.25, causal=causal, absolute=True)
        for gr, mg in zip(grads, mags):
            assert np.all(np.abs(gr) <= mg * (1 + 1e-12) + 1e-15)
        # a non-negative upstream gradient makes every dV term non-negative
        gp = np.abs(g)
        dv = attention_bwd(q, k, v, gp, scale=0.25, causal=causal)[2]
        dv_abs = attention_bwd(q, k, v, gp, scale=0.25, causal=causal, absolute=True)[2]
        assert np.allclose(dv, dv_abs, rtol=1e-12, atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_given_exact_forward_output_is_the_gradient(causal):
    """D from a given forward output equals D = rowsum(P * dP) when that
    output is the exact one; a perturbed output moves every dQ row along
    scale * sum_u P_tu K_u by exactly -delta(D_t) (dS gains -P delta(D))."""
    q, k, v = draw_attn_case(1, 4, 2, 40, 8, "f32", seed=41)
    g = np.random.default_rng(42).standard_normal(q.shape)
    o = attention(q, k, v, scale=0.3, causal=causal)
    a = attention_bwd(q, k, v, g, scale=0.3, causal=causal)
    b = attention_bwd(q, k, v, g, scale=0.3, causal=causal, o=o)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) <= 1e-12 * max(1.0, np.max(np.abs(x)))
    delta = np.random.default_rng(43).standard_normal(o.shape) * 1e-3
    c = attention_bwd(q, k, v, g, scale=0.3, causal=causal, o=o + delta)
    dD = (g * delta).sum(-1)                                   # [B, H, N]
    kr = np.repeat(k, 2, axis=1)                               # K of each query head's group
    pk = attention(q, kr, kr, scale=0.3, causal=causal)        # sum_u P_tu K_u per row
    expect = a[0] - 0.3 * dD[..., None] * pk
    assert np.max(np.abs(c[0] - expect)) <= 1e-10
