"""Pins for the oracle on the wider shape family: head dims 32 and 128,
query-head counts that H_kv does not divide (the general floor(i*H_kv/H_q)
grouping), and packed variable-length batches (``attention_varlen``).

Each ties the oracle to something other than itself: hand-enumerated head
maps, a pure-Python brute force whose groups are defined by an inequality
rather than the floor formula, torch's SDPA in float64 with an explicit
block-diagonal mask, scipy's logsumexp, and invariants of packing.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, attention_varlen, kv_head_index
from synth import draw_attn_case, draw_varlen

# floor(i * H_kv / H_q) worked out by hand for every query head i
HAND_MAPS = {
    (6, 4): [0, 0, 1, 2, 2, 3],       # i*4/6 = 0, .67, 1.33, 2, 2.67, 3.33
    (5, 2): [0, 0, 0, 1, 1],          # i*2/5 = 0, .4, .8, 1.2, 1.6
    (7, 3): [0, 0, 0, 1, 1, 2, 2],    # i*3/7 = 0, .43, .86, 1.29, 1.71, 2.14, 2.57
    (3, 2): [0, 0, 1],                # i*2/3 = 0, .67, 1.33
    (12, 8): [0, 0, 1, 2, 2, 3, 4, 4, 5, 6, 6, 7],
}


@pytest.mark.parametrize("hq_hkv", sorted(HAND_MAPS))
def test_kv_head_index_matches_hand_tables(hq_hkv):
    H_q, H_kv = hq_hkv
    assert [kv_head_index(i, H_q, H_kv) for i in range(H_q)] == HAND_MAPS[hq_hkv]


def _members(G, H_q, H_kv):
    """Query heads of group G: G*H_q <= i*H_kv < (G+1)*H_q."""
    return [i for i in range(H_q) if G * H_q <= i * H_kv < (G + 1) * H_q]


def _brute_packed(q, k, v, cu, scale, causal):
    """Pure-Python loops (math.exp, math.fsum) over packed sequences:
    q [H_q, T, d], k/v [H_kv, T, d]; tiny inputs only."""
    H_q, T, d = q.shape
    H_kv = k.shape[0]
    out = np.zeros((H_q, T, d))
    for a, b in zip(cu, cu[1:]):
        for G in range(H_kv):
            for i in _members(G, H_q, H_kv):
                for t in range(a, b):
                    keys = range(a, t + 1) if causal else range(a, b)
                    s = [scale * math.fsum(float(q[i, t, c]) * float(k[G, u, c]) for c in range(d))
                         for u in keys]
                    mx = max(s)
                    w = [math.exp(x - mx) for x in s]
                    tot = math.fsum(w)
                    for c in range(d):
                        out[i, t, c] = math.fsum(wu * float(v[G, u, c]) for wu, u in zip(w, keys)) / tot
    return out


def test_group_membership_brute_force_covers_every_head():
    for (H_q, H_kv), table in HAND_MAPS.items():
        seen = sorted(i for G in range(H_kv) for i in _members(G, H_q, H_kv))
        assert seen == list(range(H_q))
        for G in range(H_kv):
            assert _members(G, H_q, H_kv) == [i for i in range(H_q) if table[i] == G]


# ------------------------------------------------ uneven groups, dense layout
@pytest.mark.parametrize("H_q,H_kv", [(6, 4), (5, 2), (7, 3), (3, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_uneven_groups_match_bruteforce(H_q, H_kv, causal):
    q, k, v = draw_attn_case(2, H_q, H_kv, 11, 8, "f32", seed=H_q * 10 + H_kv)
    got = attention(q, k, v, scale=0.35, causal=causal)
    for b in range(2):
        ref = _brute_packed(q[b], k[b], v[b], [0, 11], 0.35, causal)
        assert np.max(np.abs(got[b] - ref)) <= 1e-12


@pytest.mark.parametrize("hq_hkv", [(6, 4), (5, 2), (12, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_uneven_groups_match_torch_sdpa_fp64(hq_hkv, causal):
    """SDPA on K/V heads gathered by the hand-enumerated map."""
    H_q, H_kv = hq_hkv
    q, k, v = draw_attn_case(2, H_q, H_kv, 50, 16, "bf16", seed=21)
    idx = torch.tensor(HAND_MAPS[hq_hkv])
    tk = torch.from_numpy(k).double().index_select(1, idx)
    tv = torch.from_numpy(v).double().index_select(1, idx)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).double(), tk, tv, is_causal=causal, scale=0.25).numpy()
    got = attention(q, k, v, scale=0.25, causal=causal)
    assert np.max(np.abs(got - ref)) <= 1e-12


# ------------------------------------------------------------- head dims
@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dims_32_128_match_bruteforce_and_sdpa(d, causal):
    q, k, v = draw_attn_case(1, 4, 2, 9, d, "f32", seed=d)
    scale = 1.0 / math.sqrt(d)
    got = attention(q, k, v, scale=scale, causal=causal)
    ref = _brute_packed(q[0], k[0], v[0], [0, 9], scale, causal)
    assert np.max(np.abs(got[0] - ref)) <= 1e-12
    tq = torch.from_numpy(q).double()
    tk = torch.from_numpy(k).double().repeat_interleave(2, dim=1)
    tv = torch.from_numpy(v).double().repeat_interleave(2, dim=1)
    sd = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal).numpy()
    assert np.max(np.abs(attention(q, k, v, causal=causal) - sd)) <= 1e-12   # default scale 1/sqrt(d)


# ------------------------------------------------------------- packed batches
def _sdpa_packed(q, k, v, cu, scale, causal):
    """torch SDPA (fp64) over the whole pack with a block-diagonal mask (and
    the causal triangle inside each block)."""
    H_q, T, _ = q.shape
    H_kv = k.shape[0]
    seq = np.zeros(T, dtype=np.int64)
    for n, (a, b) in enumerate(zip(cu, cu[1:])):
        seq[a:b] = n
    seq = torch.from_numpy(seq)
    mask = seq[:, None] == seq[None, :]
    if causal:
        pos = torch.arange(T)
        mask = mask & (pos[None, :] <= pos[:, None])
    idx = torch.tensor([kv_head_index(i, H_q, H_kv) for i in range(H_q)])
    tk = torch.from_numpy(k).double().index_select(0, idx)[None]
    tv = torch.from_numpy(v).double().index_select(0, idx)[None]
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).double()[None], tk, tv, attn_mask=mask, scale=scale).numpy()[0]


@pytest.mark.parametrize("lens,H_q,H_kv", [([5, 1, 9, 3], 4, 2), ([7, 7], 6, 4), ([13], 2, 1),
                                            ([2, 0, 4, 0, 1], 3, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_matches_bruteforce(lens, H_q, H_kv, causal):
    q, k, v, cu = draw_varlen(lens, H_q, H_kv, 8, "f32", seed=sum(lens) + H_q)
    got = attention_varlen(q, k, v, cu, scale=0.4, causal=causal)
    ref = _brute_packed(q, k, v, cu, 0.4, causal)
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_matches_sdpa_block_diagonal_mask(causal):
    lens = [37, 1, 64, 100, 3, 0, 51]
    q, k, v, cu = draw_varlen(lens, 8, 4, 16, "bf16", seed=31)
    got = attention_varlen(q, k, v, cu, scale=0.25, causal=causal)
    ref = _sdpa_packed(q, k, v, cu, 0.25, causal)
    assert np.max(np.abs(got - ref)) <= 1e-12
    # planted mistake: the pack taken as one sequence (other sequences' keys
    # visible, causal positions not restarting) disagrees with the reference
    whole = attention(q[None], k[None], v[None], scale=0.25, causal=causal)[0]
    assert np.max(np.abs(whole - ref)) > 1e-3


def test_varlen_lse_matches_scipy():
    from scipy.special import logsumexp
    lens = [6, 10, 1]
    q, k, v, cu = draw_varlen(lens, 2, 1, 8, "f32", seed=5)
    _, lse = attention_varlen(q, k, v, cu, scale=0.5, causal=True, return_lse=True)
    for i in range(2):
        for a, b in zip(cu, cu[1:]):
            s = 0.5 * (q[i, a:b].astype(np.float64) @ k[0, a:b].astype(np.float64).T)
            for r in range(b - a):
                assert abs(lse[i, a + r] - logsumexp(s[r, :r + 1])) <= 1e-12


def test_varlen_sequence_order_and_empty_sequences():
    """Reordering the sequences of a pack reorders the output blocks; empty
    sequences change nothing."""
    lens = [9, 4, 12]
    q, k, v, cu = draw_varlen(lens, 4, 2, 8, "f32", seed=8)
    base = attention_varlen(q, k, v, cu, scale=0.3, causal=True)
    order = [2, 0, 1]
    segs = [(cu[n], cu[n + 1]) for n in order]
    perm = np.concatenate([np.arange(a, b) for a, b in segs])
    cu2 = np.concatenate([[0], np.cumsum([lens[n] for n in order])])
    got = attention_varlen(q[:, perm], k[:, perm], v[:, perm], cu2, scale=0.3, causal=True)
    assert np.array_equal(got, base[:, perm])
    cu3 = [0, 0, 9, 9, 13, 25, 25]
    assert np.array_equal(attention_varlen(q, k, v, cu3, scale=0.3, causal=True), base)


def test_varlen_rejects_bad_offsets():
    q, k, v, cu = draw_varlen([3, 4], 2, 1, 8, "f32", seed=1)
    for bad in ([0, 5, 4, 7], [1, 7], [0, 3, 8]):
        with pytest.raises(ValueError):
            attention_varlen(q, k, v, bad)


# ----------------------------------------------------- packed-batch backward
def _autograd_packed(q, k, v, g, cu, scale, causal):
    """torch autograd through fp64 SDPA over the whole pack with the explicit
    block-diagonal (causal-within-block) mask; K/V gathered by kv_head_index,
    so autograd sums each K/V head's group."""
    H_q, T, _ = q.shape
    H_kv = k.shape[0]
    seq = np.zeros(T, dtype=np.int64)
    for n, (a, b) in enumerate(zip(cu, cu[1:])):
        seq[a:b] = n
    seq = torch.from_numpy(seq)
    mask = seq[:, None] == seq[None, :]
    if causal:
        pos = torch.arange(T)
        mask = mask & (pos[None, :] <= pos[:, None])
    idx = torch.tensor([kv_head_index(i, H_q, H_kv) for i in range(H_q)])
    tq = torch.from_numpy(q).double().requires_grad_(True)
    tk = torch.from_numpy(k).double().requires_grad_(True)
    tv = torch.from_numpy(v).double().requires_grad_(True)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq[None], tk.index_select(0, idx)[None], tv.index_select(0, idx)[None], attn_mask=mask, scale=scale)
    o.backward(torch.from_numpy(g)[None])
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("lens,H_q,H_kv", [([9, 1, 20, 0, 7], 8, 4), ([12, 12], 6, 4), ([5, 16], 5, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_bwd_matches_torch_autograd(lens, H_q, H_kv, causal):
    from oracle import attention_bwd_varlen
    q, k, v, cu = draw_varlen(lens, H_q, H_kv, 8, "bf16", seed=sum(lens) + 3)
    g = np.random.default_rng(7).standard_normal(q.shape)
    got = attention_bwd_varlen(q, k, v, g, cu, scale=0.3, causal=causal)
    ref = _autograd_packed(q, k, v, g, cu, 0.3, causal)
    for a, b in zip(got, ref):
        assert np.max(np.abs(a - b)) <= 1e-11


def test_varlen_bwd_matches_finite_differences_of_forward():
    """Central differences of the (separately pinned) packed forward oracle."""
    from oracle import attention_bwd_varlen
    lens = [3, 0, 4]
    q, k, v, cu = draw_varlen(lens, 3, 2, 2, "f32", seed=9)
    q, k, v = (x.astype(np.float64) for x in (q, k, v))
    g = np.random.default_rng(10).standard_normal(q.shape)
    got = attention_bwd_varlen(q, k, v, g, cu, scale=0.8, causal=True)
    eps = 1e-6

    def loss(qq, kk, vv):
        return float(np.sum(attention_varlen(qq, kk, vv, cu, scale=0.8, causal=True) * g))

    for which, arr in enumerate((q, k, v)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            args = [q, k, v]
            up = arr.copy(); up[idx] += eps
            dn = arr.copy(); dn[idx] -= eps
            args[which] = up; lp = loss(*args)
            args[which] = dn; lm = loss(*args)
            fd[idx] = (lp - lm) / (2 * eps)
        assert np.max(np.abs(got[which] - fd)) <= 1e-7 * max(1.0, np.max(np.abs(fd)))
