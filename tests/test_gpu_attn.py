"""GPU parity of sqa_attn_fwd (through the C ABI) against the fp64 oracle.

Small shapes are checked on every row; N >= 32k workloads on 4096 seeded
sampled positions of every head plus the tile-boundary rows. Tolerances are
in tests/parity.py.
"""
import functools
import math

import numpy as np
import pytest

from oracle import attention as oracle_attention
from synth import WORKLOADS, boundary_rows, draw_attn_case, draw_qkv, sample_rows, select_variant
from tests.parity import (LSE_BF16, check_global, check_rows, log, oracle_threads, to_dev, to_host)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_query_attention_sqa_amd as sqa  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    sqa.load_library()
    yield
    torch.cuda.synchronize()


def _run(q, k, v, dtype, scale, causal, return_lse=False):
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    r = sqa.sqa_attn_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=return_lse)
    torch.cuda.synchronize()
    return r


# --------------------------------------------------------- small, all rows
# 161 and 192 keys are six 32-key tiles: exactly one turn of the d = 64
# kernel's six-slot ring, where no tile is issued at the pair barrier
SMALL_N = [1, 2, 15, 17, 63, 64, 65, 127, 129, 161, 192, 200, 1000]
SMALL_HEADS = [(1, 1), (2, 1), (8, 4), (4, 1), (16, 1), (3, 3), (6, 2)]


@pytest.mark.parametrize("d", [64, 16])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("N", SMALL_N)
@pytest.mark.parametrize("Hq,Hkv", SMALL_HEADS)
def test_bf16_small_all_rows(Hq, Hkv, N, causal, d):
    label = f"bf16 small Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}"
    log(f"[case] {label}")
    B = 2 if N <= 200 else 1
    q, k, v = draw_attn_case(B, Hq, Hkv, N, d, "bf16", seed=N * 31 + Hq)
    scale = 1.0 / math.sqrt(d)
    o = to_host(_run(q, k, v, "bf16", scale, causal))
    ref = oracle_attention(q, k, v, scale=scale, causal=bool(causal))
    check_global(o, ref, "bf16", label)
    check_rows(o, ref, label)


# d = 16 grids of at most two workgroups per CU run eight-wave workgroups
# whose two key-range parts are merged through LDS; larger grids the
# four-wave workgroups. On 256 CUs, N = 1024 (8,4) has 512 workgroups at B = 8
# (the last grid with parts) and 576 at B = 9 (the first without); N = 960
# gives odd tile counts per workgroup (the second part one tile short).
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("B,N", [(8, 1024), (9, 1024), (8, 960)])
def test_bf16_d16_grid_bound_all_rows(B, N, causal):
    label = f"bf16 d=16 B={B} N={N} (8,4) causal={causal}"
    log(f"[case] {label}")
    q, k, v = draw_attn_case(B, 8, 4, N, 16, "bf16", seed=B * 1000 + N)
    o, lse = _run(q, k, v, "bf16", 0.25, causal, return_lse=True)
    ref, ref_lse = oracle_attention(q, k, v, scale=0.25, causal=bool(causal), return_lse=True,
                                    threads=oracle_threads())
    o = to_host(o)
    check_global(o, ref, "bf16", label)
    check_rows(o, ref, label)
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= LSE_BF16


@pytest.mark.parametrize("d", [16, 64])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("N,Hq,Hkv", [(1, 2, 1), (17, 8, 4), (255, 4, 4), (256, 2, 2),
                                      (257, 8, 2), (700, 16, 1)])
def test_f32_small_all_rows(N, Hq, Hkv, causal, d):
    label = f"f32 small Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}"
    log(f"[case] {label}")
    q, k, v = draw_attn_case(1, Hq, Hkv, N, d, "f32", seed=N + 5)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(q, k, v, "f32", scale, causal, return_lse=True)
    ref, ref_lse = oracle_attention(q, k, v, scale=scale, causal=bool(causal), return_lse=True)
    check_global(to_host(o), ref, "f32", label)
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= 1e-4


# ------------------------------------------------- SQAT-m attention core fp32
@pytest.mark.parametrize("causal", [0, 1])
def test_sqatm_core_f32_all_rows(causal):
    w = WORKLOADS["sqatm_core_f32"]
    Hq, Hkv = w.variants[0]
    log(f"[case] {w.name} causal={causal}")
    q, k, v = draw_qkv(w.B, w.H, w.N, w.d, "f32", seed=0)
    q, k, v = select_variant(q, k, v, Hq, Hkv)
    o, lse = _run(q, k, v, "f32", w.scale, causal, return_lse=True)
    ref, ref_lse = oracle_attention(q, k, v, scale=w.scale, causal=bool(causal), return_lse=True)
    check_global(to_host(o), ref, "f32", f"{w.name} causal={causal}")
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= 1e-4


# ------------------------------------------------------ long sequences, bf16
@functools.lru_cache(maxsize=1)
def _workload_inputs(name):
    w = WORKLOADS[name]
    log(f"[gen] {name}")
    return draw_qkv(w.B, w.H, w.N, w.d, w.dtype, seed=0, peaky=w.peaky)


def _long_case(name, Hq, Hkv, causal):
    w = WORKLOADS[name]
    label = f"{name} ({Hq},{Hkv}) causal={causal}"
    log(f"[case] {label}")
    q, k, v = select_variant(*_workload_inputs(name), Hq, Hkv)
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o, lse = sqa.sqa_attn_fwd(tq, tk, tv, scale=w.scale, causal=bool(causal), return_lse=True)
    torch.cuda.synchronize()
    rows = sample_rows(w.N, w.sampled_rows)
    brows = boundary_rows(w.N)
    idx_r = torch.from_numpy(rows).to("cuda")
    idx_b = torch.from_numpy(brows).to("cuda")
    got = o.index_select(2, idx_r).float().cpu().numpy().astype(np.float64)
    got_b = o.index_select(2, idx_b).float().cpu().numpy().astype(np.float64)
    got_lse = lse.index_select(2, idx_r).cpu().numpy()
    del tq, tk, tv, o, lse
    torch.cuda.empty_cache()
    th = oracle_threads()
    ref, ref_lse = oracle_attention(q, k, v, scale=w.scale, causal=bool(causal), rows=rows,
                                    threads=th, return_lse=True)
    check_global(got, ref, "bf16", label + " sampled")
    ref_b = oracle_attention(q, k, v, scale=w.scale, causal=bool(causal), rows=brows, threads=th)
    check_rows(got_b, ref_b, label + " boundary rows")
    lse_err = float(np.max(np.abs(got_lse - ref_lse)))
    log(f"[parity] {label} lse max_err={lse_err:.3e}")
    assert lse_err <= LSE_BF16


@pytest.mark.parametrize("Hq,Hkv", WORKLOADS["long32k_bf16"].variants)
def test_long32k(Hq, Hkv):
    _long_case("long32k_bf16", Hq, Hkv, 0)


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("Hq,Hkv", WORKLOADS["long131k_bf16"].variants)
def test_long131k(Hq, Hkv, causal):
    _long_case("long131k_bf16", Hq, Hkv, causal)


@pytest.mark.parametrize("Hq,Hkv", WORKLOADS["long200k_peaky_bf16"].variants)
def test_long200k_peaky(Hq, Hkv):
    _long_case("long200k_peaky_bf16", Hq, Hkv, 0)


# ------------------------------------------------------------ invariants
@pytest.mark.parametrize("d", [16, 64])
@pytest.mark.parametrize("causal", [0, 1])
def test_constant_values_give_exactly_one(d, causal):
    q, k, _ = draw_attn_case(1, 8, 4, 777, d, "bf16", seed=3)
    v = np.ones((1, 4, 777, d), dtype=np.float32)
    o = _run(q, k, v, "bf16", 1.0 / math.sqrt(d), causal)
    assert torch.all(o == 1.0).item()


@pytest.mark.parametrize("causal", [0, 1])
def test_identical_keys_give_mean(causal):
    N, d = 300, 64
    q, k, v = draw_attn_case(1, 4, 2, N, d, "bf16", seed=4)
    k[:] = k[:, :, :1, :]
    o = to_host(_run(q, k, v, "bf16", 0.125, causal))
    vv = v.astype(np.float64)
    if causal:
        mean = np.cumsum(vv, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    else:
        mean = np.broadcast_to(vv.mean(axis=2, keepdims=True), vv.shape)
    ref = np.repeat(mean, 2, axis=1)
    check_global(o, ref, "bf16", f"identical keys causal={causal}")


@pytest.mark.parametrize("d", [64, 16, 32, 128])
@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5])
def test_scale_values(scale, d):
    q, k, v = draw_attn_case(1, 8, 4, 333, d, "bf16", seed=5)
    for causal in (0, 1):
        o = to_host(_run(q, k, v, "bf16", scale, causal))
        ref = oracle_attention(q, k, v, scale=scale, causal=bool(causal))
        check_global(o, ref, "bf16", f"scale={scale} d={d} causal={causal}")


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [0, 1])
def test_score_jumps_in_later_tiles(d, causal):
    """Keys from position 600 on are scaled by 4 and keys 1100-1109 by 16
    (powers of two: still exact in bf16), so the row maximum jumps by far more
    than 2^20 in probability in tiles after the first one; every row is
    compared with the oracle."""
    N = 1500
    label = f"score jumps d={d} causal={causal}"
    log(f"[case] {label}")
    q, k, v = draw_attn_case(1, 8, 4, N, d, "bf16", seed=23)
    k[:, :, 600:] *= 4.0
    k[:, :, 1100:1110] *= 4.0
    o = to_host(_run(q, k, v, "bf16", 1.0 / math.sqrt(d), causal))
    ref = oracle_attention(q, k, v, scale=1.0 / math.sqrt(d), causal=bool(causal))
    check_global(o, ref, "bf16", label)
    check_rows(o, ref, label)


def test_permutation_equivariance_noncausal():
    N = 500
    q, k, v = draw_attn_case(1, 4, 2, N, 64, "bf16", seed=6)
    rng = np.random.default_rng(0)
    pq, pk = rng.permutation(N), rng.permutation(N)
    o = to_host(_run(q, k, v, "bf16", 0.125, 0))
    o_q = to_host(_run(np.ascontiguousarray(q[:, :, pq]), k, v, "bf16", 0.125, 0))
    o_k = to_host(_run(q, np.ascontiguousarray(k[:, :, pk]), np.ascontiguousarray(v[:, :, pk]),
                       "bf16", 0.125, 0))
    ref = oracle_attention(q, k, v, scale=0.125)
    check_global(o_q, o[:, :, pq], "bf16", "query permutation")
    check_global(o_k, o, "bf16", "key permutation")
    check_global(o, ref, "bf16", "unpermuted")


def test_deterministic_and_canaries():
    B, Hq, Hkv, N, d = 1, 8, 4, 1000, 64
    q, k, v = draw_attn_case(B, Hq, Hkv, N, d, "bf16", seed=7)
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    n = B * Hq * N * d
    pad = 4096
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = buf[pad:pad + n].view(B, Hq, N, d)
    outs = []
    for causal in (0, 1, 0):
        sqa.sqa_attn_fwd(tq, tk, tv, scale=0.125, causal=bool(causal), out=out)
        torch.cuda.synchronize()
        outs.append(out.clone())
        assert torch.isnan(buf[:pad]).all().item() and torch.isnan(buf[pad + n:]).all().item()
    assert torch.equal(outs[0], outs[2])
    for _ in range(3):
        again = sqa.sqa_attn_fwd(tq, tk, tv, scale=0.125, causal=False)
        torch.cuda.synchronize()
        assert torch.equal(again, outs[0])


def test_batches_are_independent():
    q, k, v = draw_attn_case(3, 8, 2, 130, 64, "bf16", seed=8)
    o = to_host(_run(q, k, v, "bf16", 0.125, 1))
    for b in range(3):
        ob = to_host(_run(q[b:b + 1], k[b:b + 1], v[b:b + 1], "bf16", 0.125, 1))
        assert np.array_equal(ob[0], o[b])


def test_lse_bf16_matches_oracle():
    q, k, v = draw_attn_case(2, 8, 4, 1000, 64, "bf16", seed=9)
    for causal in (0, 1):
        _, lse = _run(q, k, v, "bf16", 0.125, causal, return_lse=True)
        _, ref = oracle_attention(q, k, v, scale=0.125, causal=bool(causal), return_lse=True)
        err = float(np.max(np.abs(lse.cpu().numpy() - ref)))
        log(f"[parity] lse bf16 causal={causal} err={err:.3e}")
        assert err <= LSE_BF16


# ------------------------------------------------------------- error paths
def test_error_paths_on_device():
    q = torch.zeros(1, 8, 64, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16, device="cuda")
    kk = torch.zeros(1, 9, 64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sqa.SQAError) as e:                 # H_kv > H_q
        sqa.sqa_attn_fwd(q, kk, kk)
    assert e.value.status == 2
    with pytest.raises(sqa.SQAError) as e:                 # d = 48
        sqa.sqa_attn_fwd(q[..., :48].contiguous(), k[..., :48].contiguous(), k[..., :48].contiguous())
    assert e.value.status == 3
    flat = torch.zeros(1 + 8 * 64 * 64, dtype=torch.bfloat16, device="cuda")
    mis = flat[1:].view(1, 8, 64, 64)           # 2-byte offset: misaligned
    with pytest.raises(sqa.SQAError) as e:
        sqa.sqa_attn_fwd(mis, k, k)
    assert e.value.status == 4
    with pytest.raises(sqa.SQAError) as e:
        sqa.sqa_attn_fwd(q, k, k, out=q)
    assert e.value.status == 7
    empty = torch.zeros(0, 8, 64, 64, dtype=torch.bfloat16, device="cuda")
    sqa.sqa_attn_fwd(empty, empty[:, :4], empty[:, :4])
