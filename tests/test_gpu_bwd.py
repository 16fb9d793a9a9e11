"""GPU parity of sqa_attn_bwd (through the C ABI) against the fp64 backward
oracle.

As in training, the forward's o and lse (sqa_attn_fwd on the GPU) feed the
backward. dq, dk and dv are compared on every element with the bf16 bar:
max |g - g_ref| <= 1e-2 * max |g_ref| + 2^-14 per tensor (a CPU simulation of the
kernel's rounding -- bf16 P and dS, D from the bf16 forward output -- stays
below 0.7 % on these inputs, peaky keys included). Shapes: small ragged N
across head groupings and both masks, N in the thousands with ragged tails,
and the 32k SQA (8,4) shape.
"""
import math

import numpy as np
import pytest

from oracle import attention as oracle_attention
from oracle import attention_bwd as oracle_bwd
from synth import WORKLOADS, bf16_round, draw_attn_case, draw_qkv, draw_upstream, select_variant
from tests.parity import ROW_FLOOR, check_global, check_rows_scaled, log, oracle_threads, to_dev, to_host

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


def _run_bwd(q, k, v, do, scale, causal):
    tq, tk, tv, tdo = (to_dev(a, "bf16") for a in (q, k, v, do))
    o, lse = sqa.sqa_attn_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True)
    dq, dk, dv = sqa.sqa_attn_bwd(tq, tk, tv, o, tdo, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return to_host(dq), to_host(dk), to_host(dv)


def _check(got, ref, label):
    # the bf16 resolution floor covers gradients that vanish identically
    # (N = 1: dS = P (dP - D) = 0, computed as a difference of fp32 sums)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        check_global(g, r, "bf16", f"{label} {name}", floor=ROW_FLOOR)


def _check_rows_given_forward(q, k, v, do, scale, causal, label):
    """The backward alone, per row. Its inputs o and lse come from the
    oracle's forward (o rounded to bf16, lse to fp32), and the oracle's
    backward takes D_t = sum_c dout_tc o_tc from that same o, as the
    library's backward is defined to. Every query row of dq and every key row
    of dk and dv is then held to its own magnitude (its absolute-term sums,
    tests/parity.py), so that an error confined to rows much smaller than
    the tensor's largest (early query rows and late keys under a causal mask,
    ordinary keys next to peaky ones) cannot hide under the global bar."""
    th = oracle_threads()
    o_ref, lse_ref = oracle_attention(q, k, v, scale=scale, causal=bool(causal), threads=th, return_lse=True)
    o_in = bf16_round(o_ref.astype(np.float32))
    tq, tk, tv, to, tdo = (to_dev(a, "bf16") for a in (q, k, v, o_in, do))
    tl = torch.from_numpy(lse_ref.astype(np.float32)).to("cuda")
    grads = sqa.sqa_attn_bwd(tq, tk, tv, to, tdo, tl, scale=scale, causal=bool(causal))
    torch.cuda.synchronize()
    got = [to_host(g) for g in grads]
    ref = oracle_bwd(q, k, v, do, scale=scale, causal=bool(causal), threads=th, o=o_in)
    mags = oracle_bwd(q, k, v, do, scale=scale, causal=bool(causal), threads=th, o=o_in, absolute=True)
    for name, g, r, m in zip(("dq", "dk", "dv"), got, ref, mags):
        check_global(g, r, "bf16", f"{label} {name}", floor=ROW_FLOOR)
        check_rows_scaled(g, r, m, f"{label} {name}")


# --------------------------------------------------------- small, all elements
SMALL_N = [1, 2, 31, 32, 33, 64, 65, 100, 257, 1000]
SMALL_HEADS = [(1, 1), (2, 1), (8, 4), (4, 1), (16, 1), (3, 3), (6, 2)]


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("N", SMALL_N)
@pytest.mark.parametrize("Hq,Hkv", SMALL_HEADS)
def test_bwd_small_all_elements(Hq, Hkv, N, causal):
    label = f"bwd small Hq={Hq} Hkv={Hkv} N={N} causal={causal}"
    log(f"[case] {label}")
    B = 2 if N <= 100 else 1
    q, k, v = draw_attn_case(B, Hq, Hkv, N, 64, "bf16", seed=N * 17 + Hq)
    do = draw_upstream(q.shape, "bf16", seed=N + 101)
    got = _run_bwd(q, k, v, do, 0.125, causal)
    ref = oracle_bwd(q, k, v, do, scale=0.125, causal=bool(causal), threads=oracle_threads())
    _check(got, ref, label)


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("N,Hq,Hkv", [(4096, 8, 4), (8200, 4, 2), (5001, 16, 1), (3000, 4, 4)])
def test_bwd_medium_all_elements(N, Hq, Hkv, causal):
    label = f"bwd medium Hq={Hq} Hkv={Hkv} N={N} causal={causal}"
    log(f"[case] {label}")
    q, k, v = draw_attn_case(1, Hq, Hkv, N, 64, "bf16", seed=N)
    do = draw_upstream(q.shape, "bf16", seed=N + 7)
    got = _run_bwd(q, k, v, do, 0.125, causal)
    ref = oracle_bwd(q, k, v, do, scale=0.125, causal=bool(causal), threads=oracle_threads())
    _check(got, ref, label)


@pytest.mark.parametrize("scale", [0.5, -0.125])
def test_bwd_other_scales(scale):
    label = f"bwd scale={scale}"
    log(f"[case] {label}")
    q, k, v = draw_attn_case(1, 8, 4, 777, 64, "bf16", seed=3)
    do = draw_upstream(q.shape, "bf16", seed=4)
    got = _run_bwd(q, k, v, do, scale, 1)
    ref = oracle_bwd(q, k, v, do, scale=scale, causal=True, threads=oracle_threads())
    _check(got, ref, label)


def test_bwd_peaky_keys():
    """1 % of the keys scaled by 8, as in the 200k workload, at N = 4096."""
    label = "bwd peaky N=4096 (4,4)"
    log(f"[case] {label}")
    qa, ka, va = draw_qkv(1, 16, 4096, 64, "bf16", seed=0, peaky=True)
    q, k, v = select_variant(qa, ka, va, 4, 4)
    do = draw_upstream(q.shape, "bf16", seed=12)
    got = _run_bwd(q, k, v, do, 0.125, 0)
    ref = oracle_bwd(q, k, v, do, scale=0.125, causal=False, threads=oracle_threads())
    _check(got, ref, label)


# ------------------------------------------------- the 32k SQA (8,4) shape
@pytest.mark.parametrize("causal", [0, 1])
def test_bwd_long32k_sqa(causal):
    w = WORKLOADS["long32k_bf16"]
    label = f"bwd {w.name} (8,4) causal={causal}"
    log(f"[case] {label}")
    qa, ka, va = draw_qkv(w.B, w.H, w.N, w.d, "bf16", seed=0)
    q, k, v = select_variant(qa, ka, va, 8, 4)
    do = draw_upstream(q.shape, "bf16", seed=55)
    got = _run_bwd(q, k, v, do, w.scale, causal)
    log(f"[oracle] {label} (fp64 backward, all rows)")
    ref = oracle_bwd(q, k, v, do, scale=w.scale, causal=bool(causal), threads=oracle_threads())
    _check(got, ref, label)


# ------------------------------------- per-row gates, forward outputs given
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("N,Hq,Hkv,d", [(4096, 8, 4, 64), (3000, 4, 4, 64), (2113, 8, 2, 128), (777, 6, 4, 64)])
def test_bwd_rows_given_forward(N, Hq, Hkv, d, causal):
    label = f"bwd rows Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}"
    log(f"[case] {label}")
    q, k, v = draw_attn_case(1, Hq, Hkv, N, d, "bf16", seed=N + 3)
    do = draw_upstream(q.shape, "bf16", seed=N + 4)
    _check_rows_given_forward(q, k, v, do, 1.0 / math.sqrt(d), causal, label)


def test_bwd_rows_given_forward_peaky():
    label = "bwd rows peaky N=4096 (4,4)"
    log(f"[case] {label}")
    qa, ka, va = draw_qkv(1, 16, 4096, 64, "bf16", seed=0, peaky=True)
    q, k, v = select_variant(qa, ka, va, 4, 4)
    do = draw_upstream(q.shape, "bf16", seed=12)
    _check_rows_given_forward(q, k, v, do, 0.125, 0, label)


@pytest.mark.parametrize("causal", [0, 1])
def test_bwd_rows_given_forward_long32k(causal):
    w = WORKLOADS["long32k_bf16"]
    label = f"bwd rows {w.name} (8,4) causal={causal}"
    log(f"[case] {label}")
    qa, ka, va = draw_qkv(w.B, w.H, w.N, w.d, "bf16", seed=0)
    q, k, v = select_variant(qa, ka, va, 8, 4)
    do = draw_upstream(q.shape, "bf16", seed=55)
    _check_rows_given_forward(q, k, v, do, w.scale, causal, label)


# ------------------------------------------------------ closed forms on device
@pytest.mark.parametrize("causal", [0, 1])
def test_bwd_unit_upstream_value_column_sums(causal):
    """dO = 1: rows of P sum to 1, so every column of dV_j sums to g*N."""
    Hq, Hkv, N = 8, 2, 1111
    q, k, v = draw_attn_case(1, Hq, Hkv, N, 64, "bf16", seed=8)
    _, _, dv = _run_bwd(q, k, v, np.ones(q.shape, np.float32), 0.125, causal)
    sums = dv.sum(axis=2)
    assert np.max(np.abs(sums - (Hq // Hkv) * N)) <= 1e-2 * (Hq // Hkv) * N


def test_bwd_key_grads_sum_to_zero():
    q, k, v = draw_attn_case(1, 8, 4, 2048, 64, "bf16", seed=9)
    do = draw_upstream(q.shape, "bf16", seed=10)
    _, dk, _ = _run_bwd(q, k, v, do, 0.125, 1)
    tot = np.abs(dk).sum(axis=2)
    assert np.all(np.abs(dk.sum(axis=2)) <= 1e-2 * tot + 1e-6)


def test_bwd_zero_scale():
    """scale 0: dq and dk are exactly 0, dv is the mean of dO over the visible rows."""
    Hq, Hkv, N = 4, 2, 300
    q, k, v = draw_attn_case(1, Hq, Hkv, N, 64, "bf16", seed=11)
    do = draw_upstream(q.shape, "bf16", seed=12)
    dq, dk, dv = _run_bwd(q, k, v, do, 0.0, 1)
    assert np.max(np.abs(dq)) == 0.0 and np.max(np.abs(dk)) == 0.0
    ref = oracle_bwd(q, k, v, do, scale=0.0, causal=True)[2]
    check_global(dv, ref, "bf16", "bwd scale 0 dv", floor=ROW_FLOOR)


def test_bwd_deterministic_and_batch_independent():
    q, k, v = draw_attn_case(2, 8, 4, 1500, 64, "bf16", seed=13)
    do = draw_upstream(q.shape, "bf16", seed=14)
    a = _run_bwd(q, k, v, do, 0.125, 1)
    b = _run_bwd(q, k, v, do, 0.125, 1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    one = _run_bwd(q[1:], k[1:], v[1:], do[1:], 0.125, 1)
    for x, y in zip(a, one):
        assert np.array_equal(x[1:], y)


def test_bwd_error_paths():
    q, k, v = draw_attn_case(1, 8, 4, 64, 64, "bf16", seed=15)
    tq, tk, tv = (to_dev(a, "bf16") for a in (q, k, v))
    o, lse = sqa.sqa_attn_fwd(tq, tk, tv, return_lse=True)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(sqa.SQAError) as e:
        sqa.sqa_attn_bwd(tq, tk, tv, o, o, lse, workspace=small)
    assert e.value.status == 5
    q16, k16, v16 = (to_dev(a, "bf16") for a in draw_attn_case(1, 8, 4, 64, 16, "bf16", seed=16))
    o16, lse16 = sqa.sqa_attn_fwd(q16, k16, v16, return_lse=True)
    with pytest.raises(sqa.SQAError) as e:
        sqa.sqa_attn_bwd(q16, k16, v16, o16, o16, lse16)
    assert e.value.status == 3
    torch.cuda.synchronize()
