"""GPU parity of the key-range split forward (sqa_attn_fwd_split,
sqa_attn_fwd_varlen_split) against the fp64 oracle.

Each long sequence's keys are cut into ranges computed by separate
workgroups and merged by their softmax states; the result must meet the
same bf16 bar as the unsplit call, on every row, for forced split counts
(2, 3, 4) over ragged lengths, both masks, uneven head groups and packed
batches with one dominant sequence, plus the library's own choice at the
packed 32k workload. Tolerances are in tests/parity.py.
"""
import functools

import numpy as np
import pytest

from oracle import attention as oracle_attention
from oracle import attention_varlen as oracle_varlen
from synth import draw_attn_case, draw_varlen
from tests.parity import check_global, check_rows, log, oracle_threads, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_query_attention_sqa_amd as sqa  # noqa: E402

# lse bar of the bf16 forward (natural log): the row sum adds probabilities
# rounded to bf16 (relative error at most 2^-8 each), so |LSE - LSE_ref| <=
# ln(1 + 2^-8) ~ 3.9e-3 plus fp32 rounding.
LSE_TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    sqa.load_library()
    yield
    torch.cuda.synchronize()


@functools.lru_cache(maxsize=None)
def _dense_case(B, Hq, Hkv, N, causal):
    q, k, v = draw_attn_case(B, Hq, Hkv, N, 64, "bf16", seed=N * 7 + Hq)
    ref, ref_lse = oracle_attention(q, k, v, scale=0.125, causal=bool(causal), return_lse=True,
                                    threads=oracle_threads())
    return q, k, v, ref, ref_lse


# N = 1100: 35 tiles, ranges of 32 and 3 tiles; N = 2113 and 4200: ragged
# last tiles, up to four ranges; (6,4): groups of 2 and 1 heads.
@pytest.mark.parametrize("splits", [2, 3, 4])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 8, 4, 1100), (2, 6, 4, 2113), (1, 8, 4, 4200), (1, 3, 1, 3001)])
def test_split_dense_all_rows(B, Hq, Hkv, N, causal, splits):
    label = f"split dense B={B} ({Hq},{Hkv}) N={N} causal={causal} splits={splits}"
    log(f"[case] {label}")
    q, k, v, ref, ref_lse = _dense_case(B, Hq, Hkv, N, causal)
    o, lse = sqa.sqa_attn_fwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), scale=0.125,
                              causal=bool(causal), return_lse=True, num_splits=splits)
    torch.cuda.synchronize()
    o = to_host(o)
    check_global(o, ref, "bf16", label)
    check_rows(o, ref, label)
    err = float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse)))
    assert err <= LSE_TOL, f"{label}: lse error {err:.3e}"


@functools.lru_cache(maxsize=None)
def _small_d_case(B, Hq, Hkv, N, d, causal):
    q, k, v = draw_attn_case(B, Hq, Hkv, N, d, "bf16", seed=N + d)
    ref, ref_lse = oracle_attention(q, k, v, scale=d ** -0.5, causal=bool(causal), return_lse=True,
                                    threads=oracle_threads())
    return q, k, v, ref, ref_lse


# head dims 16 and 32 (64-key tiles, ranges of at least 4 tiles, 32-row
# waves for d = 16 causal; only on request, the library never picks them)
# and 128 (32-row waves over 32-key tiles, ranges of at least 32 tiles)
@pytest.mark.parametrize("splits", [2, 3, 4])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("d", [16, 32, 128])
@pytest.mark.parametrize("B,Hq,Hkv,N", [(2, 8, 4, 1100), (1, 6, 4, 2113)])
def test_split_head_dims_16_32_128_all_rows(B, Hq, Hkv, N, d, causal, splits):
    label = f"split d={d} B={B} ({Hq},{Hkv}) N={N} causal={causal} splits={splits}"
    log(f"[case] {label}")
    q, k, v, ref, ref_lse = _small_d_case(B, Hq, Hkv, N, d, causal)
    o, lse = sqa.sqa_attn_fwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), scale=d ** -0.5,
                              causal=bool(causal), return_lse=True, num_splits=splits)
    torch.cuda.synchronize()
    o = to_host(o)
    check_global(o, ref, "bf16", label)
    check_rows(o, ref, label)
    err = float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse)))
    assert err <= LSE_TOL, f"{label}: lse error {err:.3e}"


@pytest.mark.parametrize("causal", [0, 1])
def test_split_varlen_d32(causal):
    label = f"split varlen d=32 dominant causal={causal}"
    log(f"[case] {label}")
    q, k, v, cu = draw_varlen(SPLIT_MIXES["dominant"], 8, 4, 32, "bf16", seed=19)
    ref = oracle_varlen(q, k, v, cu, scale=32 ** -0.5, causal=bool(causal), threads=oracle_threads())
    o = sqa.sqa_attn_fwd_varlen(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                torch.from_numpy(cu).to("cuda"), scale=32 ** -0.5, causal=bool(causal),
                                num_splits=3)
    torch.cuda.synchronize()
    o = to_host(o)
    check_global(o, ref, "bf16", label)
    check_rows(o, ref, label)


def test_split_one_is_the_unsplit_call_bitwise():
    q, k, v, _, _ = _dense_case(1, 8, 4, 4200, 1)
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    a, la = sqa.sqa_attn_fwd(tq, tk, tv, scale=0.125, causal=True, return_lse=True, num_splits=1)
    lib = sqa.load_library()
    b = torch.empty_like(tq)
    lb = torch.empty_like(la)
    st = lib.sqa_attn_fwd_split(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), b.data_ptr(), 1, 8, 4, 4200, 64, 1,
                                0.125, 1, lb.data_ptr(), 1, None, 0, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_split_is_deterministic_and_reuses_a_dirty_workspace():
    q, k, v, ref, _ = _dense_case(1, 8, 4, 4200, 0)
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    lib = sqa.load_library()
    nbytes = lib.sqa_attn_fwd_split_workspace_bytes(8 * 4200, 64, 1, 3)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN bytes everywhere
    outs = []
    for _ in range(2):
        o = torch.empty_like(tq)
        st = lib.sqa_attn_fwd_split(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), 1, 8, 4, 4200, 64, 1,
                                    0.125, 0, None, 3, ws.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
        assert st == 0
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    check_global(to_host(outs[0]), ref, "bf16", "split=3 on a dirty workspace")


# packed batches: one sequence far longer than the rest (the case the split
# is for), empty and one-token sequences, ragged tiles
SPLIT_MIXES = {
    "dominant": [5000, 300, 0, 1, 1500, 64],
    "two_long": [2113, 31, 3000],
}


@functools.lru_cache(maxsize=None)
def _varlen_case(mix, Hq, Hkv, causal):
    lens = SPLIT_MIXES[mix]
    q, k, v, cu = draw_varlen(lens, Hq, Hkv, 64, "bf16", seed=len(lens) + Hq)
    ref, ref_lse = oracle_varlen(q, k, v, cu, scale=0.125, causal=bool(causal), return_lse=True,
                                 threads=oracle_threads())
    return q, k, v, cu, ref, ref_lse


@pytest.mark.parametrize("splits", [2, 3])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("mix", sorted(SPLIT_MIXES))
@pytest.mark.parametrize("Hq,Hkv", [(8, 4), (6, 4)])
def test_split_varlen_all_rows(Hq, Hkv, mix, causal, splits):
    label = f"split varlen {mix} ({Hq},{Hkv}) causal={causal} splits={splits}"
    log(f"[case] {label}")
    q, k, v, cu, ref, ref_lse = _varlen_case(mix, Hq, Hkv, causal)
    o, lse = sqa.sqa_attn_fwd_varlen(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                     torch.from_numpy(cu).to("cuda"), scale=0.125, causal=bool(causal),
                                     return_lse=True, num_splits=splits)
    torch.cuda.synchronize()
    o = to_host(o)
    check_global(o, ref, "bf16", label)
    check_rows(o, ref, label)
    err = float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse)))
    assert err <= LSE_TOL, f"{label}: lse error {err:.3e}"


def test_split_errors_on_device():
    q, k, v, _, _ = _dense_case(1, 8, 4, 1100, 0)
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    with pytest.raises(sqa.SQAError):
        sqa.sqa_attn_fwd(tq, tk, tv, num_splits=0)
    with pytest.raises(sqa.SQAError):
        sqa.sqa_attn_fwd(tq.float(), tk.float(), tv.float(), num_splits=2)  # fp32 path does not split



# ------------------------------------------------------------- backward
# dQ over key ranges, dK/dV over query ranges, summed in fp32: every element
# against the fp64 oracle, the bf16 bar with the absolute floor for
# gradients that can vanish (tests/parity.py).
from oracle import attention_bwd as oracle_bwd  # noqa: E402
from oracle import attention_bwd_varlen as oracle_bwd_varlen  # noqa: E402
from synth import draw_upstream  # noqa: E402
from tests.parity import ROW_FLOOR  # noqa: E402


@functools.lru_cache(maxsize=None)
def _bwd_dense_case(B, Hq, Hkv, N, d):
    q, k, v = draw_attn_case(B, Hq, Hkv, N, d, "bf16", seed=N * 3 + Hq + d)
    do = draw_upstream(q.shape, "bf16", seed=N + 5)
    ref = oracle_bwd(q, k, v, do, scale=0.125, causal=False, threads=oracle_threads())
    return q, k, v, do, ref


@pytest.mark.parametrize("splits", [2, 3])
@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(1, 8, 4, 2113, 64), (2, 6, 4, 1100, 64), (1, 4, 2, 3001, 128)])
def test_split_bwd_dense_all_elements(B, Hq, Hkv, N, d, splits):
    label = f"split bwd B={B} ({Hq},{Hkv}) N={N} d={d} splits={splits}"
    log(f"[case] {label}")
    q, k, v, do, ref = _bwd_dense_case(B, Hq, Hkv, N, d)
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o, lse = sqa.sqa_attn_fwd(tq, tk, tv, scale=0.125, return_lse=True, num_splits=1)
    got = sqa.sqa_attn_bwd(tq, tk, tv, o, to_dev(do, "bf16"), lse, scale=0.125, num_splits=splits)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        check_global(to_host(g), r, "bf16", f"{label} {name}", floor=ROW_FLOOR)


@pytest.mark.parametrize("splits", [2, 3])
@pytest.mark.parametrize("mix", sorted(SPLIT_MIXES))
def test_split_bwd_varlen_all_elements(mix, splits):
    label = f"split bwd varlen {mix} (8,4) splits={splits}"
    log(f"[case] {label}")
    q, k, v, cu = draw_varlen(SPLIT_MIXES[mix], 8, 4, 64, "bf16", seed=len(mix) + 11)
    do = draw_upstream(q.shape, "bf16", seed=len(mix) + 12)
    tq, tk, tv, tdo = (to_dev(a, "bf16") for a in (q, k, v, do))
    tcu = torch.from_numpy(cu).to("cuda")
    o, lse = sqa.sqa_attn_fwd_varlen(tq, tk, tv, tcu, scale=0.125, return_lse=True)
    got = sqa.sqa_attn_bwd_varlen(tq, tk, tv, o, tdo, lse, tcu, scale=0.125, num_splits=splits)
    torch.cuda.synchronize()
    ref = oracle_bwd_varlen(q, k, v, do, cu, scale=0.125, causal=False, threads=oracle_threads())
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        check_global(to_host(g), r, "bf16", f"{label} {name}", floor=ROW_FLOOR)


def test_split_bwd_one_is_the_unsplit_call_bitwise():
    q, k, v, do, _ = _bwd_dense_case(1, 8, 4, 2113, 64)
    tq, tk, tv, tdo = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(do, "bf16")
    o, lse = sqa.sqa_attn_fwd(tq, tk, tv, scale=0.125, return_lse=True, num_splits=1)
    a = sqa.sqa_attn_bwd(tq, tk, tv, o, tdo, lse, scale=0.125, num_splits=1)
    lib = sqa.load_library()
    need = lib.sqa_attn_bwd_workspace_bytes(1, 8, 2113, 64, 1)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    b = [torch.empty_like(t) for t in (tq, tk, tv)]
    st = lib.sqa_attn_bwd(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), tdo.data_ptr(), lse.data_ptr(),
                          b[0].data_ptr(), b[1].data_ptr(), b[2].data_ptr(), 1, 8, 4, 2113, 64, 1, 0.125, 0,
                          ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_split_bwd_rejects_causal_and_small_workspace():
    q, k, v, do, _ = _bwd_dense_case(1, 8, 4, 2113, 64)
    tq, tk, tv, tdo = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(do, "bf16")
    o, lse = sqa.sqa_attn_fwd(tq, tk, tv, scale=0.125, causal=True, return_lse=True)
    with pytest.raises(sqa.SQAError):
        sqa.sqa_attn_bwd(tq, tk, tv, o, tdo, lse, scale=0.125, causal=True, num_splits=2)
    small = torch.empty(sqa.sqa_attn_bwd_workspace_bytes(1, 8, 2113, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(sqa.SQAError):
        sqa.sqa_attn_bwd(tq, tk, tv, o, tdo, lse, scale=0.125, workspace=small, num_splits=2)
    # the library's choice falls back to one range when the given workspace is too small for more
    sqa.sqa_attn_bwd(tq, tk, tv, o, tdo, lse, scale=0.125, workspace=small)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- tail split
# Shapes whose workgroups overrun whole rounds of 2 per CU by a small tail
# on MI355X (256 CUs, 512 slots): N = 36300 (4,4): 568 workgroups, 56 past
# one round, 9 key ranges each; N = 17900 (8,4): 560, 48 past, 10 ranges;
# B = 3, N = 11000 (4,2): 516, 4 past, 10 ranges (344 tiles). Ragged last tiles.
@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 4, 4, 36300), (1, 8, 4, 17900), (3, 4, 2, 11000)])
def test_tail_split_all_rows(B, Hq, Hkv, N):
    S = sqa.sqa_attn_fwd_tail_splits(B, Hq, Hkv, N, 64)
    if S <= 1:
        pytest.skip(f"no tail split planned for this shape on this device ({torch.cuda.get_device_name()})")
    label = f"tail split B={B} ({Hq},{Hkv}) N={N} S={S}"
    log(f"[case] {label}")
    q, k, v = draw_attn_case(B, Hq, Hkv, N, 64, "bf16", seed=N + 11)
    ref, ref_lse = oracle_attention(q, k, v, scale=0.125, causal=False, return_lse=True, threads=oracle_threads())
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o, lse = sqa.sqa_attn_fwd(tq, tk, tv, scale=0.125, return_lse=True, num_splits=1, tail=True)
    plain = sqa.sqa_attn_fwd(tq, tk, tv, scale=0.125, num_splits=1, tail=False)
    torch.cuda.synchronize()
    o = to_host(o)
    check_global(o, ref, "bf16", label)
    check_rows(o, ref, label)
    err = float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse)))
    log(f"[parity] {label} lse max_err={err:.3e}")
    assert err <= LSE_TOL, f"{label}: lse error {err:.3e}"
    # the whole units agree with the unsplit call exactly; the tail units up
    # to the fp32 order of the merge
    diff = np.abs(o - to_host(plain))
    log(f"[parity] {label} vs unsplit max diff={float(diff.max()):.3e}")
    check_global(to_host(plain), ref, "bf16", label + " unsplit")


def test_tail_split_is_deterministic_and_reuses_a_dirty_workspace():
    B, Hq, Hkv, N = 1, 8, 4, 17900
    if sqa.sqa_attn_fwd_tail_splits(B, Hq, Hkv, N, 64) <= 1:
        pytest.skip("no tail split planned for this shape on this device")
    q, k, v = (to_dev(a, "bf16") for a in draw_attn_case(B, Hq, Hkv, N, 64, "bf16", seed=5))
    lib = sqa.load_library()
    nbytes = lib.sqa_attn_fwd_tail_workspace_bytes(B, Hq, Hkv, N, 64, sqa.SQA_BF16, 0)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")   # NaN-patterned garbage
    outs = []
    for _ in range(3):
        o = torch.empty_like(q)
        st = lib.sqa_attn_fwd_tail(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, Hq, Hkv, N, 64,
                                   sqa.SQA_BF16, 0.125, 0, None, ws.data_ptr(), nbytes,
                                   torch.cuda.current_stream().cuda_stream)
        assert st == 0, lib.sqa_last_error()
        torch.cuda.synchronize()
        outs.append(o)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
    assert not torch.isnan(outs[0].float()).any().item()
