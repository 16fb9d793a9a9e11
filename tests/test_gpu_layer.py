"""GPU parity of sqa_layer_fwd (projections + RoPE + SQA + output projection)
against the fp64 oracle layer, on every output element."""
import math

import numpy as np
import pytest

from oracle import layer as oracle_layer
from synth import WORKLOADS, draw_layer
from tests.parity import check_global, check_rows, log, oracle_threads, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_query_attention_sqa_amd as sqa  # noqa: E402


def _layer_case(B, N, D, H, Hq, Hkv, base, causal, seed=0, label=""):
    x, wq, wk, wv, wo = draw_layer(B, N, D, H, Hq, Hkv, seed=seed)
    d = D // H
    scale = 1.0 / math.sqrt(d)
    args = [to_dev(a, "bf16") for a in (x, wq, wk, wv, wo)]
    y = sqa.sqa_layer_fwd(*args, H=H, H_q=Hq, H_kv=Hkv, rope_base=base, scale=scale,
                          causal=bool(causal))
    torch.cuda.synchronize()
    got = to_host(y)
    ref = oracle_layer(x, wq, wk, wv, wo, H, Hq, Hkv, rope_base=base, scale=scale,
                       causal=bool(causal), threads=oracle_threads())
    check_global(got, ref, "bf16", label)
    return got, ref


def test_sqatm_layer_all_outputs():
    w = WORKLOADS["sqatm_layer_bf16"]
    Hq, Hkv = w.variants[0]
    log(f"[case] {w.name}")
    got, ref = _layer_case(w.B, w.N, w.d_model, w.H, Hq, Hkv, w.rope_base, 1, label=w.name)
    check_rows(got[:2], ref[:2], w.name + " rows of batches 0-1")


@pytest.mark.parametrize("B,N,D,H,Hq,Hkv,causal", [
    (1, 1, 256, 16, 8, 4, 1), (2, 70, 256, 16, 8, 4, 1), (1, 129, 256, 16, 16, 1, 0),
    (3, 65, 256, 16, 4, 4, 1), (1, 200, 512, 8, 4, 2, 1), (2, 33, 256, 4, 2, 1, 0),
    (2, 100, 256, 16, 6, 4, 1), (1, 77, 512, 8, 5, 2, 0),     # H_kv not dividing H_q
])
def test_layer_shapes(B, N, D, H, Hq, Hkv, causal):
    label = f"layer B={B} N={N} D={D} H={H} ({Hq},{Hkv}) causal={causal}"
    log(f"[case] {label}")
    _layer_case(B, N, D, H, Hq, Hkv, 10000.0, causal, seed=B * 7 + N, label=label)


def test_layer_workspace_too_small_is_rejected():
    x = torch.zeros(1, 64, 256, dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros(256, 128, dtype=torch.bfloat16, device="cuda")
    wk = torch.zeros(256, 64, dtype=torch.bfloat16, device="cuda")
    wo = torch.zeros(128, 256, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(sqa.SQAError) as e:
        sqa.sqa_layer_fwd(x, wq, wk, wk.clone(), wo, H=16, H_q=8, H_kv=4, workspace=ws)
    assert e.value.status == 5
