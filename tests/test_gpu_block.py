"""GPU parity of sqa_block_fwd (through the C ABI) against the fp64 block
oracle: RMSNorm -> SQA layer -> residual -> RMSNorm -> SwiGLU -> residual.

Weights default to N(0, 1/fan_in) so that each sub-layer changes the
residual stream by O(1): with small weights the updates would sit below the
bf16 resolution of y and a broken sub-layer could pass. Each sub-layer is
also checked alone (W_down = 0 leaves the attention path, W_O = 0 the feed
forward). Bar: max |y - y_ref| <= 1e-2 * max |y_ref| over every output.
"""
import math

import numpy as np
import pytest

from oracle import block as oracle_block
from synth import draw_block
from tests.parity import check_global, log, oracle_threads, to_dev, to_host

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


def _run(arrs, H, Hq, Hkv, scale, causal=True, eps=1e-6):
    y = sqa.sqa_block_fwd(*(to_dev(a, "bf16") for a in arrs), H=H, H_q=Hq, H_kv=Hkv,
                          rope_base=10000.0, scale=scale, eps=eps, causal=causal)
    torch.cuda.synchronize()
    return to_host(y)


def _ref(arrs, H, Hq, Hkv, scale, causal=True, eps=1e-6):
    return oracle_block(*arrs, H, Hq, Hkv, rope_base=10000.0, scale=scale, causal=causal, eps=eps,
                        threads=oracle_threads())


@pytest.mark.parametrize("Hq,Hkv,B", [(8, 4, 16), (16, 16, 2), (16, 4, 2), (16, 1, 2), (4, 4, 2)])
def test_block_sqatm_shape(Hq, Hkv, B):
    label = f"block SQAT-m B={B} N=1024 D=256 ({Hq},{Hkv}) F=768"
    log(f"[case] {label}")
    arrs = draw_block(B, 1024, 256, 16, Hq, Hkv, 768, seed=Hq * 10 + Hkv)
    check_global(_run(arrs, 16, Hq, Hkv, 0.25), _ref(arrs, 16, Hq, Hkv, 0.25), "bf16", label)


@pytest.mark.parametrize("N", [1, 17, 100, 333])
@pytest.mark.parametrize("D,H,F", [(256, 16, 768), (512, 8, 80), (256, 16, 16)])
def test_block_small(N, D, H, F):
    label = f"block small N={N} D={D} H={H} F={F}"
    log(f"[case] {label}")
    Hq, Hkv = H // 2, H // 4
    d = D // H
    arrs = draw_block(2, N, D, H, Hq, Hkv, F, seed=N + D)
    scale = 1.0 / math.sqrt(d)
    check_global(_run(arrs, H, Hq, Hkv, scale), _ref(arrs, H, Hq, Hkv, scale), "bf16", label)


@pytest.mark.parametrize("part", ["attention", "feed_forward"])
def test_block_sub_layers_alone(part):
    label = f"block {part} only"
    log(f"[case] {label}")
    arrs = list(draw_block(4, 1024, 256, 16, 8, 4, 768, seed=3))
    if part == "attention":
        arrs[9] = np.zeros_like(arrs[9])      # W_down = 0
    else:
        arrs[5] = np.zeros_like(arrs[5])      # W_O = 0
    x = arrs[0].astype(np.float64)
    got = _run(arrs, 16, 8, 4, 0.25)
    ref = _ref(arrs, 16, 8, 4, 0.25)
    check_global(got, ref, "bf16", label)
    # the sub-layer's own contribution, against its own magnitude (2 bf16
    # roundings of the stream: x and y, each <= 2^-9 relative)
    upd_err = np.max(np.abs((got - x) - (ref - x)))
    lim = 1e-2 * np.max(np.abs(ref - x)) + 2.0 ** -8 * np.max(np.abs(ref))
    log(f"[parity] {label} update err={upd_err:.3e} lim={lim:.3e}")
    assert upd_err <= lim


def test_block_encoder_style_and_eps():
    label = "block non-causal eps=1e-3"
    log(f"[case] {label}")
    arrs = draw_block(2, 500, 256, 16, 8, 4, 768, seed=5)
    check_global(_run(arrs, 16, 8, 4, 0.25, causal=False, eps=1e-3),
                 _ref(arrs, 16, 8, 4, 0.25, causal=False, eps=1e-3), "bf16", label)


def test_block_small_weights_recipe():
    """Weights N(0, 0.02) as in the layer workload."""
    label = "block N(0,0.02) weights"
    log(f"[case] {label}")
    arrs = draw_block(4, 1024, 256, 16, 8, 4, 768, seed=6, wstd=0.02)
    check_global(_run(arrs, 16, 8, 4, 0.25), _ref(arrs, 16, 8, 4, 0.25), "bf16", label)
