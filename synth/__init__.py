"""Seeded synthetic inputs for Sparse Query Attention workloads.

This module is shared by the oracle-side tests and the HIP path's tests and
benchmark. It holds *no* attention arithmetic: it only draws random numbers,
quantises them to the input dtype, and describes workload shapes.

Workloads follow the shapes the pages use:
  * SQAT-m (model card "SQAT-m: Sparse Query Attention Transformer mini",
    section "Architecture details"): dim 256, 16 heads for the dimension split
    (d_head = 16), 8 query groups, 4 key/value groups, message length 1024.
  * Long sequences of 32k-200k tokens (SQA paper abstract on the chatpaper
    page) for the encoder-style, compute-bound regime.

Recipe (the pages give none; these are the stated readings):
  * numpy PCG64 ``default_rng(seed)``, ``standard_normal(dtype=float32)``.
  * Draw order Q, K, V (then W_Q, W_K, W_V, W_O for the layer).
  * bf16 inputs are fp32 draws rounded to the nearest bf16, ties to even.
  * Variants of one workload are nested: the H-head tensors are drawn once and
    variant (H_q, H_kv) keeps query heads [0, H_q) and K/V heads [0, H_kv).
  * "Peaky" keys: floor(0.01*N) key positions drawn without replacement from
    ``default_rng(2)``; the whole key vector there is multiplied by 8 in every
    K/V head (exact in bf16).
  * Sampled query rows: ``count`` distinct positions from ``default_rng(1)``,
    sorted.
  * Weights ~ N(0, 0.02) (0.02 is the standard deviation).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

__all__ = [
    "bf16_round",
    "Workload",
    "WORKLOADS",
    "draw_qkv",
    "select_variant",
    "sample_rows",
    "boundary_rows",
    "draw_layer",
    "draw_attn_case",
    "draw_varlen",
    "varlen_lengths",
]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16, so the
    GPU side can convert them to bf16 losslessly and the oracle can upcast them
    to float64 losslessly. NaN/Inf are not produced by the generators.
    """
    a = np.array(x, dtype=np.float32, copy=True, order="C")
    u = a.view(np.uint32)
    if np.any((u & np.uint32(0x7F800000)) == np.uint32(0x7F800000)):
        raise ValueError("bf16_round expects finite values")
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)          # finite inputs: no uint32 wrap-around
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return a


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    H: int                      # baseline head count; sets d = d_model / H
    d: int
    variants: Tuple[Tuple[int, int], ...]   # (H_q, H_kv)
    dtype: str                  # "f32" or "bf16"
    causal: Tuple[int, ...]
    scale: float
    sampled_rows: Optional[int] = None      # None: every row is checked
    peaky: bool = False
    layer: bool = False
    block: bool = False         # whole transformer block (RMSNorm, layer, SwiGLU)
    d_ff: int = 0               # SwiGLU width of a block workload
    d_model: int = 0
    rope_base: float = 10000.0
    varlen: int = 0             # > 0: a packed batch of this many sequences summing to N tokens
    description: str = ""


WORKLOADS = {
    # SQAT-m attention core, fp32, every row.
    "sqatm_core_f32": Workload(
        name="sqatm_core_f32", B=1, N=1024, H=16, d=16, variants=((8, 4),),
        dtype="f32", causal=(0, 1), scale=0.25,
        description="SQAT-m attention core B=1 N=1024 (8,4) d=16 fp32"),
    # SQAT-m full attention layer forward, bf16, causal, every output.
    "sqatm_layer_bf16": Workload(
        name="sqatm_layer_bf16", B=16, N=1024, H=16, d=16, variants=((8, 4),),
        dtype="bf16", causal=(1,), scale=0.25, layer=True, d_model=256,
        rope_base=10000.0,
        description="SQAT-m layer B=16 N=1024 D=256 (8,4) d=16 bf16 causal"),
    # SQAT-m transformer block forward (RMSNorm, SQA layer, SwiGLU 768,
    # residuals), bf16, causal; MHA / GQA / MQA variants for the
    # time-per-batch comparison of the SQAT-m card.
    "sqatm_block_bf16": Workload(
        name="sqatm_block_bf16", B=16, N=1024, H=16, d=16,
        variants=((8, 4), (16, 16), (16, 4), (16, 1)), dtype="bf16", causal=(1,),
        scale=0.25, block=True, d_model=256, d_ff=768, rope_base=10000.0,
        description="SQAT-m block B=16 N=1024 D=256 F=768 SQA(8,4) vs MHA/GQA/MQA bf16 causal"),
    # Long-context encoder-style attention at 32k.
    "long32k_bf16": Workload(
        name="long32k_bf16", B=1, N=32768, H=16, d=64,
        variants=((8, 4), (16, 16), (16, 4), (16, 1)), dtype="bf16",
        causal=(0,), scale=0.125, sampled_rows=4096,
        description="B=1 N=32768 d=64 SQA(8,4) vs MHA/GQA-4/MQA bf16 non-causal"),
    # Wider shape family: head dims 128 and 32, uneven head groups, and a
    # packed batch of sequences of mixed lengths (32768 tokens in 8).
    "long32k_d128_bf16": Workload(
        name="long32k_d128_bf16", B=1, N=32768, H=16, d=128, variants=((8, 4), (16, 16)),
        dtype="bf16", causal=(0, 1), scale=1.0 / 128 ** 0.5, sampled_rows=4096,
        description="B=1 N=32768 d=128 SQA(8,4) vs MHA bf16"),
    "long32k_d32_bf16": Workload(
        name="long32k_d32_bf16", B=1, N=32768, H=16, d=32, variants=((8, 4), (16, 16)),
        dtype="bf16", causal=(0,), scale=1.0 / 32 ** 0.5, sampled_rows=4096,
        description="B=1 N=32768 d=32 SQA(8,4) vs MHA bf16 non-causal"),
    "long32k_uneven_bf16": Workload(
        name="long32k_uneven_bf16", B=1, N=32768, H=16, d=64, variants=((12, 8), (6, 4)),
        dtype="bf16", causal=(0,), scale=0.125, sampled_rows=4096,
        description="B=1 N=32768 d=64, H_kv not dividing H_q: (12,8), (6,4) bf16 non-causal"),
    "varlen32k_bf16": Workload(
        name="varlen32k_bf16", B=1, N=32768, H=16, d=64, variants=((8, 4), (16, 16)),
        dtype="bf16", causal=(1, 0), scale=0.125, varlen=8,
        description="packed batch of 8 sequences (mixed lengths, 32768 tokens) d=64 SQA(8,4) vs MHA bf16"),
    "long131k_bf16": Workload(
        name="long131k_bf16", B=1, N=131072, H=16, d=64,
        variants=((8, 8), (4, 4), (16, 16)), dtype="bf16", causal=(0, 1),
        scale=0.125, sampled_rows=4096,
        description="B=1 N=131072 d=64 (8,8),(4,4) vs (16,16) bf16"),
    "long200k_peaky_bf16": Workload(
        name="long200k_peaky_bf16", B=1, N=200000, H=16, d=64,
        variants=((4, 4), (16, 16)), dtype="bf16", causal=(0,), scale=0.125,
        sampled_rows=4096, peaky=True,
        description="B=1 N=200000 d=64 (4,4) vs (16,16), 1% keys x8, bf16"),
}


def _normal(rng: np.random.Generator, shape, dtype: str, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "bf16":
        x = bf16_round(x)
    return x


def draw_qkv(B: int, H: int, N: int, d: int, dtype: str, seed: int = 0,
             peaky: bool = False, heads_q: Optional[int] = None,
             heads_kv: Optional[int] = None):
    """Draw Q, K, V of shape [B, heads, N, d] as float32 arrays.

    ``heads_q``/``heads_kv`` default to H. For bf16 the values are
    bf16-representable. Draw order is Q, K, V from one generator.
    """
    hq = H if heads_q is None else heads_q
    hk = H if heads_kv is None else heads_kv
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, hq, N, d), dtype)
    k = _normal(rng, (B, hk, N, d), dtype)
    v = _normal(rng, (B, hk, N, d), dtype)
    if peaky:
        pos = np.random.default_rng(2).choice(N, size=N // 100, replace=False)
        k[:, :, pos, :] *= np.float32(8.0)
    return q, k, v


def draw_upstream(shape, dtype: str = "bf16", seed: int = 100) -> np.ndarray:
    """Upstream gradient dL/dO for backward tests: N(0, 1) of the given shape
    as float32 (bf16-representable for "bf16"), from its own seeded stream."""
    rng = np.random.default_rng(seed)
    return _normal(rng, tuple(shape), dtype)


def select_variant(q: np.ndarray, k: np.ndarray, v: np.ndarray, H_q: int, H_kv: int):
    """Nested variant: query heads [0, H_q), K/V heads [0, H_kv), contiguous."""
    return (np.ascontiguousarray(q[:, :H_q]), np.ascontiguousarray(k[:, :H_kv]),
            np.ascontiguousarray(v[:, :H_kv]))


def sample_rows(N: int, count: int = 4096, seed: int = 1) -> np.ndarray:
    """``count`` distinct query positions in [0, N), sorted (all rows if N <= count)."""
    if N <= count:
        return np.arange(N, dtype=np.int64)
    r = np.random.default_rng(seed).choice(N, size=count, replace=False)
    return np.sort(r).astype(np.int64)


def boundary_rows(N: int, tile: int = 64) -> np.ndarray:
    """Rows at tile edges and the sequence ends, where masking bugs live."""
    cand = {0, 1, tile - 1, tile, 2 * tile - 1, 2 * tile, N - tile - 1, N - tile,
            N - 2, N - 1, (N // tile) * tile, (N // tile) * tile - 1}
    return np.array(sorted(c for c in cand if 0 <= c < N), dtype=np.int64)


def draw_layer(B: int, N: int, D: int, H: int, H_q: int, H_kv: int,
               seed: int = 0, w_std: float = 0.02):
    """X [B,N,D] ~ N(0,1) and W_Q [D,H_q*d], W_K/W_V [D,H_kv*d], W_O [H_q*d,D]
    ~ N(0, w_std), all bf16-representable float32, weights in [in, out] layout."""
    d = D // H
    rng = np.random.default_rng(seed)
    x = _normal(rng, (B, N, D), "bf16")
    wq = _normal(rng, (D, H_q * d), "bf16", w_std)
    wk = _normal(rng, (D, H_kv * d), "bf16", w_std)
    wv = _normal(rng, (D, H_kv * d), "bf16", w_std)
    wo = _normal(rng, (H_q * d, D), "bf16", w_std)
    return x, wq, wk, wv, wo


def draw_block(B: int, N: int, D: int, H: int, H_q: int, H_kv: int, F: int, seed: int = 0,
               wstd: Optional[float] = None):
    """Inputs of one transformer block: x ~ N(0, 1) [B, N, D]; RMSNorm gains
    1 + N(0, 0.1) [D] (two); W_Q, W_K, W_V, W_O as in ``draw_layer``'s shapes
    and W_gate, W_up [D, F], W_down [F, D], all ~ N(0, wstd) with wstd
    defaulting to 1/sqrt(fan_in) per matrix. bf16-representable float32.
    Draw order: x, norm1, W_Q, W_K, W_V, W_O, norm2, W_gate, W_up, W_down."""
    d = D // H
    rng = np.random.default_rng(seed)
    x = _normal(rng, (B, N, D), "bf16")

    def gain():
        g = _normal(rng, (D,), "f32", std=0.1) + np.float32(1.0)
        return bf16_round(g)

    def mat(fan_in, fan_out):
        std = wstd if wstd is not None else 1.0 / np.sqrt(fan_in)
        return _normal(rng, (fan_in, fan_out), "bf16", std=std)

    n1 = gain()
    wq, wk, wv, wo = mat(D, H_q * d), mat(D, H_kv * d), mat(D, H_kv * d), mat(H_q * d, D)
    n2 = gain()
    wg, wu, wd = mat(D, F), mat(D, F), mat(F, D)
    return x, n1, wq, wk, wv, wo, n2, wg, wu, wd


def varlen_lengths(total: int, count: int, seed: int = 3, min_len: int = 1) -> np.ndarray:
    """A length mix of ``count`` sequences summing to ``total`` tokens: cut
    points drawn uniformly without replacement (``default_rng(seed)``), so
    lengths range from a few tokens to several times the mean."""
    if count < 1 or total < count * min_len:
        raise ValueError("need total >= count * min_len")
    rng = np.random.default_rng(seed)
    spare = total - count * min_len
    cuts = np.sort(rng.choice(spare + count - 1, size=count - 1, replace=False))
    parts = np.diff(np.concatenate([[-1], cuts, [spare + count - 1]])) - 1
    return (parts + min_len).astype(np.int64)


def draw_varlen(lens, H_q: int, H_kv: int, d: int, dtype: str = "bf16", seed: int = 0):
    """Packed variable-length batch: the sequences of lengths ``lens`` are
    concatenated along the token axis. Returns Q [H_q, T, d], K/V [H_kv, T, d]
    ~ N(0, 1) (bf16-representable for "bf16"; draw order Q, K, V) and the
    offsets cu_seqlens [B+1] (int32, cu[0] = 0, cu[B] = T)."""
    lens = [int(x) for x in lens]
    T = int(sum(lens))
    rng = np.random.default_rng(seed)
    q = _normal(rng, (H_q, T, d), dtype)
    k = _normal(rng, (H_kv, T, d), dtype)
    v = _normal(rng, (H_kv, T, d), dtype)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return q, k, v, cu


def draw_attn_case(B: int, H_q: int, H_kv: int, N: int, d: int, dtype: str = "bf16",
                   seed: int = 0, peaky: bool = False):
    """Q [B,H_q,N,d], K/V [B,H_kv,N,d] drawn directly at the variant's head counts."""
    return draw_qkv(B, max(H_q, H_kv), N, d, dtype, seed=seed, peaky=peaky,
                    heads_q=H_q, heads_kv=H_kv)
