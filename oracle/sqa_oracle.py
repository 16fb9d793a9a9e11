"""Plain, slow, float64 CPU oracle for Sparse Query Attention (SQA).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package. The HIP path never imports it, and it imports nothing from the
HIP path: the two share no code, tables or helpers. Seeded inputs come from
the separate ``synth`` module, which holds no attention arithmetic.

What is computed, and where it comes from
-----------------------------------------
* SQA keeps the per-head width d = d_model / H of the baseline and reduces the
  number of *query* heads H_q below H, instead of reducing key/value heads
  further ("SQAT-m: Sparse Query Attention Transformer mini", introduction and
  "Architecture details"; SQA paper abstract, chatpaper page). The attention
  FLOPs drop in proportion to H_q / H.
* Query heads are split into H_kv contiguous groups, each sharing one key head
  and one value head; one group is MQA and H groups is MHA ("GQA: Training
  Generalized Multi-Query Transformer Models", nlp-lineage page, section
  "The idea"). Query head i reads K/V head floor(i * H_kv / H_q).
* The pages name multi-head attention and the attention-score computation but
  never write the formula. The oracle uses the textbook per-head
  scaled-dot-product softmax attention:
      s_tu = scale * <Q[b,i,t,:], K[b,j,u,:]>,   u in U_t
      O[b,i,t,:] = sum_u softmax_u(s_tu) V[b,j,u,:]
  with U_t = all keys (encoder-style) or {u <= t} (causal, the SQAT-m text
  generation model), and optionally LSE[b,i,t] = log sum_u exp(s_tu).
* The backward pass (the pages place SQA's gains in training: pre-training and
  fine-tuning in the SQA abstract, training time per batch on the SQAT-m
  card's results) is the exact derivative of that forward for an upstream
  gradient dO, written out with the chain rule through the softmax:
      P = softmax(S),  dP = dO V^T,  dS = P * (dP - rowsum(P * dP)),
      dQ = scale dS K,  dK_j = scale sum_{i in group j} dS^T Q_i,
      dV_j = sum_{i in group j} P^T dO_i.
* The block (SQAT-m card, "Architecture details": dim 256, RMS Norm, SwiGLU
  feed forward with 768 dim, RoPE). The card does not give the order; the
  oracle uses the pre-norm residual block
      h = x + layer(rms_norm(x, g1)),  y = h + swiglu(rms_norm(h, g2))
  with rms_norm(x, g) = x / sqrt(mean_c x_c^2 + eps) * g and
  swiglu(z) = (silu(z W_gate) * (z W_up)) W_down, silu(u) = u / (1 + e^-u).
* Packed variable-length batches (not on the pages; the plainest reading of
  a batch of sequences of different lengths): sequences b = 0..B-1 are
  concatenated along the token axis, sequence b owning tokens
  cu[b] .. cu[b+1]-1; each attends only within itself, with positions
  restarting at 0 for the causal mask. Layout [heads, T, d].
* The layer (SQAT-m, "Architecture details" and "Model size difference"):
  Q = X W_Q (H_q*d wide), K = X W_K and V = X W_V (H_kv*d wide), RoPE on Q and
  K, SQA, then Y = O_flat W_O with W_O of H_q*d rows. Weights are [in, out].
  The pages say "RoPE" only; the oracle uses rotate-half pairs (c, c + d/2)
  with theta_c = base^(-2c/d) and angle t * theta_c. Which pairing RxLM uses
  is parity unpinned (an interleaved pairing gives the same layer output up to
  a fixed permutation of the W_Q / W_K columns).

Every function upcasts its inputs to float64 (bf16 and fp32 upcasts are
exact) and follows the definition directly: two-pass max-subtracted softmax,
BLAS matrix products, no tiling beyond chunking query rows to bound memory.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "kv_head_index",
    "attention",
    "attention_bwd",
    "attention_varlen",
    "attention_bwd_varlen",
    "rope",
    "layer",
    "layer_weight_shapes",
    "rms_norm",
    "swiglu",
    "block",
    "attention_param_count",
]


def kv_head_index(i: int, H_q: int, H_kv: int) -> int:
    """K/V head read by query head i: floor(i * H_kv / H_q).

    Contiguous grouping of query heads ("GQA ..." page, "The idea"): with H_kv
    groups of g = H_q / H_kv heads this is i // g; H_kv = 1 is MQA and
    H_kv = H_q is MHA.
    """
    if not (1 <= H_kv <= H_q):
        raise ValueError("need 1 <= H_kv <= H_q")
    if not (0 <= i < H_q):
        raise ValueError("query head index out of range")
    return (i * H_kv) // H_q


def _attend_rows(q_rows: np.ndarray, t_rows: np.ndarray, kj: np.ndarray,
                 vj: np.ndarray, scale: float, causal: bool):
    """Softmax attention of a block of query rows against one K/V head (fp64).

    q_rows [R, d] at positions t_rows [R]; kj, vj [N, d]. Returns O [R, d] and
    LSE [R]. Two passes: row max, then exp / sum / weighted sum of V.
    """
    s = (q_rows @ kj.T) * scale                       # [R, N]
    if causal:
        u = np.arange(kj.shape[0])
        s = np.where(u[None, :] <= t_rows[:, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ vj) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: Optional[float] = None,
              causal: bool = False, rows: Optional[Sequence[int]] = None,
              return_lse: bool = False, threads: int = 1, chunk_elems: int = 1 << 23):
    """SQA forward in float64.

    q: [B, H_q, N, d]; k, v: [B, H_kv, N, d]; H_kv must be in [1, H_q]. The
    general mapping floor(i*H_kv/H_q) is used, so H_kv need not divide H_q.
    ``scale`` defaults to 1/sqrt(d). ``rows`` selects query positions (the
    same positions for every (b, head)); the result then has len(rows) rows.
    ``threads`` > 1 spreads (b, head, row-chunk) tasks over threads (numpy
    releases the GIL in BLAS and ufuncs); results do not depend on it.
    Returns O [B, H_q, R, d] float64 (and LSE [B, H_q, R] if return_lse).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("expected 4-D [B, H, N, d] arrays")
    B, H_q, N, d = q.shape
    Bk, H_kv, Nk, dk = k.shape
    if (Bk, Nk, dk) != (B, N, d) or v.shape != k.shape:
        raise ValueError("q/k/v shapes disagree")
    if not (1 <= H_kv <= H_q):
        raise ValueError("need 1 <= H_kv <= H_q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    t_all = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    R = t_all.shape[0]
    out = np.empty((B, H_q, R, d), dtype=np.float64)
    lse = np.empty((B, H_q, R), dtype=np.float64)
    if R == 0 or B == 0:
        return (out, lse) if return_lse else out

    chunk = max(1, min(R, chunk_elems // max(N, 1)))
    kv64 = {}

    def kv_of(b: int, j: int):
        key = (b, j)
        if key not in kv64:
            kv64[key] = (k[b, j].astype(np.float64), v[b, j].astype(np.float64))
        return kv64[key]

    tasks = []
    for b in range(B):
        for i in range(H_q):
            j = kv_head_index(i, H_q, H_kv)
            kv_of(b, j)
            for r0 in range(0, R, chunk):
                tasks.append((b, i, j, r0, min(R, r0 + chunk)))

    def run(task):
        b, i, j, r0, r1 = task
        kj, vj = kv64[(b, j)]
        t_rows = t_all[r0:r1]
        q_rows = q[b, i, t_rows].astype(np.float64)
        o, ls = _attend_rows(q_rows, t_rows, kj, vj, float(scale), causal)
        out[b, i, r0:r1] = o
        lse[b, i, r0:r1] = ls

    if threads <= 1:
        for t in tasks:
            run(t)
    else:
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:  # pragma: no cover - threadpoolctl is installed
            threadpool_limits = None
        if threadpool_limits is not None:
            with threadpool_limits(limits=1):
                with ThreadPoolExecutor(max_workers=threads) as ex:
                    list(ex.map(run, tasks))
        else:
            with ThreadPoolExecutor(max_workers=threads) as ex:
                list(ex.map(run, tasks))
    return (out, lse) if return_lse else out


def attention_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens: Sequence[int],
                     scale: Optional[float] = None, causal: bool = False, return_lse: bool = False,
                     threads: int = 1):
    """SQA forward over packed variable-length sequences, float64.

    q: [H_q, T, d]; k, v: [H_kv, T, d]; cu_seqlens: B+1 non-decreasing token
    offsets with cu[0] = 0 and cu[B] = T. Sequence b is tokens
    cu[b] .. cu[b+1]-1 of every head; it attends only to its own keys, and its
    causal positions count from 0. Each sequence is the dense ``attention``
    above on its slice. Returns O [H_q, T, d] (and LSE [H_q, T]).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("expected 3-D [heads, T, d] arrays")
    H_q, T, d = q.shape
    if k.shape[1:] != (T, d) or v.shape != k.shape:
        raise ValueError("q/k/v shapes disagree")
    cu = [int(x) for x in cu_seqlens]
    if len(cu) < 1 or cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must rise from 0 to T")
    out = np.zeros((H_q, T, d), dtype=np.float64)
    lse = np.zeros((H_q, T), dtype=np.float64)
    for a, b in zip(cu, cu[1:]):
        if b == a:
            continue
        o, ls = attention(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], scale=scale, causal=causal,
                          return_lse=True, threads=threads)
        out[:, a:b] = o[0]
        lse[:, a:b] = ls[0]
    return (out, lse) if return_lse else out


def _attend_rows_bwd(q_rows: np.ndarray, t_rows: np.ndarray, kj: np.ndarray, vj: np.ndarray,
                     do_rows: np.ndarray, scale: float, causal: bool, absolute: bool = False,
                     o_rows: Optional[np.ndarray] = None):
    """Gradients of one block of query rows against one K/V head (fp64).

    Returns dQ [R, d] for these rows and their contributions dK_part, dV_part
    [N, d] to the head's key and value gradients. The softmax is recomputed
    exactly (two passes). With ``o_rows`` (the forward output of these rows)
    D_t = sum_c dO_tc O_tc; otherwise D_t = sum_u P_tu dP_tu, the same value
    for the exact output. With ``absolute`` the same three sums are formed
    from the absolute values of their terms instead (see ``attention_bwd``).
    """
    s = (q_rows @ kj.T) * scale                       # [R, N]
    if causal:
        u = np.arange(kj.shape[0])
        s = np.where(u[None, :] <= t_rows[:, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)              # masked entries are exactly 0
    dp = do_rows @ vj.T                               # dL/dP        [R, N]
    D = (p * dp).sum(axis=1, keepdims=True) if o_rows is None else (do_rows * o_rows).sum(axis=1, keepdims=True)
    ds = p * (dp - D)                                 # dL/dS (softmax Jacobian)
    if absolute:
        ads = np.abs(ds)
        return ((ads @ np.abs(kj)) * abs(scale), (ads.T @ np.abs(q_rows)) * abs(scale), p.T @ np.abs(do_rows))
    dq = (ds @ kj) * scale
    dk_part = (ds.T @ q_rows) * scale
    dv_part = p.T @ do_rows
    return dq, dk_part, dv_part


def attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                  scale: Optional[float] = None, causal: bool = False,
                  rows: Optional[Sequence[int]] = None, threads: int = 1,
                  chunk_elems: int = 1 << 22, absolute: bool = False, o: Optional[np.ndarray] = None):
    """Backward of ``attention`` in float64: returns (dQ, dK, dV).

    ``o`` (optional, shaped like dout): a forward output to take
    D_t = sum_c dout_tc o_tc from, as the library's backward does (it takes
    the forward's output as an input); without it D_t = sum_u P_tu dP_tu,
    which is the same for the exact output.

    ``absolute=True`` returns instead the same sums with every term replaced
    by its absolute value: |scale| sum_u |dS_tu| |K_u|,
    |scale| sum_{i,t} |dS_tu| |Q_t| and sum_{i,t} P_tu |dO_t|. These are the
    magnitudes that set the rounding error of any computation of the
    gradients (for a sum of products, |fl(sum) - sum| is bounded by a
    multiple of the sum of the products' absolute values); dS sums to zero
    along each row, so |dQ| itself can be far smaller.

    dout is the upstream gradient dL/dO, shaped like O [B, H_q, N, d]. dK and
    dV [B, H_kv, N, d] sum the contributions of every query head of a K/V
    head's group. With ``rows`` only dQ is computed, for those query positions
    ([B, H_q, R, d]); dK and dV need every row and are returned as None.
    ``threads`` > 1 splits each (b, K/V head)'s rows into slices whose partial
    sums are added in slice order, so results do not depend on it.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    dout = np.asarray(dout)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4 or dout.shape != q.shape:
        raise ValueError("expected 4-D [B, H, N, d] arrays, dout shaped like q")
    B, H_q, N, d = q.shape
    Bk, H_kv, Nk, dk_ = k.shape
    if (Bk, Nk, dk_) != (B, N, d) or v.shape != k.shape:
        raise ValueError("q/k/v shapes disagree")
    if not (1 <= H_kv <= H_q):
        raise ValueError("need 1 <= H_kv <= H_q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    scale = float(scale)
    want_kv = rows is None
    t_all = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    R = t_all.shape[0]
    dq = np.zeros((B, H_q, R, d), dtype=np.float64)
    dk = np.zeros((B, H_kv, N, d), dtype=np.float64) if want_kv else None
    dv = np.zeros((B, H_kv, N, d), dtype=np.float64) if want_kv else None
    if R == 0 or B == 0 or N == 0:
        return dq, dk, dv

    chunk = max(1, min(R, chunk_elems // max(N, 1)))
    # work items of one (b, j): (query head i, row chunk) in a fixed order
    groups = {}
    for b in range(B):
        for i in range(H_q):
            j = kv_head_index(i, H_q, H_kv)
            for r0 in range(0, R, chunk):
                groups.setdefault((b, j), []).append((i, r0, min(R, r0 + chunk)))
    nslice = max(1, min(threads, 8))
    tasks = []
    for (b, j), items in groups.items():
        per = -(-len(items) // nslice)
        for sl in range(nslice):
            part = items[sl * per:(sl + 1) * per]
            if part:
                tasks.append((b, j, sl, part))

    def run(task):
        b, j, sl, part = task
        kj = k[b, j].astype(np.float64)
        vj = v[b, j].astype(np.float64)
        dk_acc = np.zeros((N, d), dtype=np.float64) if want_kv else None
        dv_acc = np.zeros((N, d), dtype=np.float64) if want_kv else None
        for (i, r0, r1) in part:
            t_rows = t_all[r0:r1]
            gq, gk, gv = _attend_rows_bwd(q[b, i, t_rows].astype(np.float64), t_rows, kj, vj,
                                          dout[b, i, t_rows].astype(np.float64), scale, causal, absolute,
                                          None if o is None else np.asarray(o)[b, i, t_rows].astype(np.float64))
            dq[b, i, r0:r1] = gq
            if want_kv:
                dk_acc += gk
                dv_acc += gv
        return (b, j, sl, dk_acc, dv_acc)

    if threads <= 1:
        results = [run(t) for t in tasks]
    else:
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:  # pragma: no cover - threadpoolctl is installed
            threadpool_limits = None
        if threadpool_limits is not None:
            with threadpool_limits(limits=1):
                with ThreadPoolExecutor(max_workers=threads) as ex:
                    results = list(ex.map(run, tasks))
        else:
            with ThreadPoolExecutor(max_workers=threads) as ex:
                results = list(ex.map(run, tasks))
    if want_kv:
        for (b, j, sl, gk, gv) in sorted(results, key=lambda r: (r[0], r[1], r[2])):
            dk[b, j] += gk
            dv[b, j] += gv
    return dq, dk, dv


def attention_bwd_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                         cu_seqlens: Sequence[int], scale: Optional[float] = None, causal: bool = False,
                         threads: int = 1):
    """Backward of ``attention_varlen`` in float64: (dQ [H_q, T, d], dK, dV
    [H_kv, T, d]). Sequences are independent, so each is the dense backward
    above on its slice."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    dout = np.asarray(dout)
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3 or dout.shape != q.shape:
        raise ValueError("expected 3-D [heads, T, d] arrays, dout shaped like q")
    H_q, T, d = q.shape
    if k.shape[1:] != (T, d) or v.shape != k.shape:
        raise ValueError("q/k/v shapes disagree")
    cu = [int(x) for x in cu_seqlens]
    if len(cu) < 1 or cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must rise from 0 to T")
    dq = np.zeros((H_q, T, d), dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for a, b in zip(cu, cu[1:]):
        if b == a:
            continue
        gq, gk, gv = attention_bwd(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], dout[None, :, a:b],
                                   scale=scale, causal=causal, threads=threads)
        dq[:, a:b] = gq[0]
        dk[:, a:b] = gk[0]
        dv[:, a:b] = gv[0]
    return dq, dk, dv


def rope(x: np.ndarray, base: float, positions: Optional[np.ndarray] = None) -> np.ndarray:
    """Rotary position embedding, rotate-half convention, float64.

    x: [..., N, d] with d even; position of row n is positions[n] (default n).
    For c < d/2 the pair (x_c, x_{c+d/2}) is rotated by angle t * theta_c,
    theta_c = base^(-2c/d):
        y_c       = x_c cos - x_{c+d/2} sin
        y_{c+d/2} = x_c sin + x_{c+d/2} cos
    """
    x = np.asarray(x, dtype=np.float64)
    N, d = x.shape[-2], x.shape[-1]
    if d % 2:
        raise ValueError("RoPE needs an even head dimension")
    h = d // 2
    t = np.arange(N, dtype=np.float64) if positions is None else np.asarray(positions, np.float64)
    theta = base ** (-2.0 * np.arange(h, dtype=np.float64) / d)
    ang = t[:, None] * theta[None, :]                  # [N, h]
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)


def layer_weight_shapes(D: int, H: int, H_q: int, H_kv: int):
    """Projection shapes of one SQA layer ([in, out] layout).

    d = D / H is kept from the baseline head split; the query and output
    projections are H_q*d wide and the key/value projections H_kv*d wide
    (SQAT-m model card, "Architecture details" and "Model size difference").
    """
    if D % H:
        raise ValueError("D must be a multiple of H")
    d = D // H
    return {"W_Q": (D, H_q * d), "W_K": (D, H_kv * d), "W_V": (D, H_kv * d),
            "W_O": (H_q * d, D)}


def attention_param_count(D: int, H: int, H_q: int, H_kv: int) -> int:
    """Number of projection weights in one attention layer (no biases)."""
    return sum(a * b for a, b in layer_weight_shapes(D, H, H_q, H_kv).values())


def layer(x: np.ndarray, wq: np.ndarray, wk: np.ndarray, wv: np.ndarray, wo: np.ndarray,
          H: int, H_q: int, H_kv: int, rope_base: float = 10000.0,
          scale: Optional[float] = None, causal: bool = True,
          threads: int = 1) -> np.ndarray:
    """One SQA attention layer forward in float64.

    x [B, N, D]; weights in [in, out] layout with the shapes of
    ``layer_weight_shapes``. Head h owns projection columns [h*d, (h+1)*d).
    No biases, norms or residual. Returns Y [B, N, D].
    """
    x = np.asarray(x, dtype=np.float64)
    B, N, D = x.shape
    shapes = layer_weight_shapes(D, H, H_q, H_kv)
    for name, w in (("W_Q", wq), ("W_K", wk), ("W_V", wv), ("W_O", wo)):
        if tuple(np.shape(w)) != shapes[name]:
            raise ValueError(f"{name} has shape {np.shape(w)}, expected {shapes[name]}")
    d = D // H

    def heads(y: np.ndarray, nh: int) -> np.ndarray:       # [B,N,nh*d] -> [B,nh,N,d]
        return y.reshape(B, N, nh, d).transpose(0, 2, 1, 3)

    qh = rope(heads(x @ np.asarray(wq, np.float64), H_q), rope_base)
    kh = rope(heads(x @ np.asarray(wk, np.float64), H_kv), rope_base)
    vh = heads(x @ np.asarray(wv, np.float64), H_kv)
    o = attention(qh, kh, vh, scale=scale, causal=causal, threads=threads)
    o_flat = o.transpose(0, 2, 1, 3).reshape(B, N, H_q * d)
    return o_flat @ np.asarray(wo, np.float64)


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """RMS normalisation over the last axis in float64 (SQAT-m card,
    "Architecture details": RMS Norm): x / sqrt(mean(x^2) + eps) * weight."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    if w.shape != x.shape[-1:]:
        raise ValueError("weight must match the last axis of x")
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def swiglu(z: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """SwiGLU feed forward in float64 (SQAT-m card, "Architecture details":
    SwiGLU feed forward with 768 dim): (silu(z W_gate) * (z W_up)) W_down with
    silu(u) = u * sigmoid(u); weights [in, out]."""
    z = np.asarray(z, dtype=np.float64)
    g = z @ np.asarray(w_gate, dtype=np.float64)
    u = z @ np.asarray(w_up, dtype=np.float64)
    silu = g / (1.0 + np.exp(-g))
    return (silu * u) @ np.asarray(w_down, dtype=np.float64)


def block(x: np.ndarray, norm1: np.ndarray, wq: np.ndarray, wk: np.ndarray, wv: np.ndarray,
          wo: np.ndarray, norm2: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
          w_down: np.ndarray, H: int, H_q: int, H_kv: int, rope_base: float = 10000.0,
          scale: Optional[float] = None, causal: bool = True, eps: float = 1e-6,
          threads: int = 1) -> np.ndarray:
    """One SQAT-m transformer block forward in float64 (pre-norm residual):
    h = x + layer(rms_norm(x, norm1)); y = h + swiglu(rms_norm(h, norm2)).
    x [B, N, D]; attention weights as ``layer``; w_gate, w_up [D, F];
    w_down [F, D]. Returns y [B, N, D]."""
    x = np.asarray(x, dtype=np.float64)
    F = np.shape(w_gate)[1]
    D = x.shape[-1]
    if np.shape(w_gate) != (D, F) or np.shape(w_up) != (D, F) or np.shape(w_down) != (F, D):
        raise ValueError("feed-forward weights must be [D, F], [D, F], [F, D]")
    h = x + layer(rms_norm(x, norm1, eps), wq, wk, wv, wo, H, H_q, H_kv, rope_base=rope_base,
                  scale=scale, causal=causal, threads=threads)
    return h + swiglu(rms_norm(h, norm2, eps), w_gate, w_up, w_down)
