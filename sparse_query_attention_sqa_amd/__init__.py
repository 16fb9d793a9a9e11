"""Python binding for libsqa: Sparse Query Attention on MI355X.

Argument marshalling only. Every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/sqa.h``; torch is used for
device memory and the current HIP stream. There is no fallback path: if the
library is not built, importing the functions raises.

    sqa_attn_fwd(q, k, v, *, scale=None, causal=False, out=None, return_lse=False)
    sqa_attn_fwd_varlen(q, k, v, cu_seqlens, max_seqlen=None, *, scale=None, causal=False,
                        out=None, return_lse=False)
    sqa_attn_bwd(q, k, v, o, dout, lse, *, scale=None, causal=False, dq=None, dk=None,
                 dv=None, workspace=None)
    sqa_attn_bwd_workspace_bytes(B, H_q, N, d, dtype="bf16")
    sqa_attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, *, scale=None, causal=False)
    sqa_attn_bwd_varlen(q, k, v, o, dout, lse, cu_seqlens, max_seqlen=None, *, scale=None, causal=False,
                        dq=None, dk=None, dv=None, workspace=None)
    sqa_attn_bwd_varlen_workspace_bytes(B, H_q, T, d, dtype="bf16")
    sqa_layer_fwd(x, w_q, w_k, w_v, w_o, *, H, H_q, H_kv, rope_base=10000.0,
                  scale=None, causal=True, out=None, workspace=None)
    sqa_layer_workspace_bytes(B, N, D, H, H_q, H_kv, dtype="bf16")
    sqa_block_fwd(x, norm1, w_q, w_k, w_v, w_o, norm2, w_gate, w_up, w_down, *, H, H_q, H_kv,
                  rope_base=10000.0, scale=None, eps=1e-6, causal=True, out=None, workspace=None)
    sqa_block_workspace_bytes(B, N, D, H, H_q, H_kv, F, dtype="bf16")
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = ["SQAError", "lib_path", "load_library", "sqa_attn_fwd", "sqa_attn_fwd_varlen",
           "sqa_attn_fwd_num_splits", "sqa_attn_fwd_tail_splits", "sqa_attn_bwd", "sqa_attn_bwd_noalloc", "sqa_attn_bwd_num_splits",
           "sqa_attn_bwd_split_workspace_bytes", "sqa_attn_bwd_varlen_split_workspace_bytes",
           "sqa_attn_bwd_varlen", "sqa_attn_bwd_varlen_workspace_bytes",
           "sqa_attn_bwd_workspace_bytes", "sqa_layer_fwd", "sqa_block_fwd",
           "sqa_block_workspace_bytes",
           "sqa_layer_workspace_bytes", "sqa_status_str", "sqa_version",
           "SQA_F32", "SQA_BF16"]

SQA_F32 = 0
SQA_BF16 = 1

_STATUS = {0: "SQA_OK", 1: "SQA_ERR_NULL", 2: "SQA_ERR_SHAPE", 3: "SQA_ERR_UNSUPPORTED",
           4: "SQA_ERR_ALIGN", 5: "SQA_ERR_WORKSPACE", 6: "SQA_ERR_HIP", 7: "SQA_ERR_ARG"}

_LIB = None


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsqa.so")


class SQAError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_STATUS.get(status, status)}: {message}")


def load_library() -> ctypes.CDLL:
    """Load libsqa.so (built in-tree by ``__graft_entry__.build()``)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"libsqa.so is not built ({path}); run __graft_entry__.build() "
                          "or python -m sparse_query_attention_sqa_amd._build")
    lib = ctypes.CDLL(path)
    i64, vp, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    lib.sqa_attn_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, f32,
                                 ctypes.c_int, vp, vp]
    lib.sqa_attn_fwd.restype = ctypes.c_int
    lib.sqa_attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                        f32, ctypes.c_int, vp, vp]
    lib.sqa_attn_fwd_varlen.restype = ctypes.c_int
    lib.sqa_attn_fwd_split.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, f32,
                                       ctypes.c_int, vp, i64, vp, ctypes.c_size_t, vp]
    lib.sqa_attn_fwd_split.restype = ctypes.c_int
    lib.sqa_attn_fwd_varlen_split.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                              f32, ctypes.c_int, vp, i64, vp, ctypes.c_size_t, vp]
    lib.sqa_attn_fwd_varlen_split.restype = ctypes.c_int
    lib.sqa_attn_fwd_num_splits.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, i64]
    lib.sqa_attn_fwd_num_splits.restype = i64
    lib.sqa_attn_fwd_tail_splits.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.sqa_attn_fwd_tail_splits.restype = i64
    lib.sqa_attn_fwd_tail_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.sqa_attn_fwd_tail_workspace_bytes.restype = ctypes.c_size_t
    lib.sqa_attn_fwd_tail.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, f32, ctypes.c_int,
                                      vp, vp, ctypes.c_size_t, vp]
    lib.sqa_attn_fwd_tail.restype = ctypes.c_int
    lib.sqa_attn_fwd_split_workspace_bytes.argtypes = [i64, i64, ctypes.c_int, i64]
    lib.sqa_attn_fwd_split_workspace_bytes.restype = ctypes.c_size_t
    lib.sqa_attn_bwd_split.argtypes = [vp] * 9 + [i64] * 5 + [ctypes.c_int, f32, ctypes.c_int, i64, vp,
                                                              ctypes.c_size_t, vp]
    lib.sqa_attn_bwd_split.restype = ctypes.c_int
    lib.sqa_attn_bwd_varlen_split.argtypes = [vp] * 10 + [i64] * 6 + [ctypes.c_int, f32, ctypes.c_int, i64, vp,
                                                                      ctypes.c_size_t, vp]
    lib.sqa_attn_bwd_varlen_split.restype = ctypes.c_int
    lib.sqa_attn_bwd_split_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, i64]
    lib.sqa_attn_bwd_split_workspace_bytes.restype = ctypes.c_size_t
    lib.sqa_attn_bwd_varlen_split_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, i64]
    lib.sqa_attn_bwd_varlen_split_workspace_bytes.restype = ctypes.c_size_t
    lib.sqa_attn_bwd_num_splits.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, i64]
    lib.sqa_attn_bwd_num_splits.restype = i64
    lib.sqa_attn_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.sqa_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.sqa_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                 ctypes.c_int, f32, ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.sqa_attn_bwd.restype = ctypes.c_int
    lib.sqa_attn_bwd_noalloc.argtypes = [vp] * 9 + [i64] * 5 + [ctypes.c_int, f32, ctypes.c_int, vp]
    lib.sqa_attn_bwd_noalloc.restype = ctypes.c_int
    lib.sqa_attn_bwd_varlen_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.sqa_attn_bwd_varlen_workspace_bytes.restype = ctypes.c_size_t
    lib.sqa_attn_bwd_varlen.argtypes = [vp] * 10 + [i64] * 6 + [ctypes.c_int, f32, ctypes.c_int, vp,
                                                                ctypes.c_size_t, vp]
    lib.sqa_attn_bwd_varlen.restype = ctypes.c_int
    lib.sqa_layer_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int]
    lib.sqa_layer_workspace_bytes.restype = ctypes.c_size_t
    lib.sqa_layer_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, f32,
                                  ctypes.c_int, ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.sqa_layer_fwd.restype = ctypes.c_int
    lib.sqa_block_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i64, ctypes.c_int]
    lib.sqa_block_workspace_bytes.restype = ctypes.c_size_t
    lib.sqa_block_fwd.argtypes = [vp] * 11 + [i64] * 7 + [f32, f32, f32, ctypes.c_int, ctypes.c_int,
                                                          vp, ctypes.c_size_t, vp]
    lib.sqa_block_fwd.restype = ctypes.c_int
    lib.sqa_status_str.argtypes = [ctypes.c_int]
    lib.sqa_status_str.restype = ctypes.c_char_p
    lib.sqa_last_error.argtypes = []
    lib.sqa_last_error.restype = ctypes.c_char_p
    lib.sqa_version.argtypes = []
    lib.sqa_version.restype = ctypes.c_int
    _LIB = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().sqa_last_error().decode(errors="replace")
        raise SQAError(status, msg)


def sqa_status_str(status: int) -> str:
    return load_library().sqa_status_str(status).decode()


def sqa_version() -> int:
    return load_library().sqa_version()


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SQA_BF16
    if t.dtype == torch.float32:
        return SQA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _require_device(*ts) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("libsqa takes GPU tensors only (no CPU fallback)")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def sqa_attn_fwd(q, k, v, *, scale: Optional[float] = None, causal: bool = False, out=None,
                 return_lse: bool = False, num_splits: Optional[int] = None, tail: Optional[bool] = None):
    """SQA attention forward on the GPU.

    q [B, H_q, N, d]; k, v [B, H_kv, N, d]; bf16 or fp32, contiguous, on the
    same GPU; d in {16, 32, 64, 128}. Query head i reads K/V head
    floor(i * H_kv / H_q). Returns o [B, H_q, N, d] (and lse [B, H_q, N] fp32
    if ``return_lse``). ``num_splits``: key-range splits (bf16, d = 64 only;
    None: the library's choice, sqa_attn_fwd_num_splits); with more than one
    a workspace is allocated from torch's caching allocator. ``tail``: the
    tail-split schedule (sqa_attn_fwd_tail) where the library plans one;
    None uses it when num_splits is also left to the library, False never.
    """
    torch = _torch()
    lib = load_library()
    _require_device(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected 4-D [B, H, N, d] tensors")
    if k.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("k and v must match; q, k, v must share a dtype")
    B, H_q, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError("q and k/v shapes disagree")
    H_kv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require_device(out)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    lse = torch.empty((B, H_q, N), dtype=torch.float32, device=q.device) if return_lse else None
    if tail is None:
        tail = num_splits is None
    if num_splits is None:
        num_splits = lib.sqa_attn_fwd_num_splits(B, H_q, H_kv, N, d, _dtype_code(q), int(bool(causal)), 0)
    tail_bytes = 0
    if num_splits == 1 and tail:
        tail_bytes = int(lib.sqa_attn_fwd_tail_workspace_bytes(B, H_q, H_kv, N, d, _dtype_code(q),
                                                               int(bool(causal))))
    if tail_bytes > 0:
        ws = torch.empty(tail_bytes, dtype=torch.uint8, device=q.device)
        st = lib.sqa_attn_fwd_tail(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H_q, H_kv,
                                   N, d, _dtype_code(q), float(scale), int(bool(causal)),
                                   lse.data_ptr() if lse is not None else None, ws.data_ptr(), tail_bytes,
                                   _stream_handle(q.device))
    elif num_splits == 1:
        st = lib.sqa_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H_q, H_kv,
                              N, d, _dtype_code(q), float(scale), int(bool(causal)),
                              lse.data_ptr() if lse is not None else None, _stream_handle(q.device))
    else:
        ws, nbytes = _split_workspace(lib, B * H_q * N, d, q, num_splits)
        st = lib.sqa_attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H_q, H_kv,
                                    N, d, _dtype_code(q), float(scale), int(bool(causal)),
                                    lse.data_ptr() if lse is not None else None, int(num_splits),
                                    ws, nbytes, _stream_handle(q.device))
    _check(st)
    return (out, lse) if return_lse else out


def _split_workspace(lib, rows: int, d: int, q, num_splits: int):
    """Device workspace for a split forward (None, 0 when it needs none)."""
    nbytes = lib.sqa_attn_fwd_split_workspace_bytes(rows, d, _dtype_code(q), int(num_splits))
    if nbytes == 0:
        return None, 0
    buf = _torch().empty(nbytes, dtype=_torch().uint8, device=q.device)
    return buf.data_ptr(), nbytes


def sqa_attn_fwd_tail_splits(B: int, H_q: int, H_kv: int, N: int, d: int, dtype: str = "bf16",
                             causal: bool = False) -> int:
    """Key ranges per tail workgroup the library plans (1: no tail split)."""
    code = SQA_BF16 if dtype == "bf16" else SQA_F32
    return int(load_library().sqa_attn_fwd_tail_splits(B, H_q, H_kv, N, d, code, int(bool(causal))))


def sqa_attn_fwd_num_splits(B: int, H_q: int, H_kv: int, N: int, d: int, dtype: str = "bf16",
                            causal: bool = False, T: int = 0) -> int:
    """The library's recommended key-range splits (packed batch: T tokens, N = max_seqlen)."""
    code = SQA_BF16 if dtype == "bf16" else SQA_F32
    return int(load_library().sqa_attn_fwd_num_splits(B, H_q, H_kv, N, d, code, int(bool(causal)), T))


def sqa_attn_fwd_varlen(q, k, v, cu_seqlens, max_seqlen: Optional[int] = None, *,
                        scale: Optional[float] = None, causal: bool = False, out=None,
                        return_lse: bool = False, num_splits: Optional[int] = None):
    """SQA attention forward over a packed batch of variable-length sequences.

    q [H_q, T, d]; k, v [H_kv, T, d] (bf16 or fp32); cu_seqlens: int32 GPU
    tensor [B + 1] of token offsets (0, ..., T). Sequence b is tokens
    cu[b] .. cu[b+1]-1 and attends only within itself. ``max_seqlen`` (the
    longest sequence) sizes the launch; if None it is read from cu_seqlens,
    which synchronises with the device. Returns o [H_q, T, d] (and lse
    [H_q, T] fp32 if ``return_lse``). ``num_splits`` as in sqa_attn_fwd (the
    library's choice is made for the longest sequence).
    """
    torch = _torch()
    lib = load_library()
    _require_device(q, k, v, cu_seqlens)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("expected 3-D [H, T, d] tensors")
    if k.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("k and v must match; q, k, v must share a dtype")
    H_q, T, d = q.shape
    if k.shape[1] != T or k.shape[2] != d:
        raise ValueError("q and k/v shapes disagree")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of B + 1 offsets")
    B = cu_seqlens.numel() - 1
    if max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if B > 0 else 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require_device(out)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    lse = torch.empty((H_q, T), dtype=torch.float32, device=q.device) if return_lse else None
    if num_splits is None:
        num_splits = lib.sqa_attn_fwd_num_splits(B, H_q, k.shape[0], int(max_seqlen), d, _dtype_code(q),
                                                 int(bool(causal)), T)
    if num_splits == 1:
        st = lib.sqa_attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     cu_seqlens.data_ptr(), B, H_q, k.shape[0], T, int(max_seqlen), d,
                                     _dtype_code(q), float(scale), int(bool(causal)),
                                     lse.data_ptr() if lse is not None else None, _stream_handle(q.device))
    else:
        ws, nbytes = _split_workspace(lib, H_q * T, d, q, num_splits)
        st = lib.sqa_attn_fwd_varlen_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                           cu_seqlens.data_ptr(), B, H_q, k.shape[0], T, int(max_seqlen), d,
                                           _dtype_code(q), float(scale), int(bool(causal)),
                                           lse.data_ptr() if lse is not None else None, int(num_splits),
                                           ws, nbytes, _stream_handle(q.device))
    _check(st)
    return (out, lse) if return_lse else out


def sqa_attn_bwd_workspace_bytes(B: int, H_q: int, N: int, d: int, dtype: str = "bf16") -> int:
    code = SQA_BF16 if dtype == "bf16" else SQA_F32
    return int(load_library().sqa_attn_bwd_workspace_bytes(B, H_q, N, d, code))


def sqa_attn_bwd(q, k, v, o, dout, lse, *, scale: Optional[float] = None, causal: bool = False,
                 dq=None, dk=None, dv=None, workspace=None, num_splits: Optional[int] = None):
    """Gradients of ``sqa_attn_fwd`` for the upstream gradient ``dout``.

    q, o, dout [B, H_q, N, d]; k, v [B, H_kv, N, d] bf16 (d = 64 or 128); lse
    [B, H_q, N] fp32 from ``sqa_attn_fwd(..., return_lse=True)`` with the same
    scale and causal flag. Returns (dq, dk, dv); dk and dv sum over the query
    heads of each K/V head's group. ``workspace`` is an optional uint8 GPU
    tensor of at least ``sqa_attn_bwd_split_workspace_bytes`` bytes for the
    split count used. ``num_splits``: range splits (encoder-style only; None:
    the library's choice, sqa_attn_bwd_num_splits, reduced to 1 if a given
    workspace is too small for it).
    """
    torch = _torch()
    lib = load_library()
    _require_device(q, k, v, o, dout, lse)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected 4-D [B, H, N, d] tensors")
    if k.shape != v.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("k/v and q/o/dout shapes must match")
    if len({q.dtype, k.dtype, v.dtype, o.dtype, dout.dtype}) != 1:
        raise ValueError("q, k, v, o and dout must share a dtype")
    if lse.dtype != torch.float32:
        raise ValueError("lse must be float32")
    B, H_q, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d or tuple(lse.shape) != (B, H_q, N):
        raise ValueError("q, k/v and lse shapes disagree")
    H_kv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    outs = []
    for t, like in ((dq, q), (dk, k), (dv, v)):
        if t is None:
            t = torch.empty_like(like)
        else:
            _require_device(t)
            if t.shape != like.shape or t.dtype != like.dtype:
                raise ValueError("gradient outputs must match their inputs in shape and dtype")
        outs.append(t)
    code = _dtype_code(q)
    need_of = lambda ns: int(lib.sqa_attn_bwd_split_workspace_bytes(B, H_q, H_kv, N, d, code, ns))
    num_splits = _bwd_splits(lib, num_splits, workspace, need_of,
                             lambda: lib.sqa_attn_bwd_num_splits(B, H_q, H_kv, N, d, code, int(bool(causal)), 0))
    if workspace is None:
        workspace = torch.empty(max(need_of(num_splits), 1), dtype=torch.uint8, device=q.device)
    else:
        _require_device(workspace)
    st = lib.sqa_attn_bwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                lse.data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
                                B, H_q, H_kv, N, d, code, float(scale), int(bool(causal)), int(num_splits),
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                _stream_handle(q.device))
    _check(st)
    return outs[0], outs[1], outs[2]


def sqa_attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, *, scale: Optional[float] = None,
                         causal: bool = False) -> None:
    """``sqa_attn_bwd`` into caller-provided dq, dk, dv with no allocation at
    all (no workspace: the library's fixed per-GPU buffer holds the row
    terms), for code under graph capture or loops that may not allocate.
    Same results as ``sqa_attn_bwd``; raises SQAError (SQA_ERR_WORKSPACE)
    for problems whose row terms exceed that buffer. Calls that overlap on
    one GPU share the buffer and race."""
    lib = load_library()
    _require_device(q, k, v, o, dout, lse, dq, dk, dv)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected 4-D [B, H, N, d] tensors")
    if k.shape != v.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("k/v and q/o/dout shapes must match")
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("dq, dk and dv must match q, k and v in shape")
    if len({q.dtype, k.dtype, v.dtype, o.dtype, dout.dtype, dq.dtype, dk.dtype, dv.dtype}) != 1:
        raise ValueError("q, k, v, o, dout and the gradients must share a dtype")
    B, H_q, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d or tuple(lse.shape) != (B, H_q, N):
        raise ValueError("q, k/v and lse shapes disagree")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.sqa_attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                  lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                  B, H_q, k.shape[1], N, d, _dtype_code(q), float(scale), int(bool(causal)),
                                  _stream_handle(q.device))
    _check(st)


def _bwd_splits(lib, num_splits, workspace, need_of, auto) -> int:
    """Range splits of a backward call: the requested count, or the library's
    choice, reduced to 1 when the caller's workspace is too small for it."""
    if num_splits is not None:
        return int(num_splits)
    ns = int(auto())
    if ns > 1 and workspace is not None and workspace.numel() * workspace.element_size() < need_of(ns):
        ns = 1
    return ns


def sqa_attn_bwd_num_splits(B: int, H_q: int, H_kv: int, N: int, d: int, dtype: str = "bf16",
                            causal: bool = False, T: int = 0) -> int:
    """The library's recommended range splits of the backward (packed batch: T tokens, N = max_seqlen)."""
    code = SQA_BF16 if dtype == "bf16" else SQA_F32
    return int(load_library().sqa_attn_bwd_num_splits(B, H_q, H_kv, N, d, code, int(bool(causal)), T))


def sqa_attn_bwd_split_workspace_bytes(B: int, H_q: int, H_kv: int, N: int, d: int, num_splits: int,
                                       dtype: str = "bf16") -> int:
    code = SQA_BF16 if dtype == "bf16" else SQA_F32
    return int(load_library().sqa_attn_bwd_split_workspace_bytes(B, H_q, H_kv, N, d, code, num_splits))


def sqa_attn_bwd_varlen_split_workspace_bytes(B: int, H_q: int, H_kv: int, T: int, d: int, num_splits: int,
                                              dtype: str = "bf16") -> int:
    code = SQA_BF16 if dtype == "bf16" else SQA_F32
    return int(load_library().sqa_attn_bwd_varlen_split_workspace_bytes(B, H_q, H_kv, T, d, code, num_splits))


def sqa_attn_bwd_varlen_workspace_bytes(B: int, H_q: int, T: int, d: int, dtype: str = "bf16") -> int:
    code = SQA_BF16 if dtype == "bf16" else SQA_F32
    return int(load_library().sqa_attn_bwd_varlen_workspace_bytes(B, H_q, T, d, code))


def sqa_attn_bwd_varlen(q, k, v, o, dout, lse, cu_seqlens, max_seqlen: Optional[int] = None, *,
                        scale: Optional[float] = None, causal: bool = False, dq=None, dk=None, dv=None,
                        workspace=None, num_splits: Optional[int] = None):
    """Gradients of ``sqa_attn_fwd_varlen`` for the upstream gradient ``dout``.

    q, o, dout [H_q, T, d]; k, v [H_kv, T, d] bf16 (d = 64 or 128); lse [H_q, T] fp32
    from ``sqa_attn_fwd_varlen(..., return_lse=True)``; cu_seqlens the same
    int32 GPU offsets. Returns (dq, dk, dv). ``max_seqlen`` as in the forward;
    ``workspace`` and ``num_splits`` as in ``sqa_attn_bwd`` (the split choice
    is made for the longest sequence).
    """
    torch = _torch()
    lib = load_library()
    _require_device(q, k, v, o, dout, lse, cu_seqlens)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("expected 3-D [H, T, d] tensors")
    if k.shape != v.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("k/v and q/o/dout shapes must match")
    if len({q.dtype, k.dtype, v.dtype, o.dtype, dout.dtype}) != 1:
        raise ValueError("q, k, v, o and dout must share a dtype")
    if lse.dtype != torch.float32:
        raise ValueError("lse must be float32")
    H_q, T, d = q.shape
    if k.shape[1] != T or k.shape[2] != d or tuple(lse.shape) != (H_q, T):
        raise ValueError("q, k/v and lse shapes disagree")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of B + 1 offsets")
    B = cu_seqlens.numel() - 1
    if max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if B > 0 else 0
    H_kv = k.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    outs = []
    for t, like in ((dq, q), (dk, k), (dv, v)):
        if t is None:
            t = torch.empty_like(like)
        else:
            _require_device(t)
            if t.shape != like.shape or t.dtype != like.dtype:
                raise ValueError("gradient outputs must match their inputs in shape and dtype")
        outs.append(t)
    code = _dtype_code(q)
    need_of = lambda ns: int(lib.sqa_attn_bwd_varlen_split_workspace_bytes(B, H_q, H_kv, T, d, code, ns))
    num_splits = _bwd_splits(lib, num_splits, workspace, need_of,
                             lambda: lib.sqa_attn_bwd_num_splits(B, H_q, H_kv, int(max_seqlen), d, code,
                                                                 int(bool(causal)), T))
    if workspace is None:
        workspace = torch.empty(max(need_of(num_splits), 1), dtype=torch.uint8, device=q.device)
    else:
        _require_device(workspace)
    st = lib.sqa_attn_bwd_varlen_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                       lse.data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
                                       cu_seqlens.data_ptr(), B, H_q, H_kv, T, int(max_seqlen), d, code,
                                       float(scale), int(bool(causal)), int(num_splits), workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(), _stream_handle(q.device))
    _check(st)
    return outs[0], outs[1], outs[2]


def sqa_layer_workspace_bytes(B: int, N: int, D: int, H: int, H_q: int, H_kv: int,
                              dtype: str = "bf16") -> int:
    code = SQA_BF16 if dtype == "bf16" else SQA_F32
    return int(load_library().sqa_layer_workspace_bytes(B, N, D, H, H_q, H_kv, code))


def sqa_layer_fwd(x, w_q, w_k, w_v, w_o, *, H: int, H_q: int, H_kv: int,
                  rope_base: float = 10000.0, scale: Optional[float] = None,
                  causal: bool = True, out=None, workspace=None):
    """One SQA attention layer forward: projections, RoPE, SQA, output projection.

    x [B, N, D] bf16; w_q [D, H_q*d], w_k/w_v [D, H_kv*d], w_o [H_q*d, D]
    bf16 in [in, out] layout, d = D // H. Returns y [B, N, D] bf16.
    ``workspace`` is an optional uint8 GPU tensor of at least
    ``sqa_layer_workspace_bytes`` bytes (allocated here if omitted).
    """
    torch = _torch()
    lib = load_library()
    _require_device(x, w_q, w_k, w_v, w_o)
    if x.dim() != 3:
        raise ValueError("x must be [B, N, D]")
    B, N, D = x.shape
    d = D // H if H else 0
    if scale is None:
        scale = 1.0 / math.sqrt(d) if d > 0 else 1.0
    if out is None:
        out = torch.empty_like(x)
    else:
        _require_device(out)
    need = int(lib.sqa_layer_workspace_bytes(B, N, D, H, H_q, H_kv, _dtype_code(x)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    else:
        _require_device(workspace)
    st = lib.sqa_layer_fwd(x.data_ptr(), w_q.data_ptr(), w_k.data_ptr(), w_v.data_ptr(),
                           w_o.data_ptr(), out.data_ptr(), B, N, D, H, H_q, H_kv,
                           float(rope_base), float(scale), int(bool(causal)), _dtype_code(x),
                           workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                           _stream_handle(x.device))
    _check(st)
    return out


def sqa_block_workspace_bytes(B: int, N: int, D: int, H: int, H_q: int, H_kv: int, F: int,
                              dtype: str = "bf16") -> int:
    code = SQA_BF16 if dtype == "bf16" else SQA_F32
    return int(load_library().sqa_block_workspace_bytes(B, N, D, H, H_q, H_kv, F, code))


def sqa_block_fwd(x, norm1, w_q, w_k, w_v, w_o, norm2, w_gate, w_up, w_down, *, H: int, H_q: int,
                  H_kv: int, rope_base: float = 10000.0, scale: Optional[float] = None,
                  eps: float = 1e-6, causal: bool = True, out=None, workspace=None):
    """One pre-norm transformer block: h = x + layer(rms_norm(x)); y = h + SwiGLU(rms_norm(h)).

    x [B, N, D] bf16; norm1/norm2 [D]; attention weights as ``sqa_layer_fwd``;
    w_gate, w_up [D, F], w_down [F, D]; all bf16. Returns y [B, N, D].
    """
    torch = _torch()
    lib = load_library()
    _require_device(x, norm1, w_q, w_k, w_v, w_o, norm2, w_gate, w_up, w_down)
    if x.dim() != 3 or w_gate.dim() != 2:
        raise ValueError("x must be [B, N, D] and w_gate [D, F]")
    B, N, D = x.shape
    F = w_gate.shape[1]
    d = D // H if H else 0
    if scale is None:
        scale = 1.0 / math.sqrt(d) if d > 0 else 1.0
    if out is None:
        out = torch.empty_like(x)
    else:
        _require_device(out)
    code = _dtype_code(x)
    need = int(lib.sqa_block_workspace_bytes(B, N, D, H, H_q, H_kv, F, code))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    else:
        _require_device(workspace)
    st = lib.sqa_block_fwd(x.data_ptr(), norm1.data_ptr(), w_q.data_ptr(), w_k.data_ptr(),
                           w_v.data_ptr(), w_o.data_ptr(), norm2.data_ptr(), w_gate.data_ptr(),
                           w_up.data_ptr(), w_down.data_ptr(), out.data_ptr(), B, N, D, H, H_q, H_kv,
                           F, float(rope_base), float(scale), float(eps), int(bool(causal)), code,
                           workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                           _stream_handle(x.device))
    _check(st)
    return out
