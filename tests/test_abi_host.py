"""Host-side checks of the C-ABI library: it loads without a GPU, exports every
symbol include/sqa.h declares, and rejects invalid arguments before any HIP
call (no compute is launched here)."""
import ctypes
import os
import re

import pytest

import sparse_query_attention_sqa_amd as sqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sqa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(sqa_[a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sqa.lib_path()):
        pytest.fail("libsqa.so is not built; run __graft_entry__.build()")
    return sqa.load_library()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ["sqa_attn_fwd", "sqa_attn_fwd_varlen", "sqa_layer_fwd", "sqa_layer_workspace_bytes",
              "sqa_status_str", "sqa_last_error", "sqa_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(sqa.lib_path())
    for name in _declared_functions():
        assert hasattr(raw, name), name


def test_version_and_status_strings(lib):
    assert lib.sqa_version() >= 100
    for code, name in [(0, "SQA_OK"), (1, "SQA_ERR_NULL"), (2, "SQA_ERR_SHAPE"),
                       (3, "SQA_ERR_UNSUPPORTED"), (4, "SQA_ERR_ALIGN"),
                       (5, "SQA_ERR_WORKSPACE"), (6, "SQA_ERR_HIP"), (7, "SQA_ERR_ARG")]:
        assert sqa.sqa_status_str(code) == name
    assert sqa.sqa_status_str(99) == "SQA_ERR_UNKNOWN"


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation


def _no_gpu_present():
    """Fake-pointer calls run only where no GPU exists, so that a validation
    bug can never turn into a launch on real hardware (device_count does not
    initialise the HIP runtime)."""
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


cpu_only = pytest.mark.skipif(not _no_gpu_present(),
                              reason="fake-pointer validation tests run on GPU-less hosts only")


def _attn(lib, q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000, B=1, Hq=8,
          Hkv=4, N=1024, d=64, dtype=1, scale=0.125, causal=0, lse=None):
    return lib.sqa_attn_fwd(q, k, v, o, B, Hq, Hkv, N, d, dtype, scale, causal, lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(o=None), 1),
    (dict(Hkv=9), 2), (dict(Hkv=0), 2), (dict(Hkv=16), 2), (dict(Hq=0), 2), (dict(N=-1), 2),
    (dict(B=-2), 2), (dict(N=1 << 31), 2),
    (dict(d=48), 3), (dict(d=256), 3), (dict(d=8), 3), (dict(dtype=5), 3),
    (dict(q=FAKE + 2), 4), (dict(o=FAKE + 0x300008), 4),
    (dict(scale=float("inf")), 7), (dict(scale=float("nan")), 7), (dict(causal=2), 7),
    (dict(o=FAKE), 7),                               # o aliases q
    (dict(lse=FAKE + 0x200000 + 64), 7),             # lse inside v
    (dict(lse=FAKE + 0x400001), 4),
])
@cpu_only
def test_attn_rejects_invalid_arguments(lib, kw, code):
    assert _attn(lib, **kw) == code
    assert lib.sqa_last_error().decode() != ""


@cpu_only
def test_zero_size_is_a_noop(lib):
    assert _attn(lib, q=None, k=None, v=None, o=None, B=0) == 0
    assert _attn(lib, q=None, k=None, v=None, o=None, N=0) == 0
    assert lib.sqa_last_error().decode() == ""


def _varlen(lib, q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000, cu=FAKE + 0x400000,
            B=4, Hq=8, Hkv=4, T=4096, maxlen=2048, d=64, dtype=1, scale=0.125, causal=1, lse=None):
    return lib.sqa_attn_fwd_varlen(q, k, v, o, cu, B, Hq, Hkv, T, maxlen, d, dtype, scale, causal, lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(cu=None), 1), (dict(o=None), 1),
    (dict(B=-1), 2), (dict(T=-1), 2), (dict(maxlen=-1), 2), (dict(maxlen=5000), 2),
    (dict(Hkv=9), 2), (dict(Hkv=0), 2), (dict(maxlen=1 << 31, T=1 << 31), 2),
    (dict(d=48), 3), (dict(dtype=7), 3),
    (dict(q=FAKE + 8), 4), (dict(cu=FAKE + 0x400002), 4), (dict(lse=FAKE + 0x500002), 4),
    (dict(scale=float("inf")), 7), (dict(causal=3), 7),
    (dict(o=FAKE + 0x200000), 7),                    # o aliases v
    (dict(o=FAKE + 0x400000 - 0x80000), 7),          # o overlaps inputs and cu_seqlens
    (dict(lse=FAKE + 0x400000), 7),                  # lse aliases cu_seqlens
])
@cpu_only
def test_varlen_rejects_invalid_arguments(lib, kw, code):
    assert _varlen(lib, **kw) == code
    assert lib.sqa_last_error().decode() != ""


@cpu_only
def test_varlen_empty_is_a_noop(lib):
    assert _varlen(lib, q=None, k=None, v=None, o=None, cu=None, B=0) == 0
    assert _varlen(lib, q=None, k=None, v=None, o=None, cu=None, T=0, maxlen=0) == 0
    assert _varlen(lib, q=None, k=None, v=None, o=None, cu=None, maxlen=0) == 0
    assert lib.sqa_last_error().decode() == ""


def _split(lib, q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000, B=1, Hq=8, Hkv=4, N=1024,
           d=64, dtype=1, scale=0.125, causal=0, lse=None, ns=2, ws=FAKE + 0x1000000, ws_bytes=1 << 24):
    return lib.sqa_attn_fwd_split(q, k, v, o, B, Hq, Hkv, N, d, dtype, scale, causal, lse, ns, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(ns=0), 7), (dict(ns=17), 7), (dict(ns=-1), 7),
    (dict(dtype=0), 3),
    (dict(ws=None), 5), (dict(ws_bytes=100), 5),
    (dict(ws=FAKE + 0x1000008), 4),
    (dict(ws=FAKE + 0x200000), 7),                   # workspace over v
    (dict(q=None), 1), (dict(Hkv=3, Hq=2), 2),
])
@cpu_only
def test_split_rejects_invalid_arguments(lib, kw, code):
    assert _split(lib, **kw) == code
    assert lib.sqa_last_error().decode() != ""


@cpu_only
def test_split_varlen_rejects_invalid_arguments(lib):
    f = lib.sqa_attn_fwd_varlen_split
    M = 0x1000000  # 16 MiB apart: the fake tensors (4 MiB each) do not overlap
    base = [FAKE, FAKE + M, FAKE + 2 * M, FAKE + 3 * M, FAKE + 4 * M, 4, 8, 4, 4096, 2048, 64, 1, 0.125, 1, None]
    assert f(*base, 2, None, 0, None) == 5
    assert f(*base, 2, FAKE + 5 * M, 1000, None) == 5               # too small
    big = 1 << 26  # > 2 x 32768 rows x 66 x 4 B
    assert f(*base, 2, FAKE + 4 * M, big, None) == 7                # workspace over cu_seqlens
    assert f(*base, 2, FAKE + 3 * M, big, None) == 7                # workspace over o
    assert f(*base, 20, FAKE + 5 * M, big, None) == 7
    assert f(*(base[:11] + [0] + base[12:]), 2, FAKE + 5 * M, big, None) == 3   # fp32
    assert f(*(base[:5] + [0] + base[6:]), 2, None, 0, None) == 0  # B = 0: nothing to do


@cpu_only
def test_split_one_needs_no_workspace(lib):
    # num_splits = 1 is the unsplit call: the workspace is not checked, so only
    # the fake tensors' validation remains (q = NULL -> SQA_ERR_NULL)
    assert _split(lib, q=None, ns=1, ws=None, ws_bytes=0) == 1


def test_split_workspace_bytes(lib):
    f = lib.sqa_attn_fwd_split_workspace_bytes
    # 3 ranges x 100 rows x (64 + 2) fp32 = 79200 B, rounded up to 256
    assert f(100, 64, 1, 3) == 79360
    assert f(8 * 32768, 64, 1, 3) == 3 * 8 * 32768 * 66 * 4
    assert f(100, 64, 1, 1) == 0
    # d = 16: 2 x 100 x (16 + 2) x 4 = 14400 B -> 14592
    assert f(100, 16, 1, 2) == 14592
    assert f(100, 128, 1, 2) == round(2 * 100 * 130 * 4 / 256 + 0.4999) * 256
    assert f(100, 64, 0, 2) == 0
    assert f(0, 64, 1, 2) == 0
    assert f(100, 64, 1, 17) == 0


def test_split_policy(lib):
    """The library's split choice (round model; 256 CUs on MI355X and as the
    fallback without a device)."""
    f = sqa.sqa_attn_fwd_num_splits
    # 1024 workgroups = exactly two rounds of 512: no split (the 32k headline)
    assert f(1, 8, 4, 32768, 64) == 1
    assert f(1, 16, 16, 32768, 64) == 1
    assert f(1, 4, 4, 131072, 64, causal=True) == 1
    # packed 32k batch whose longest sequence has 18496 tokens: its 580
    # workgroups fill 1.13 rounds -> two ranges; at (16,16) 1168 fill 2.28
    # rounds and the other sequences fill the tail -> none
    assert f(8, 8, 4, 18496, 64, T=32768) == 2
    assert f(8, 16, 16, 18496, 64, T=32768) == 1
    # ... but not when the longest holds under a quarter of the tokens, or is short
    assert f(64, 8, 4, 8000, 64, T=65536) == 1
    assert f(8, 8, 4, 2000, 64, T=4000) == 1
    # one dense 18496-token sequence: 580 workgroups, 1.13 rounds -> 1.5
    assert f(1, 8, 4, 18496, 64) == 2
    # (6,4): 768 workgroups, 1.5 rounds -> 1.5 rounds of half-length ones
    assert f(1, 6, 4, 32768, 64) == 2
    # never under a causal mask
    assert f(1, 8, 4, 18496, 64, causal=True) == 1
    assert f(8, 8, 4, 18496, 64, causal=True, T=32768) == 1
    assert f(1, 8, 4, 4096, 64, causal=True) == 1
    # a quarter of a round fills the chip with four ranges; half a round with two
    assert f(1, 8, 4, 4096, 64) == 4
    assert f(2, 8, 4, 4096, 64) == 2
    # ranges keep at least 1024 keys: a 1000-key sequence is not split
    assert f(1, 8, 4, 1000, 64) == 1
    # the library's choice: d = 64 only (d = 128 packed measured slower split)
    assert f(1, 8, 4, 18496, 128) == 1
    assert f(8, 8, 4, 18496, 128, T=32768) == 1
    assert f(1, 8, 4, 18496, 32) == 1
    assert f(1, 8, 4, 18496, 64, dtype="f32") == 1
    assert f(0, 8, 4, 18496, 64) == 1 and f(1, 4, 8, 18496, 64) == 1


def test_bwd_split_workspace_and_policy(lib):
    f = lib.sqa_attn_bwd_split_workspace_bytes
    rt = lib.sqa_attn_bwd_workspace_bytes(1, 8, 1000, 64, 1)
    assert f(1, 8, 4, 1000, 64, 1, 1) == rt
    # 2 ranges x (8000 dQ rows + 2 x 4000 dK/dV rows) x 64 fp32
    assert f(1, 8, 4, 1000, 64, 1, 2) == rt + 2 * 16000 * 64 * 4
    assert f(1, 8, 4, 1000, 64, 1, 0) == 0 and f(1, 8, 4, 1000, 64, 1, 17) == 0
    assert f(1, 4, 8, 1000, 64, 1, 2) == 0 and f(1, 8, 4, 1000, 32, 1, 2) == 0
    g = lib.sqa_attn_bwd_varlen_split_workspace_bytes
    assert g(3, 8, 4, 5000, 64, 1, 1) == lib.sqa_attn_bwd_varlen_workspace_bytes(3, 8, 5000, 64, 1)
    assert g(3, 8, 4, 5000, 64, 1, 3) == g(3, 8, 4, 5000, 64, 1, 1) + 3 * (40000 + 40000) * 64 * 4
    n = sqa.sqa_attn_bwd_num_splits
    assert n(1, 8, 4, 32768, 64) == 1                  # 1024 / 512 dK/dV workgroups per slot: whole rounds
    assert n(1, 8, 4, 18496, 64) == 2                  # 580 dK/dV workgroups: 1.13 rounds
    assert n(8, 8, 4, 18496, 64, T=32768) == 2         # packed: 580 dK/dV workgroups of the longest, 1.13 rounds
    assert n(8, 16, 16, 18496, 64, T=32768) == 1       # 2320 of them, 4.5 rounds: the others fill the tail
    assert n(1, 8, 4, 18496, 64, causal=True) == 1     # never under a causal mask
    assert n(1, 8, 4, 18496, 32) == 1 and n(1, 8, 4, 1000, 64) == 1


@cpu_only
def test_bwd_split_rejects_invalid_arguments(lib):
    M = 0x1000000
    args = [FAKE + i * M for i in range(9)] + [1, 8, 4, 1000, 64, 1, 0.125, 0]
    f = lib.sqa_attn_bwd_split
    assert f(*args, 0, FAKE + 9 * M, 1 << 24, None) == 7
    assert f(*args, 17, FAKE + 9 * M, 1 << 24, None) == 7
    assert f(*(args[:-1] + [1]), 2, FAKE + 9 * M, 1 << 24, None) == 3   # causal
    assert f(*args, 2, FAKE + 9 * M, 1000, None) == 5                   # too small for the partials
    assert f(*args, 2, FAKE + 9 * M + 8, 1 << 24, None) == 4


def test_layer_workspace_bytes(lib):
    # SQAT-m layer: B=16 N=1024 D=256 H=16 (8,4): Q and O 4 MiB each, K and V
    # 2 MiB each
    assert sqa.sqa_layer_workspace_bytes(16, 1024, 256, 16, 8, 4) == 2 * 4194304 + 2 * 2097152
    # B=1 N=3: Q 768 B, K 384 B -> rounded to 768 and 512
    assert sqa.sqa_layer_workspace_bytes(1, 3, 256, 16, 8, 4) == 2 * 768 + 2 * 512
    assert sqa.sqa_layer_workspace_bytes(0, 1024, 256, 16, 8, 4) == 0
    assert sqa.sqa_layer_workspace_bytes(1, 1024, 256, 16, 8, 4, dtype="f32") == 0


def _layer(lib, x=FAKE, ws=FAKE + 0x1000000, ws_bytes=1 << 26, B=16, N=1024, D=256, H=16, Hq=8,
           Hkv=4, dtype=1, base=10000.0, causal=1):
    return lib.sqa_layer_fwd(x, FAKE + 0x100000, FAKE + 0x110000, FAKE + 0x120000,
                             FAKE + 0x130000, FAKE + 0x200000 if x else FAKE + 0x200000,
                             B, N, D, H, Hq, Hkv, base, 0.25, causal, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(ws=None), 5), (dict(ws_bytes=100), 5), (dict(dtype=0), 3),
    (dict(D=250), 2), (dict(H=0), 2), (dict(Hkv=9), 2), (dict(D=512, H=16), 3),
    (dict(D=512, H=4), 3),                           # d = 128: not a layer head dim
    (dict(base=0.0), 7), (dict(base=float("nan")), 7), (dict(ws=FAKE + 0x1000010), 4),
])
@cpu_only
def test_layer_rejects_invalid_arguments(lib, kw, code):
    assert _layer(lib, **kw) == code


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 2, 8, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sqa.sqa_attn_fwd(q, q[:, :1].contiguous(), q[:, :1].contiguous())


# ------------------------------------------------------------------ backward
def test_header_declares_the_backward():
    names = _declared_functions()
    assert "sqa_attn_bwd" in names and "sqa_attn_bwd_workspace_bytes" in names


def test_bwd_workspace_bytes(lib):
    # one (lse*log2 e, D) fp32 pair per query row, rows padded to a multiple of 32
    assert sqa.sqa_attn_bwd_workspace_bytes(1, 8, 32768, 64) == 8 * 32768 * 8
    # N = 33 pads to 64 rows: 2*3*64*8 = 3072 B
    assert sqa.sqa_attn_bwd_workspace_bytes(2, 3, 33, 64) == 3072
    # N = 1 pads to 32 rows: 32*8 = 256 B
    assert sqa.sqa_attn_bwd_workspace_bytes(1, 1, 1, 64) == 256
    assert sqa.sqa_attn_bwd_workspace_bytes(0, 8, 1024, 64) == 0
    assert sqa.sqa_attn_bwd_workspace_bytes(1, 8, 1024, 16) == 0
    assert sqa.sqa_attn_bwd_workspace_bytes(1, 8, 1024, 128) == 8 * 1024 * 8
    assert sqa.sqa_attn_bwd_workspace_bytes(1, 8, 1024, 64, dtype="f32") == 0


def _bwd(lib, q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000,
         do=FAKE + 0x400000, lse=FAKE + 0x500000, dq=FAKE + 0x600000, dk=FAKE + 0x700000,
         dv=FAKE + 0x800000, B=1, Hq=8, Hkv=4, N=1024, d=64, dtype=1, scale=0.125, causal=0,
         ws=FAKE + 0x900000, ws_bytes=1 << 20):
    return lib.sqa_attn_bwd(q, k, v, o, do, lse, dq, dk, dv, B, Hq, Hkv, N, d, dtype, scale,
                            causal, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(lse=None), 1), (dict(dv=None), 1),
    (dict(Hkv=9), 2), (dict(N=-1), 2),
    (dict(d=16), 3), (dict(dtype=0), 3), (dict(d=256), 3), (dict(d=32), 3),
    (dict(do=FAKE + 0x400008), 4), (dict(lse=FAKE + 0x500002), 4), (dict(ws=FAKE + 0x900008), 4),
    (dict(ws=None), 5), (dict(ws_bytes=65535), 5),
    (dict(scale=float("nan")), 7), (dict(causal=-1), 7),
    (dict(dq=FAKE + 0x300000), 7),                   # dq aliases o
    (dict(dk=FAKE + 0x600000 + 4096), 7),            # dk inside dq
    (dict(ws=FAKE + 0x800000), 7),                   # workspace aliases dv
])
@cpu_only
def test_bwd_rejects_invalid_arguments(lib, kw, code):
    assert _bwd(lib, **kw) == code
    assert lib.sqa_last_error().decode() != ""


@cpu_only
def test_bwd_zero_size_is_a_noop(lib):
    assert _bwd(lib, q=None, B=0, ws=None) == 0
    assert _bwd(lib, N=0, ws=None) == 0


def _bwd_noalloc(lib, q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000,
                 do=FAKE + 0x400000, lse=FAKE + 0x500000, dq=FAKE + 0x600000, dk=FAKE + 0x700000,
                 dv=FAKE + 0x800000, B=1, Hq=8, Hkv=4, N=1024, d=64, dtype=1, scale=0.125, causal=0):
    return lib.sqa_attn_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, B, Hq, Hkv, N, d, dtype, scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(Hkv=9), 2), (dict(d=16), 3), (dict(lse=FAKE + 0x500002), 4),
    (dict(scale=float("inf")), 7), (dict(dq=FAKE + 0x300000), 7),
])
@cpu_only
def test_bwd_noalloc_rejects_invalid_arguments(lib, kw, code):
    # every check runs before the buffer lookup, so no HIP call is made
    assert _bwd_noalloc(lib, **kw) == code
    assert lib.sqa_last_error().decode() != ""


@cpu_only
def test_bwd_noalloc_rejects_problems_over_its_buffer(lib):
    # 32 query heads x 262144 rows x 8 B = 64 MiB of row terms > the 32 MiB
    # buffer (16 heads x 262144 rows is exactly 32 MiB: accepted by the size
    # rule, so it is not called here, where there is no device)
    g = 1 << 32  # tensors of up to 1 GiB each, spaced apart so none overlap
    ptrs = dict(q=FAKE, k=FAKE + g, v=FAKE + 2 * g, o=FAKE + 3 * g, do=FAKE + 4 * g, lse=FAKE + 5 * g,
                dq=FAKE + 6 * g, dk=FAKE + 7 * g, dv=FAKE + 8 * g)
    assert sqa.sqa_attn_bwd_workspace_bytes(1, 16, 262144, 64) == 32 << 20
    assert _bwd_noalloc(lib, Hq=32, Hkv=8, N=262144, **ptrs) == 5
    assert "buffer" in lib.sqa_last_error().decode()
    assert _bwd_noalloc(lib, B=0, q=None) == 0     # empty problems return at once
    assert _bwd_noalloc(lib, N=0) == 0


def test_bwd_varlen_workspace_bytes(lib):
    # 8 B per (query head, packed row), plus 32 padding rows per head
    assert sqa.sqa_attn_bwd_varlen_workspace_bytes(3, 8, 1000, 64) == 8 * 8 * 1032
    assert sqa.sqa_attn_bwd_varlen_workspace_bytes(1, 1, 1, 64) == 512   # 33 rows x 8 B, rounded up
    assert sqa.sqa_attn_bwd_varlen_workspace_bytes(0, 8, 1000, 64) == 0
    assert sqa.sqa_attn_bwd_varlen_workspace_bytes(2, 8, 1000, 128) == 8 * 8 * 1032   # same for d = 128
    assert sqa.sqa_attn_bwd_varlen_workspace_bytes(2, 8, 1000, 32) == 0


def _bwd_varlen(lib, q=FAKE, cu=FAKE + 0xa00000, dq=FAKE + 0x600000, B=2, Hq=8, Hkv=4, T=1024, maxlen=600,
                d=64, dtype=1, ws=FAKE + 0x900000, ws_bytes=1 << 20):
    return lib.sqa_attn_bwd_varlen(q, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000,
                                   FAKE + 0x500000, dq, FAKE + 0x700000, FAKE + 0x800000, cu, B, Hq, Hkv, T,
                                   maxlen, d, dtype, 0.125, 1, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(cu=None), 1), (dict(dq=None), 1),
    (dict(B=-1), 2), (dict(maxlen=2000), 2), (dict(Hkv=9), 2),
    (dict(d=32), 3), (dict(dtype=0), 3),
    (dict(cu=FAKE + 0xa00002), 4), (dict(ws=FAKE + 0x900008), 4),
    (dict(ws=None), 5), (dict(ws_bytes=100), 5),
    (dict(dq=FAKE + 0x100000), 7),                   # dq overlaps k
    (dict(ws=FAKE + 0xa00000), 7),                   # workspace overlaps cu_seqlens
])
@cpu_only
def test_bwd_varlen_rejects_invalid_arguments(lib, kw, code):
    assert _bwd_varlen(lib, **kw) == code
    assert lib.sqa_last_error().decode() != ""


# ------------------------------------------------------------------ block
def test_block_workspace_bytes(lib):
    # SQAT-m block B=16 N=1024 D=256 (8,4) F=768: the layer's workspace plus the
    # normalised input and residual stream (8 MiB each) and the SwiGLU
    # activations (24 MiB)
    layer = 2 * 4194304 + 2 * 2097152
    assert sqa.sqa_block_workspace_bytes(16, 1024, 256, 16, 8, 4, 768) == layer + 2 * 8388608 + 25165824
    assert sqa.sqa_block_workspace_bytes(16, 1024, 256, 16, 8, 4, 0) == 0
    assert sqa.sqa_block_workspace_bytes(0, 1024, 256, 16, 8, 4, 768) == 0


def _block(lib, x=FAKE, ws=FAKE + 0x4000000, ws_bytes=1 << 27, B=16, N=1024, D=256, H=16, Hq=8,
           Hkv=4, F=768, eps=1e-6, dtype=1, g2=FAKE + 0x150000):
    return lib.sqa_block_fwd(x, FAKE + 0x140000, FAKE + 0x100000, FAKE + 0x110000,
                             FAKE + 0x120000, FAKE + 0x130000, g2, FAKE + 0x160000,
                             FAKE + 0x1a0000, FAKE + 0x1e0000, FAKE + 0x2000000, B, N, D, H, Hq,
                             Hkv, F, 10000.0, 0.25, eps, 1, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(g2=None), 1), (dict(ws=None), 5), (dict(ws_bytes=1 << 20), 5),
    (dict(F=0), 3), (dict(F=100), 3), (dict(dtype=0), 3), (dict(D=250), 2),
    (dict(eps=-1.0), 7), (dict(eps=float("nan")), 7), (dict(g2=FAKE + 0x150002), 4),
    (dict(ws=FAKE + 0x4000010), 4), (dict(ws=FAKE + 0x1e0000), 7),
])
@cpu_only
def test_block_rejects_invalid_arguments(lib, kw, code):
    assert _block(lib, **kw) == code


# ------------------------------------------------------ launch limits -> SHAPE
SPACING = 1 << 40  # fake tensors this far apart never overlap, whatever their size


def _spaced(n):
    return [FAKE + i * SPACING for i in range(n)]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dtype", [
    (1, 8, 4, 1 << 24, 64, 1),      # d = 64: N * 128 B reaches 2^31 (buffer descriptor range)
    (1, 8, 4, 1 << 23, 128, 1),     # d = 128: N * 256 B reaches 2^31
    (1 << 31, 1, 1, 1, 16, 1),      # B * H_kv reaches 2^31 (grid)
    (1 << 31, 1, 1, 1, 32, 1),
    (1 << 31, 2, 1, 1, 64, 1),
    (1 << 31, 1, 1, 1, 16, 0),      # fp32: workgroup count reaches 2^31
])
@cpu_only
def test_attn_launch_limits_are_shape_errors(lib, B, Hq, Hkv, N, d, dtype):
    q, k, v, o = _spaced(4)
    st = lib.sqa_attn_fwd(q, k, v, o, B, Hq, Hkv, N, d, dtype, 0.125, 0, None, None)
    msg = lib.sqa_last_error().decode()
    assert st == 2, (st, msg)
    assert "launch limit" in msg


@cpu_only
def test_varlen_launch_limit_is_a_shape_error(lib):
    q, k, v, o, cu = _spaced(5)
    st = lib.sqa_attn_fwd_varlen(q, k, v, o, cu, 1, 8, 4, 1 << 24, 1 << 24, 64, 1, 0.125, 0, None, None)
    assert st == 2 and "launch limit" in lib.sqa_last_error().decode()


@pytest.mark.parametrize("N,d", [(1 << 24, 64), (1 << 23, 128)])
@cpu_only
def test_bwd_launch_limits_are_shape_errors(lib, N, d):
    q, k, v, o, do, lse, dq, dk, dv, ws = _spaced(10)
    st = lib.sqa_attn_bwd(q, k, v, o, do, lse, dq, dk, dv, 1, 8, 4, N, d, 1, 0.125, 0, ws, 1 << 36, None)
    assert st == 2 and "launch limit" in lib.sqa_last_error().decode()
    st = lib.sqa_attn_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, 1, 1, 1, N, d, 1, 0.125, 0, None)
    # one query head: its row terms (N * 8 B, 64 or 128 MiB) exceed the
    # no-alloc buffer's 32 MiB, which is checked before the dry run
    assert st == 5


@cpu_only
def test_bwd_row_term_limit_is_a_shape_error(lib):
    # 64 query heads of 2^23 rows: within the per-head limit, but the row
    # terms (two planes of 4 bytes per row, one DMA spanning both) pass 2^31 bytes
    q, k, v, o, do, lse, dq, dk, dv, ws = _spaced(10)
    st = lib.sqa_attn_bwd(q, k, v, o, do, lse, dq, dk, dv, 1, 64, 64, 1 << 23, 64, 1, 0.125, 0, ws, 1 << 36, None)
    assert st == 2 and "launch limit" in lib.sqa_last_error().decode()


@cpu_only
def test_layer_launch_limit_is_a_shape_error(lib):
    # X [1, 2^22, 256] bf16 is 2^31 bytes: past the projections' 32-bit offsets
    x, wq, wk, wv, wo, y, ws = _spaced(7)
    st = lib.sqa_layer_fwd(x, wq, wk, wv, wo, y, 1, 1 << 22, 256, 16, 8, 4, 10000.0, 0.25, 1, 1, ws, 1 << 36,
                           None)
    assert st == 2 and "launch limit" in lib.sqa_last_error().decode()


# ------------------------------------------------------------- tail split
@cpu_only
def test_tail_plan_on_256_cus(lib):
    # without a device the plan assumes MI355X's 256 CUs: 512 slots
    assert sqa.sqa_attn_fwd_tail_splits(1, 4, 4, 200000, 64) == 9      # 3128 workgroups: 6 rounds + 56
    need = lib.sqa_attn_fwd_tail_workspace_bytes(1, 4, 4, 200000, 64, 1, 0)
    assert need == (9 * 56 * 256 * 66 * 4 + 255) // 256 * 256
    assert sqa.sqa_attn_fwd_tail_splits(1, 8, 4, 17900, 64) == 10      # 560 workgroups: 1 round + 48
    assert sqa.sqa_attn_fwd_tail_splits(1, 8, 4, 32768, 64) == 1       # 1024: whole rounds
    assert sqa.sqa_attn_fwd_tail_splits(1, 16, 16, 200000, 64) == 2    # 12512: 24 rounds + 224
    assert sqa.sqa_attn_fwd_tail_splits(1, 4, 4, 200000, 64, causal=True) == 1
    assert sqa.sqa_attn_fwd_tail_splits(1, 4, 4, 200000, 128) == 1
    assert sqa.sqa_attn_fwd_tail_splits(1, 6, 4, 200000, 64) == 1      # uneven groups
    assert sqa.sqa_attn_fwd_tail_splits(1, 4, 4, 1000, 64) == 1        # under one round
    assert lib.sqa_attn_fwd_tail_workspace_bytes(1, 8, 4, 32768, 64, 1, 0) == 0


@cpu_only
def test_tail_rejects_invalid_arguments(lib):
    q, k, v, o, ws = _spaced(5)
    f = lib.sqa_attn_fwd_tail
    assert f(q, k, v, o, 1, 4, 4, 200000, 64, 1, 0.125, 0, None, None, 0, None) == 5        # no workspace
    assert f(q, k, v, o, 1, 4, 4, 200000, 64, 1, 0.125, 0, None, ws, 1000, None) == 5       # too small
    assert f(q, k, v, o, 1, 4, 4, 200000, 64, 1, 0.125, 0, None, FAKE + 8, 1 << 30, None) == 4
    assert f(q, k, v, o, 1, 4, 4, 200000, 64, 1, 0.125, 0, None, k, 1 << 30, None) == 7     # overlaps k
    assert f(None, k, v, o, 1, 4, 4, 200000, 64, 1, 0.125, 0, None, ws, 1 << 30, None) == 1
    assert f(q, k, v, o, 1, 4, 0, 200000, 64, 1, 0.125, 0, None, ws, 1 << 30, None) == 2    # no plan: plain checks
    assert f(q, k, v, o, 1, 4, 4, 200000, 64, 1, float("nan"), 0, None, ws, 1 << 30, None) == 7
