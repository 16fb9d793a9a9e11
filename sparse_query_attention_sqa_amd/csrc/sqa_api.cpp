// C-ABI entry points of libsqa (declared and documented in include/sqa.h).
//
// Every argument is checked before anything is launched; on error nothing is
// enqueued and the outputs are untouched. The library holds no state besides
// a thread-local error string, never allocates device memory and never
// synchronises: all work goes onto the caller's stream.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <string>

#include "kernels.h"
#include "sqa.h"

namespace {

thread_local std::string g_err;

sqa_status fail(sqa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

sqa_status hip_fail(hipError_t e, const char* what) {
  return fail(SQA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A launcher's dry run failed: the sizes pass the argument rules but exceed
// a 32-bit limit of the kernels (grid size, offsets, buffer ranges).
sqa_status limit_fail(const char* what) {
  return fail(SQA_ERR_SHAPE, "%s: the sizes exceed a launch limit of the kernels (see include/sqa.h)", what);
}

// Dry-run the attention launch, then launch it.
sqa_status launch_attn(sqa::AttnProblem p, int dtype, hipStream_t st) {
  p.dry_run = true;
  hipError_t e = (dtype == SQA_BF16) ? sqa::launch_attn_fwd_bf16(p, st) : sqa::launch_attn_fwd_f32(p, st);
  if (e != hipSuccess) return limit_fail("attention");
  p.dry_run = false;
  e = (dtype == SQA_BF16) ? sqa::launch_attn_fwd_bf16(p, st) : sqa::launch_attn_fwd_f32(p, st);
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  return SQA_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

constexpr int64_t kMaxN = (int64_t(1) << 30);          // positions per sequence
constexpr int64_t kMaxElems = (int64_t(1) << 40);      // elements per tensor

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Product of non-negative factors <= lim, without overflowing int64_t.
bool prod_le(std::initializer_list<int64_t> factors, int64_t lim) {
  int64_t p = 1;
  for (const int64_t f : factors) {
    if (f < 0) return false;
    if (f == 0) return true;
    if (p > lim / f) return false;
    p *= f;
  }
  return p <= lim;
}

// Shape rules shared by the attention and layer entry points.
sqa_status check_heads(int64_t H_q, int64_t H_kv) {
  if (H_q < 1) return fail(SQA_ERR_SHAPE, "H_q must be >= 1 (got %lld)", (long long)H_q);
  if (H_kv < 1 || H_kv > H_q)
    return fail(SQA_ERR_SHAPE, "H_kv must be in [1, H_q] (got H_kv=%lld, H_q=%lld)", (long long)H_kv,
                (long long)H_q);
  if (H_q > 4096) return fail(SQA_ERR_SHAPE, "H_q too large (%lld)", (long long)H_q);
  return SQA_OK;
}

sqa_status check_attn(int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t d, int dtype,
                      float scale, int causal) {
  if (B < 0 || N < 0 || d < 0) return fail(SQA_ERR_SHAPE, "negative size");
  sqa_status s = check_heads(H_q, H_kv);
  if (s != SQA_OK) return s;
  if (dtype != SQA_F32 && dtype != SQA_BF16) return fail(SQA_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (d != 16 && d != 32 && d != 64 && d != 128)
    return fail(SQA_ERR_UNSUPPORTED, "head dim d=%lld not supported (16, 32, 64 or 128)", (long long)d);
  if (!std::isfinite(scale)) return fail(SQA_ERR_ARG, "scale must be finite");
  if (causal != 0 && causal != 1) return fail(SQA_ERR_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (N > kMaxN) return fail(SQA_ERR_SHAPE, "N=%lld exceeds the supported maximum", (long long)N);
  if (B > 0 && N > 0 && !prod_le({B, H_q, N, d}, kMaxElems))
    return fail(SQA_ERR_SHAPE, "tensor too large");
  return SQA_OK;
}

constexpr int64_t kMaxSplits = 16;

sqa_status check_splits(int64_t num_splits, int64_t d, int dtype) {
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(SQA_ERR_ARG, "num_splits must be in [1, %lld] (got %lld)", (long long)kMaxSplits,
                (long long)num_splits);
  if (num_splits > 1 && dtype != SQA_BF16) return fail(SQA_ERR_UNSUPPORTED, "key-range splits need bf16");
  return SQA_OK;
}

sqa_status check_bwd_splits(int64_t num_splits, int causal) {
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(SQA_ERR_ARG, "num_splits must be in [1, %lld] (got %lld)", (long long)kMaxSplits,
                (long long)num_splits);
  if (num_splits > 1 && causal) return fail(SQA_ERR_UNSUPPORTED, "range splits of the backward are encoder-style only");
  return SQA_OK;
}

// Workspace of a split forward: present, aligned, large enough and clear of
// every tensor argument (tensors[i] spans sizes[i] bytes).
sqa_status check_split_workspace(int64_t num_splits, int64_t rows, int64_t d, const void* ws, size_t ws_bytes,
                                 const void* const* tensors, const size_t* sizes) {
  if (num_splits <= 1) return SQA_OK;
  const size_t need = sqa::attn_split_workspace_bytes(rows, d, (int)num_splits);
  if (ws == nullptr || ws_bytes < need)
    return fail(SQA_ERR_WORKSPACE, "split workspace of %zu bytes needed (got %zu)", need, ws ? ws_bytes : (size_t)0);
  if (!aligned(ws, 16)) return fail(SQA_ERR_ALIGN, "workspace must be 16-byte aligned");
  for (int i = 0; i < 5; ++i)
    if (overlaps(ws, need, tensors[i], sizes[i])) return fail(SQA_ERR_ARG, "workspace overlaps a tensor");
  return SQA_OK;
}

}  // namespace

namespace sqa {

// Compute units of the current device (256, MI355X's count, if the query
// fails), cached per device ordinal; concurrent first calls store the same
// value.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace sqa

extern "C" {

sqa_status sqa_attn_fwd(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H_q,
                        int64_t H_kv, int64_t N, int64_t d, int dtype, float scale, int causal,
                        float* lse, void* stream) {
  return sqa_attn_fwd_split(q, k, v, o, B, H_q, H_kv, N, d, dtype, scale, causal, lse, 1, nullptr, 0, stream);
}

sqa_status sqa_attn_fwd_split(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H_q,
                              int64_t H_kv, int64_t N, int64_t d, int dtype, float scale, int causal, float* lse,
                              int64_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  sqa_status s = check_attn(B, H_q, H_kv, N, d, dtype, scale, causal);
  if (s != SQA_OK) return s;
  s = check_splits(num_splits, d, dtype);
  if (s != SQA_OK) return s;
  if (B == 0 || N == 0) return SQA_OK;
  if (!q || !k || !v || !o) return fail(SQA_ERR_NULL, "q, k, v and o must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(SQA_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(SQA_ERR_ALIGN, "lse must be 4-byte aligned");
  const size_t esz = dtype == SQA_BF16 ? 2 : 4;
  const size_t nq = (size_t)(B * H_q * N * d) * esz, nkv = (size_t)(B * H_kv * N * d) * esz;
  const size_t nl = lse ? (size_t)(B * H_q * N) * 4 : 0;
  if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv))
    return fail(SQA_ERR_ARG, "o overlaps an input");
  if (lse && (overlaps(lse, nl, o, nq) || overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) ||
              overlaps(lse, nl, v, nkv)))
    return fail(SQA_ERR_ARG, "lse overlaps another tensor");
  const void* tensors[5] = {q, k, v, o, lse};
  const size_t sizes[5] = {nq, nkv, nkv, nq, nl};
  s = check_split_workspace(num_splits, B * H_q * N, d, workspace, workspace_bytes, tensors, sizes);
  if (s != SQA_OK) return s;

  sqa::AttnProblem p{q, k, v, o, lse, B, H_q, H_kv, N, d, scale, causal};
  p.nsplit = (int)num_splits;
  p.split_ws = num_splits > 1 ? static_cast<float*>(workspace) : nullptr;
  return launch_attn(p, dtype, static_cast<hipStream_t>(stream));
}

sqa_status sqa_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens,
                               int64_t B, int64_t H_q, int64_t H_kv, int64_t T, int64_t max_seqlen, int64_t d,
                               int dtype, float scale, int causal, float* lse, void* stream) {
  return sqa_attn_fwd_varlen_split(q, k, v, o, cu_seqlens, B, H_q, H_kv, T, max_seqlen, d, dtype, scale, causal,
                                   lse, 1, nullptr, 0, stream);
}

sqa_status sqa_attn_fwd_varlen_split(const void* q, const void* k, const void* v, void* o,
                                     const int32_t* cu_seqlens, int64_t B, int64_t H_q, int64_t H_kv,
                                     int64_t T, int64_t max_seqlen, int64_t d, int dtype, float scale,
                                     int causal, float* lse, int64_t num_splits, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (B < 0 || T < 0 || max_seqlen < 0) return fail(SQA_ERR_SHAPE, "negative size");
  // shape rules of one sequence of the longest length; the total is checked below
  sqa_status s = check_attn(B > 0 ? 1 : 0, H_q, H_kv, max_seqlen, d, dtype, scale, causal);
  if (s != SQA_OK) return s;
  s = check_splits(num_splits, d, dtype);
  if (s != SQA_OK) return s;
  if (max_seqlen > T) return fail(SQA_ERR_SHAPE, "max_seqlen=%lld exceeds T=%lld", (long long)max_seqlen,
                                  (long long)T);
  if (!prod_le({T, H_q, d}, kMaxElems)) return fail(SQA_ERR_SHAPE, "tensor too large");
  if (B > 0x7fffffffLL) return fail(SQA_ERR_SHAPE, "too many sequences");
  if (B == 0 || T == 0 || max_seqlen == 0) return SQA_OK;
  if (!q || !k || !v || !o || !cu_seqlens) return fail(SQA_ERR_NULL, "q, k, v, o and cu_seqlens must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(SQA_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  if (!aligned(cu_seqlens, 4) || (lse && !aligned(lse, 4)))
    return fail(SQA_ERR_ALIGN, "cu_seqlens and lse must be 4-byte aligned");
  const size_t esz = dtype == SQA_BF16 ? 2 : 4;
  const size_t nq = (size_t)(H_q * T * d) * esz, nkv = (size_t)(H_kv * T * d) * esz;
  const size_t nl = lse ? (size_t)(H_q * T) * 4 : 0, ncu = (size_t)(B + 1) * 4;
  if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv) || overlaps(o, nq, cu_seqlens, ncu))
    return fail(SQA_ERR_ARG, "o overlaps an input");
  if (lse && (overlaps(lse, nl, o, nq) || overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) ||
              overlaps(lse, nl, v, nkv) || overlaps(lse, nl, cu_seqlens, ncu)))
    return fail(SQA_ERR_ARG, "lse overlaps another tensor");
  if (num_splits > 1 && overlaps(workspace, workspace_bytes, cu_seqlens, ncu))
    return fail(SQA_ERR_ARG, "workspace overlaps cu_seqlens");
  const void* tensors[5] = {q, k, v, o, lse};
  const size_t sizes[5] = {nq, nkv, nkv, nq, nl};
  s = check_split_workspace(num_splits, H_q * T, d, workspace, workspace_bytes, tensors, sizes);
  if (s != SQA_OK) return s;

  sqa::AttnProblem p{q, k, v, o, lse, B, H_q, H_kv, max_seqlen, d, scale, causal, cu_seqlens, T};
  p.nsplit = (int)num_splits;
  p.split_ws = num_splits > 1 ? static_cast<float*>(workspace) : nullptr;
  return launch_attn(p, dtype, static_cast<hipStream_t>(stream));
}

int64_t sqa_attn_fwd_num_splits(int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t d, int dtype,
                                int causal, int64_t T) {
  if (B <= 0 || N <= 0 || H_q < 1 || H_kv < 1 || H_kv > H_q || H_q > 4096 || N > kMaxN || T < 0) return 1;
  if (T > 0 && N > T) return 1;
  if (!prod_le({B, H_q, N, d > 0 ? d : 1}, kMaxElems) || !prod_le({T, H_q, d > 0 ? d : 1}, kMaxElems)) return 1;
  // d = 128: the packed 32k batch ran 903 TFLOP/s unsplit, 848 / 821 with 2 / 3
  // ranges (its 32-row waves already give the longest sequence 1156
  // workgroups); d = 16/32: slower under a causal mask. Splits there run on
  // request only.
  if (d != 64 || dtype != SQA_BF16) return 1;
  return sqa::attn_fwd_auto_splits(B, H_q, H_kv, N, T, causal != 0, sqa::device_cus(), 64);
}

namespace {

// The tail-split plan for these sizes on the current device (0: none).
int tail_plan(int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t d, int dtype, int causal, int64_t* units) {
  *units = 0;
  if (B <= 0 || N <= 0 || H_q < 1 || H_kv < 1 || H_kv > H_q || H_q > 4096 || N > kMaxN) return 0;
  if (d != 64 || dtype != SQA_BF16 || causal != 0 || !prod_le({B, H_q, N, d}, kMaxElems)) return 0;
  return sqa::attn_fwd_tail_plan(B, H_q, H_kv, N, false, sqa::device_cus(), units);
}

}  // namespace

int64_t sqa_attn_fwd_tail_splits(int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t d, int dtype,
                                 int causal) {
  int64_t units = 0;
  const int S = tail_plan(B, H_q, H_kv, N, d, dtype, causal, &units);
  return S > 1 ? S : 1;
}

size_t sqa_attn_fwd_tail_workspace_bytes(int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t d, int dtype,
                                         int causal) {
  int64_t units = 0;
  const int S = tail_plan(B, H_q, H_kv, N, d, dtype, causal, &units);
  return S > 1 ? round256(sqa::attn_tail_workspace_bytes(units, S)) : 0;
}

sqa_status sqa_attn_fwd_tail(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H_q,
                             int64_t H_kv, int64_t N, int64_t d, int dtype, float scale, int causal, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  int64_t units = 0;
  const int S = tail_plan(B, H_q, H_kv, N, d, dtype, causal, &units);
  if (S <= 1)  // no tail to split: the plain forward (validates everything)
    return sqa_attn_fwd_split(q, k, v, o, B, H_q, H_kv, N, d, dtype, scale, causal, lse, 1, nullptr, 0, stream);
  sqa_status s = check_attn(B, H_q, H_kv, N, d, dtype, scale, causal);
  if (s != SQA_OK) return s;
  if (!q || !k || !v || !o) return fail(SQA_ERR_NULL, "q, k, v and o must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(SQA_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(SQA_ERR_ALIGN, "lse must be 4-byte aligned");
  const size_t nq = (size_t)(B * H_q * N * d) * 2, nkv = (size_t)(B * H_kv * N * d) * 2;
  const size_t nl = lse ? (size_t)(B * H_q * N) * 4 : 0;
  if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv))
    return fail(SQA_ERR_ARG, "o overlaps an input");
  if (lse && (overlaps(lse, nl, o, nq) || overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) ||
              overlaps(lse, nl, v, nkv)))
    return fail(SQA_ERR_ARG, "lse overlaps another tensor");
  const size_t need = sqa::attn_tail_workspace_bytes(units, S);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SQA_ERR_WORKSPACE, "tail workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(SQA_ERR_ALIGN, "workspace must be 16-byte aligned");
  const void* ts[5] = {q, k, v, o, lse};
  const size_t tn[5] = {nq, nkv, nkv, nq, nl};
  for (int i = 0; i < 5; ++i)
    if (overlaps(workspace, need, ts[i], tn[i])) return fail(SQA_ERR_ARG, "workspace overlaps a tensor");
  sqa::AttnProblem p{q, k, v, o, lse, B, H_q, H_kv, N, d, scale, causal};
  p.tail_split = S;
  p.tail_units = units;
  p.tail_ws = static_cast<float*>(workspace);
  return launch_attn(p, dtype, static_cast<hipStream_t>(stream));
}

size_t sqa_attn_fwd_split_workspace_bytes(int64_t rows, int64_t d, int dtype, int64_t num_splits) {
  if (rows <= 0 || rows > kMaxElems || num_splits <= 1 || num_splits > kMaxSplits) return 0;
  if ((d != 16 && d != 32 && d != 64 && d != 128) || dtype != SQA_BF16) return 0;
  return round256(sqa::attn_split_workspace_bytes(rows, d, (int)num_splits));
}

size_t sqa_attn_bwd_workspace_bytes(int64_t B, int64_t H_q, int64_t N, int64_t d, int dtype) {
  if (B <= 0 || H_q <= 0 || N <= 0 || (d != 64 && d != 128) || dtype != SQA_BF16) return 0;
  if (N > kMaxN || !prod_le({B, H_q, N, d}, kMaxElems)) return 0;
  return round256(sqa::attn_bwd_rowterm_bytes(B, H_q, N));
}

sqa_status sqa_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H_q,
                        int64_t H_kv, int64_t N, int64_t d, int dtype, float scale, int causal,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return sqa_attn_bwd_split(q, k, v, o, dout, lse, dq, dk, dv, B, H_q, H_kv, N, d, dtype, scale, causal, 1,
                            workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Dry-run the backward's launches, then launch them.
sqa_status run_bwd(sqa::BwdProblem p, hipStream_t st) {
  p.dry_run = true;
  if (sqa::launch_attn_bwd_bf16(p, st) != hipSuccess) return limit_fail("backward");
  p.dry_run = false;
  const hipError_t e = sqa::launch_attn_bwd_bf16(p, st);
  if (e != hipSuccess) return hip_fail(e, "backward kernel launch");
  return SQA_OK;
}

// Every argument rule of the dense backward except the workspace's; `need`
// receives the workspace bytes num_splits needs (0 for an empty problem,
// which returns SQA_OK with nothing to launch).
sqa_status check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H_q, int64_t H_kv,
                     int64_t N, int64_t d, int dtype, float scale, int causal, int64_t num_splits, size_t* need) {
  *need = 0;
  sqa_status s = check_attn(B, H_q, H_kv, N, d, dtype, scale, causal);
  if (s != SQA_OK) return s;
  if (dtype != SQA_BF16 || (d != 64 && d != 128))
    return fail(SQA_ERR_UNSUPPORTED, "backward supports bf16 with d=64 or d=128 (got dtype %d, d=%lld)", dtype,
                (long long)d);
  s = check_bwd_splits(num_splits, causal);
  if (s != SQA_OK) return s;
  if (B == 0 || N == 0) return SQA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return fail(SQA_ERR_NULL, "q, k, v, o, dout, lse, dq, dk and dv must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(SQA_ERR_ALIGN, "q, k, v, o, dout, dq, dk and dv must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(SQA_ERR_ALIGN, "lse must be 4-byte aligned");
  const size_t nq = (size_t)(B * H_q * N * d) * 2, nkv = (size_t)(B * H_kv * N * d) * 2;
  const size_t nl = (size_t)(B * H_q * N) * 4;
  const void* ins[6] = {q, k, v, o, dout, lse};
  const size_t in_n[6] = {nq, nkv, nkv, nq, nq, nl};
  const void* outs[3] = {dq, dk, dv};
  const size_t out_n[3] = {nq, nkv, nkv};
  for (int a = 0; a < 3; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlaps(outs[a], out_n[a], ins[b], in_n[b])) return fail(SQA_ERR_ARG, "an output overlaps an input");
    for (int b = a + 1; b < 3; ++b)
      if (overlaps(outs[a], out_n[a], outs[b], out_n[b])) return fail(SQA_ERR_ARG, "outputs must not overlap");
  }
  *need = sqa_attn_bwd_split_workspace_bytes(B, H_q, H_kv, N, d, dtype, num_splits);
  return SQA_OK;
}

sqa_status launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H_q, int64_t H_kv,
                      int64_t N, int64_t d, int dtype, float scale, int causal, int64_t num_splits, void* workspace,
                      void* stream) {
  sqa::BwdProblem p{q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H_q, H_kv, N, d, scale, causal};
  p.nsplit = (int)num_splits;
  p.split_ws = num_splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                         sqa_attn_bwd_workspace_bytes(B, H_q, N, d, dtype))
                              : nullptr;
  return run_bwd(p, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

sqa_status sqa_attn_bwd_split(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H_q,
                              int64_t H_kv, int64_t N, int64_t d, int dtype, float scale, int causal,
                              int64_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  size_t need = 0;
  sqa_status s = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H_q, H_kv, N, d, dtype, scale, causal, num_splits,
                           &need);
  if (s != SQA_OK || need == 0) return s;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SQA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(SQA_ERR_ALIGN, "workspace must be 16-byte aligned");
  const size_t nq = (size_t)(B * H_q * N * d) * 2, nkv = (size_t)(B * H_kv * N * d) * 2;
  const size_t nl = (size_t)(B * H_q * N) * 4;
  const void* ts[9] = {q, k, v, o, dout, lse, dq, dk, dv};
  const size_t tn[9] = {nq, nkv, nkv, nq, nq, nl, nq, nkv, nkv};
  for (int i = 0; i < 9; ++i)
    if (overlaps(workspace, need, ts[i], tn[i])) return fail(SQA_ERR_ARG, "the workspace overlaps a tensor");
  return launch_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H_q, H_kv, N, d, dtype, scale, causal, num_splits,
                    workspace, stream);
}

sqa_status sqa_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H_q,
                                int64_t H_kv, int64_t N, int64_t d, int dtype, float scale, int causal,
                                void* stream) {
  g_err.clear();
  size_t need = 0;
  sqa_status s = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H_q, H_kv, N, d, dtype, scale, causal, 1, &need);
  if (s != SQA_OK || need == 0) return s;
  if (need > sqa::kNoAllocScratchBytes)
    return fail(SQA_ERR_WORKSPACE,
                "the row terms need %zu bytes, more than the %zu-byte buffer of the allocation-free backward",
                need, sqa::kNoAllocScratchBytes);
  void* scratch = nullptr;
  const hipError_t e = sqa::noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "looking up the allocation-free backward's buffer");
  return launch_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H_q, H_kv, N, d, dtype, scale, causal, 1, scratch,
                    stream);
}

size_t sqa_attn_bwd_varlen_workspace_bytes(int64_t B, int64_t H_q, int64_t T, int64_t d, int dtype) {
  if (B <= 0 || H_q <= 0 || T <= 0 || (d != 64 && d != 128) || dtype != SQA_BF16) return 0;
  if (T > kMaxN || !prod_le({T, H_q, d}, kMaxElems)) return 0;
  return round256(sqa::attn_bwd_rowterm_bytes_packed(H_q, T));
}

size_t sqa_attn_bwd_split_workspace_bytes(int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t d, int dtype,
                                          int64_t num_splits) {
  const size_t rt = sqa_attn_bwd_workspace_bytes(B, H_q, N, d, dtype);
  if (rt == 0 || H_kv < 1 || H_kv > H_q || num_splits < 1 || num_splits > kMaxSplits) return 0;
  return rt + round256(sqa::attn_bwd_split_bytes(B * H_q * N, B * H_kv * N, d, (int)num_splits));
}

size_t sqa_attn_bwd_varlen_split_workspace_bytes(int64_t B, int64_t H_q, int64_t H_kv, int64_t T, int64_t d,
                                                 int dtype, int64_t num_splits) {
  const size_t rt = sqa_attn_bwd_varlen_workspace_bytes(B, H_q, T, d, dtype);
  if (rt == 0 || H_kv < 1 || H_kv > H_q || num_splits < 1 || num_splits > kMaxSplits) return 0;
  return rt + round256(sqa::attn_bwd_split_bytes(H_q * T, H_kv * T, d, (int)num_splits));
}

int64_t sqa_attn_bwd_num_splits(int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t d, int dtype,
                                int causal, int64_t T) {
  if (B <= 0 || N <= 0 || H_q < 1 || H_kv < 1 || H_kv > H_q || H_q > 4096 || N > kMaxN || T < 0) return 1;
  if (T > 0 && N > T) return 1;
  if (!prod_le({B, H_q, N, d > 0 ? d : 1}, kMaxElems) || !prod_le({T, H_q, d > 0 ? d : 1}, kMaxElems)) return 1;
  if ((d != 64 && d != 128) || dtype != SQA_BF16) return 1;
  return sqa::attn_bwd_auto_splits(B, H_q, H_kv, N, T, d, causal != 0, sqa::device_cus());
}

sqa_status sqa_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens,
                               int64_t B, int64_t H_q, int64_t H_kv, int64_t T, int64_t max_seqlen, int64_t d,
                               int dtype, float scale, int causal, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return sqa_attn_bwd_varlen_split(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, B, H_q, H_kv, T, max_seqlen, d,
                                   dtype, scale, causal, 1, workspace, workspace_bytes, stream);
}

sqa_status sqa_attn_bwd_varlen_split(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                     const float* lse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens,
                                     int64_t B, int64_t H_q, int64_t H_kv, int64_t T, int64_t max_seqlen, int64_t d,
                                     int dtype, float scale, int causal, int64_t num_splits, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (B < 0 || T < 0 || max_seqlen < 0) return fail(SQA_ERR_SHAPE, "negative size");
  sqa_status s = check_attn(B > 0 ? 1 : 0, H_q, H_kv, max_seqlen, d, dtype, scale, causal);
  if (s != SQA_OK) return s;
  if (dtype != SQA_BF16 || (d != 64 && d != 128))
    return fail(SQA_ERR_UNSUPPORTED, "backward supports bf16 with d=64 or d=128 (got dtype %d, d=%lld)", dtype,
                (long long)d);
  if (max_seqlen > T) return fail(SQA_ERR_SHAPE, "max_seqlen=%lld exceeds T=%lld", (long long)max_seqlen,
                                  (long long)T);
  if (T > kMaxN || !prod_le({T, H_q, d}, kMaxElems)) return fail(SQA_ERR_SHAPE, "tensor too large");
  if (B > 0x7fffffffLL) return fail(SQA_ERR_SHAPE, "too many sequences");
  s = check_bwd_splits(num_splits, causal);
  if (s != SQA_OK) return s;
  if (B == 0 || T == 0 || max_seqlen == 0) return SQA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !cu_seqlens)
    return fail(SQA_ERR_NULL, "q, k, v, o, dout, lse, dq, dk, dv and cu_seqlens must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(SQA_ERR_ALIGN, "q, k, v, o, dout, dq, dk and dv must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(cu_seqlens, 4)) return fail(SQA_ERR_ALIGN, "lse and cu_seqlens must be 4-byte aligned");
  const size_t need = sqa_attn_bwd_varlen_split_workspace_bytes(B, H_q, H_kv, T, d, dtype, num_splits);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SQA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(SQA_ERR_ALIGN, "workspace must be 16-byte aligned");
  const size_t nq = (size_t)(H_q * T * d) * 2, nkv = (size_t)(H_kv * T * d) * 2;
  const size_t nl = (size_t)(H_q * T) * 4, ncu = (size_t)(B + 1) * 4;
  const void* ins[7] = {q, k, v, o, dout, lse, cu_seqlens};
  const size_t in_n[7] = {nq, nkv, nkv, nq, nq, nl, ncu};
  const void* outs[4] = {dq, dk, dv, workspace};
  const size_t out_n[4] = {nq, nkv, nkv, need};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 7; ++b)
      if (overlaps(outs[a], out_n[a], ins[b], in_n[b]))
        return fail(SQA_ERR_ARG, "an output or the workspace overlaps an input");
    for (int b = a + 1; b < 4; ++b)
      if (overlaps(outs[a], out_n[a], outs[b], out_n[b]))
        return fail(SQA_ERR_ARG, "outputs and workspace must not overlap each other");
  }
  sqa::BwdProblem p{q,  k,  v,  o,   dout, lse,       dq,    dk,     dv,         workspace,
                    B,  H_q, H_kv, max_seqlen, d, scale, causal, cu_seqlens, T};
  p.nsplit = (int)num_splits;
  p.split_ws = num_splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                         sqa_attn_bwd_varlen_workspace_bytes(B, H_q, T, d, dtype))
                              : nullptr;
  return run_bwd(p, static_cast<hipStream_t>(stream));
}

size_t sqa_layer_workspace_bytes(int64_t B, int64_t N, int64_t D, int64_t H, int64_t H_q, int64_t H_kv,
                                 int dtype) {
  if (B <= 0 || N <= 0 || D <= 0 || H <= 0 || H_q <= 0 || H_kv <= 0) return 0;
  if (dtype != SQA_BF16 || D % H != 0) return 0;
  const int64_t d = D / H;
  if (!prod_le({B, N, H_q > H_kv ? H_q : H_kv, d}, kMaxElems)) return 0;
  const size_t esz = 2;
  const size_t nq = (size_t)(B * H_q * N * d) * esz, nkv = (size_t)(B * H_kv * N * d) * esz;
  return 2 * round256(nq) + 2 * round256(nkv);
}

namespace {

// Shape and argument rules of the layer (shared with the block).
sqa_status check_layer(int64_t B, int64_t N, int64_t D, int64_t H, int64_t H_q, int64_t H_kv, float rope_base,
                       float scale, int causal, int dtype, int64_t* d_out) {
  if (B < 0 || N < 0 || D < 0 || H < 0) return fail(SQA_ERR_SHAPE, "negative size");
  if (H < 1 || D < 1 || D % H != 0)
    return fail(SQA_ERR_SHAPE, "D must be a positive multiple of H (got D=%lld, H=%lld)", (long long)D,
                (long long)H);
  const int64_t d = D / H;
  if (dtype != SQA_BF16) return fail(SQA_ERR_UNSUPPORTED, "the layer supports bf16 only");
  if (d != 16 && d != 64)
    return fail(SQA_ERR_UNSUPPORTED, "the layer supports head dims 16 and 64 (got D/H=%lld)", (long long)d);
  sqa_status s = check_attn(B, H_q, H_kv, N, d, dtype, scale, causal);
  if (s != SQA_OK) return s;
  if (!std::isfinite(rope_base) || rope_base <= 0.f) return fail(SQA_ERR_ARG, "rope_base must be finite and > 0");
  if (D % 16 != 0) return fail(SQA_ERR_UNSUPPORTED, "D must be a multiple of 16");
  if (!prod_le({B, N, D}, kMaxElems)) return fail(SQA_ERR_SHAPE, "tensor too large");
  *d_out = d;
  return SQA_OK;
}

// Launch the layer on already validated arguments; `resid` (nullable) is
// added to the output projection.
sqa_status run_layer(const void* x, const void* w_q, const void* w_k, const void* w_v, const void* w_o,
                     const void* resid, void* y, int64_t B, int64_t N, int64_t D, int64_t d, int64_t H_q,
                     int64_t H_kv, float rope_base, float scale, int causal, char* ws, hipStream_t st) {
  const size_t nq = round256((size_t)(B * H_q * N * d) * 2), nkv = round256((size_t)(B * H_kv * N * d) * 2);
  void* qb = ws;
  void* kb = ws + nq;
  void* vb = ws + nq + nkv;
  void* ob = ws + nq + 2 * nkv;
  sqa::QkvProblem qp{x, w_q, w_k, w_v, qb, kb, vb, B, N, D, H_q, H_kv, d, rope_base};
  sqa::AttnProblem ap{qb, kb, vb, ob, nullptr, B, H_q, H_kv, N, d, scale, causal};
  sqa::OprojProblem op{ob, w_o, y, B, N, D, H_q, d, resid};
  qp.dry_run = ap.dry_run = op.dry_run = true;
  if (sqa::launch_qkv_rope(qp, st) != hipSuccess) return limit_fail("qkv projection");
  if (sqa::launch_attn_fwd_bf16(ap, st) != hipSuccess) return limit_fail("attention");
  if (sqa::launch_out_proj(op, st) != hipSuccess) return limit_fail("output projection");
  qp.dry_run = ap.dry_run = op.dry_run = false;
  hipError_t e = sqa::launch_qkv_rope(qp, st);
  if (e != hipSuccess) return hip_fail(e, "qkv projection launch");
  e = sqa::launch_attn_fwd_bf16(ap, st);
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  e = sqa::launch_out_proj(op, st);
  if (e != hipSuccess) return hip_fail(e, "output projection launch");
  return SQA_OK;
}

}  // namespace

sqa_status sqa_layer_fwd(const void* x, const void* w_q, const void* w_k, const void* w_v,
                         const void* w_o, void* y, int64_t B, int64_t N, int64_t D, int64_t H,
                         int64_t H_q, int64_t H_kv, float rope_base, float scale, int causal,
                         int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  int64_t d = 0;
  sqa_status s = check_layer(B, N, D, H, H_q, H_kv, rope_base, scale, causal, dtype, &d);
  if (s != SQA_OK) return s;
  if (B == 0 || N == 0) return SQA_OK;
  if (!x || !w_q || !w_k || !w_v || !w_o || !y) return fail(SQA_ERR_NULL, "inputs and y must be non-NULL");
  if (!aligned(x, 16) || !aligned(w_q, 16) || !aligned(w_k, 16) || !aligned(w_v, 16) || !aligned(w_o, 16) ||
      !aligned(y, 16))
    return fail(SQA_ERR_ALIGN, "x, weights and y must be 16-byte aligned");
  const size_t need = sqa_layer_workspace_bytes(B, N, D, H, H_q, H_kv, dtype);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SQA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if (!aligned(workspace, 256)) return fail(SQA_ERR_ALIGN, "workspace must be 256-byte aligned");
  const size_t nx = (size_t)(B * N * D) * 2;
  const size_t nwq = (size_t)(D * H_q * d) * 2, nwk = (size_t)(D * H_kv * d) * 2;
  if (overlaps(y, nx, x, nx) || overlaps(y, nx, w_q, nwq) || overlaps(y, nx, w_k, nwk) ||
      overlaps(y, nx, w_v, nwk) || overlaps(y, nx, w_o, nwq))
    return fail(SQA_ERR_ARG, "y overlaps an input");
  if (overlaps(workspace, need, x, nx) || overlaps(workspace, need, y, nx) || overlaps(workspace, need, w_q, nwq) ||
      overlaps(workspace, need, w_k, nwk) || overlaps(workspace, need, w_v, nwk) || overlaps(workspace, need, w_o, nwq))
    return fail(SQA_ERR_ARG, "workspace overlaps an input or y");
  return run_layer(x, w_q, w_k, w_v, w_o, nullptr, y, B, N, D, d, H_q, H_kv, rope_base, scale, causal,
                   static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

size_t sqa_block_workspace_bytes(int64_t B, int64_t N, int64_t D, int64_t H, int64_t H_q, int64_t H_kv,
                                 int64_t F, int dtype) {
  const size_t lw = sqa_layer_workspace_bytes(B, N, D, H, H_q, H_kv, dtype);
  if (lw == 0 || F <= 0 || !prod_le({B, N, F}, kMaxElems)) return 0;
  return lw + 2 * round256((size_t)(B * N * D) * 2) + round256((size_t)(B * N * F) * 2);
}

sqa_status sqa_block_fwd(const void* x, const void* norm1, const void* w_q, const void* w_k, const void* w_v,
                         const void* w_o, const void* norm2, const void* w_gate, const void* w_up,
                         const void* w_down, void* y, int64_t B, int64_t N, int64_t D, int64_t H, int64_t H_q,
                         int64_t H_kv, int64_t F, float rope_base, float scale, float eps, int causal, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  int64_t d = 0;
  sqa_status s = check_layer(B, N, D, H, H_q, H_kv, rope_base, scale, causal, dtype, &d);
  if (s != SQA_OK) return s;
  if (F < 1 || F % 16 != 0) return fail(SQA_ERR_UNSUPPORTED, "F must be a positive multiple of 16 (got %lld)",
                                        (long long)F);
  if (!std::isfinite(eps) || eps < 0.f) return fail(SQA_ERR_ARG, "eps must be finite and >= 0");
  if (B == 0 || N == 0) return SQA_OK;
  if (!prod_le({B, N, F}, kMaxElems)) return fail(SQA_ERR_SHAPE, "tensor too large");
  const void* ins[10] = {x, norm1, w_q, w_k, w_v, w_o, norm2, w_gate, w_up, w_down};
  for (const void* p : ins)
    if (!p) return fail(SQA_ERR_NULL, "inputs must be non-NULL");
  if (!y) return fail(SQA_ERR_NULL, "y must be non-NULL");
  for (const void* p : ins)
    if (!aligned(p, 16)) return fail(SQA_ERR_ALIGN, "inputs must be 16-byte aligned");
  if (!aligned(y, 16)) return fail(SQA_ERR_ALIGN, "y must be 16-byte aligned");
  const size_t need = sqa_block_workspace_bytes(B, N, D, H, H_q, H_kv, F, dtype);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SQA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL");
  if (!aligned(workspace, 256)) return fail(SQA_ERR_ALIGN, "workspace must be 256-byte aligned");
  const size_t nx = (size_t)(B * N * D) * 2;
  const size_t nwq = (size_t)(D * H_q * d) * 2, nwk = (size_t)(D * H_kv * d) * 2, nf = (size_t)(D * F) * 2;
  const size_t in_n[10] = {nx, (size_t)D * 2, nwq, nwk, nwk, nwq, (size_t)D * 2, nf, nf, nf};
  for (int i = 0; i < 10; ++i) {
    if (overlaps(y, nx, ins[i], in_n[i])) return fail(SQA_ERR_ARG, "y overlaps an input");
    if (overlaps(workspace, need, ins[i], in_n[i])) return fail(SQA_ERR_ARG, "workspace overlaps an input");
  }
  if (overlaps(workspace, need, y, nx)) return fail(SQA_ERR_ARG, "workspace overlaps y");

  char* ws = static_cast<char*>(workspace);
  const size_t lw = sqa_layer_workspace_bytes(B, N, D, H, H_q, H_kv, dtype);
  void* xn = ws + lw;                            // normalised input of a sub-layer
  void* hb = ws + lw + round256(nx);             // residual stream after attention
  void* gb = ws + lw + 2 * round256(nx);         // SwiGLU activations [M, F]
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t M = B * N;
  sqa::GateUpProblem gp{xn, w_gate, w_up, gb, M, D, F};
  sqa::DenseProblem dp{gb, w_down, hb, y, M, F, D};
  gp.dry_run = dp.dry_run = true;
  if (sqa::launch_rms_norm(x, norm1, xn, M, D, eps, st, true) != hipSuccess) return limit_fail("RMSNorm");
  if (sqa::launch_gate_up(gp, st) != hipSuccess) return limit_fail("SwiGLU gate/up projection");
  if (sqa::launch_dense_residual(dp, st) != hipSuccess) return limit_fail("down projection");
  {
    // the layer's own launches, dry (run_layer repeats this before launching)
    const size_t nq = round256((size_t)(B * H_q * N * d) * 2), nkv = round256((size_t)(B * H_kv * N * d) * 2);
    sqa::QkvProblem qp{xn, w_q, w_k, w_v, ws, ws + nq, ws + nq + nkv, B, N, D, H_q, H_kv, d, rope_base};
    sqa::AttnProblem ap{ws, ws + nq, ws + nq + nkv, ws + nq + 2 * nkv, nullptr, B, H_q, H_kv, N, d, scale, causal};
    sqa::OprojProblem op{ws + nq + 2 * nkv, w_o, hb, B, N, D, H_q, d, x};
    qp.dry_run = ap.dry_run = op.dry_run = true;
    if (sqa::launch_qkv_rope(qp, st) != hipSuccess) return limit_fail("qkv projection");
    if (sqa::launch_attn_fwd_bf16(ap, st) != hipSuccess) return limit_fail("attention");
    if (sqa::launch_out_proj(op, st) != hipSuccess) return limit_fail("output projection");
  }
  gp.dry_run = dp.dry_run = false;
  hipError_t e = sqa::launch_rms_norm(x, norm1, xn, M, D, eps, st);
  if (e != hipSuccess) return hip_fail(e, "RMSNorm launch");
  s = run_layer(xn, w_q, w_k, w_v, w_o, x, hb, B, N, D, d, H_q, H_kv, rope_base, scale, causal, ws, st);
  if (s != SQA_OK) return s;
  e = sqa::launch_rms_norm(hb, norm2, xn, M, D, eps, st);
  if (e != hipSuccess) return hip_fail(e, "RMSNorm launch");
  e = sqa::launch_gate_up(gp, st);
  if (e != hipSuccess) return hip_fail(e, "SwiGLU gate/up launch");
  e = sqa::launch_dense_residual(dp, st);
  if (e != hipSuccess) return hip_fail(e, "down projection launch");
  return SQA_OK;
}

const char* sqa_status_str(int status) {
  switch (status) {
    case SQA_OK: return "SQA_OK";
    case SQA_ERR_NULL: return "SQA_ERR_NULL";
    case SQA_ERR_SHAPE: return "SQA_ERR_SHAPE";
    case SQA_ERR_UNSUPPORTED: return "SQA_ERR_UNSUPPORTED";
    case SQA_ERR_ALIGN: return "SQA_ERR_ALIGN";
    case SQA_ERR_WORKSPACE: return "SQA_ERR_WORKSPACE";
    case SQA_ERR_HIP: return "SQA_ERR_HIP";
    case SQA_ERR_ARG: return "SQA_ERR_ARG";
    default: return "SQA_ERR_UNKNOWN";
  }
}

const char* sqa_last_error(void) { return g_err.c_str(); }

int sqa_version(void) { return 100; }

}  // extern "C"
