/*
 * libsqa -- Sparse Query Attention (SQA) forward on AMD Instinct MI355X (gfx950).
 *
 * SQA is full-sequence softmax attention in which the number of query heads
 * H_q is cut below the baseline head count H while the head width d stays
 * d_model / H, so the attention-score FLOPs fall in proportion to H_q / H
 * (SQA paper abstract, chatpaper page; SQAT-m model card, "Architecture
 * details"). Query heads form H_kv contiguous groups that each share one key
 * head and one value head, as in grouped-query attention ("GQA: Training
 * Generalized Multi-Query Transformer Models", nlp-lineage page, "The idea"):
 * query head i reads K/V head floor(i * H_kv / H_q).
 *
 * Conventions shared by every entry point
 *   - Pointers to tensors are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors), 16-byte aligned, contiguous row-major, with the shapes given.
 *     The caller owns every buffer; the library never allocates, frees or
 *     synchronises, and keeps no state across calls except a thread-local
 *     error string.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream. Work is enqueued asynchronously; results are visible after the
 *     caller synchronises the stream.
 *   - Every argument is checked before anything is launched. On any error
 *     nothing is launched and the outputs are left untouched. Launch failures
 *     return SQA_ERR_HIP (detail in sqa_last_error()). Faults during execution
 *     surface at the caller's next synchronisation.
 *   - Zero-sized problems (B == 0 or N == 0) return SQA_OK and launch nothing.
 *   - No exceptions or output cross this interface.
 *
 * Size limits (SQA_ERR_SHAPE, checked before anything is launched):
 *   - N (or max_seqlen) <= 2^30 and every tensor <= 2^40 elements.
 *   - bf16 attention with d = 64: N <= 16777215 (one head's K or V rows,
 *     N * 128 bytes, must stay below 2^31, the range of a buffer
 *     descriptor); d = 128: N <= 8388607. The backward has the same limits,
 *     and its row terms (B * H_q * N rounded up to whole 32-row tiles per
 *     head; packed: H_q * (T + 32)) must stay below 2^29 - 64 rows.
 *   - Grid sizes: B * H_kv, B * H_q and every kernel's workgroup count must
 *     stay below 2^31.
 *   - Layer and block: the activations [B*N, D] and every weight matrix
 *     below 2^31 bytes (32-bit offsets of the projection kernels), and one
 *     sequence's heads (H_q * N * d bf16 values) below 2^31 bytes.
 *   A problem past these limits returns SQA_ERR_SHAPE with the kernel whose
 *   limit it exceeds named in sqa_last_error(); SQA_ERR_HIP is reserved for
 *   failures the HIP runtime reports.
 */
#ifndef SQA_H_
#define SQA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SQA_OK = 0,
  SQA_ERR_NULL = 1,        /* a required pointer is NULL                         */
  SQA_ERR_SHAPE = 2,       /* negative size, H_kv not in [1, H_q], past a limit   */
  SQA_ERR_UNSUPPORTED = 3, /* valid but not implemented: d, dtype, ...            */
  SQA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                     */
  SQA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required              */
  SQA_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed           */
  SQA_ERR_ARG = 7          /* other invalid argument (non-finite scale, aliasing) */
} sqa_status;

typedef enum { SQA_F32 = 0, SQA_BF16 = 1 } sqa_dtype;

/*
 * sqa_attn_fwd -- SQA attention forward.
 *
 * For every b < B, query head i < H_q, position t < N, with
 * j = floor(i * H_kv / H_q) (contiguous query-head groups, "GQA ..." page,
 * "The idea"; groups differ in size by at most one head when H_kv does not
 * divide H_q):
 *   s_tu      = scale * sum_c q[b,i,t,c] * k[b,j,u,c]          for u in U_t
 *   o[b,i,t,:] = sum_{u in U_t} softmax_u(s_tu) * v[b,j,u,:]
 *   lse[b,i,t] = log sum_{u in U_t} exp(s_tu)                   (natural log)
 * U_t = {0..N-1} if causal == 0 (encoder-style, full sequence) and {0..t} if
 * causal == 1 (decoder). The pages name the attention but do not write the
 * formula; this is the textbook scaled-dot-product form.
 *
 *   q    [B, H_q,  N, d]  input,  dtype
 *   k, v [B, H_kv, N, d]  input,  dtype
 *   o    [B, H_q,  N, d]  output, dtype; must not overlap q, k or v
 *   lse  [B, H_q,  N]     optional output, fp32; NULL to skip
 *   d     16, 32, 64 or 128.  1 <= H_kv <= H_q.
 *   dtype SQA_BF16: bf16 in/out; scores, softmax state and the output
 *         accumulator are fp32, the probabilities are rounded to bf16 for the
 *         P.V product, the output is rounded to nearest-even bf16.
 *         SQA_F32: fp32 in/out with fp32 arithmetic throughout.
 *   scale any finite float (1/sqrt(d) is the usual choice).
 * Errors: SQA_ERR_NULL, SQA_ERR_SHAPE, SQA_ERR_UNSUPPORTED (d, dtype),
 * SQA_ERR_ALIGN, SQA_ERR_ARG (scale not finite, causal not 0/1, o overlaps an
 * input), SQA_ERR_HIP.
 */
sqa_status sqa_attn_fwd(const void* q, const void* k, const void* v, void* o,
                        int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t d,
                        int dtype, float scale, int causal, float* lse, void* stream);

/*
 * sqa_attn_fwd_varlen -- sqa_attn_fwd over a packed batch of sequences of
 * different lengths. The B sequences are concatenated along the token axis:
 * sequence b owns tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of every head,
 * attends only to its own keys, and its causal positions count from 0 (a
 * batch of different-length sequences; the pages do not describe one, this
 * is the plain reading). Per sequence the result equals sqa_attn_fwd with
 * B = 1 on that sequence's rows.
 *
 *   q, o       [H_q,  T, d]  input / output, dtype; o must not overlap an input
 *   k, v       [H_kv, T, d]  inputs, dtype
 *   cu_seqlens [B + 1]       input, DEVICE int32 array: cu[0] = 0,
 *                            non-decreasing, cu[B] = T, every length
 *                            cu[b+1] - cu[b] <= max_seqlen. Not read by the
 *                            host; offsets outside this contract give
 *                            unspecified (but in-bounds) results.
 *   lse        [H_q, T]      optional output, fp32 natural log; NULL to skip
 *   max_seqlen the longest sequence (sizes the launch), <= T
 *   d, dtype, scale, causal, head counts: as sqa_attn_fwd. Empty sequences
 *   are allowed.
 * Errors: as sqa_attn_fwd; cu_seqlens must be 4-byte aligned.
 */
sqa_status sqa_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                               const int32_t* cu_seqlens, int64_t B, int64_t H_q, int64_t H_kv,
                               int64_t T, int64_t max_seqlen, int64_t d, int dtype, float scale,
                               int causal, float* lse, void* stream);

/*
 * sqa_attn_fwd_num_splits -- the number of key-range splits the library
 * recommends for sqa_attn_fwd_split / sqa_attn_fwd_varlen_split on the
 * current device (1: none). Dense (T = 0; B sequences of N tokens): it
 * models the launch as rounds of workgroups over the device's compute
 * units and splits an encoder-style launch when its workgroups fill less
 * than one round (up to 4 splits) or when two splits cut the rounds of
 * whole-row workgroups by at least 10 %. Packed (T > 0 tokens in B
 * sequences, N = max_seqlen): 2 when the longest sequence has at least
 * 2048 tokens and holds at least a quarter of the T (its workgroups then
 * form the tail of the launch). Never under a causal mask (measured
 * slower), never at d = 16, 32 or 128 (measured slower or no gain) and
 * never for dtype != SQA_BF16. Returns 1 for invalid sizes.
 */
int64_t sqa_attn_fwd_num_splits(int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t d, int dtype,
                                int causal, int64_t T);

/*
 * sqa_attn_fwd_split_workspace_bytes -- bytes of device workspace a split
 * forward with num_splits > 1 needs for `rows` query rows (B * H_q * N, or
 * H_q * T packed): num_splits * rows * (d + 2) fp32 values (each range's
 * unnormalised output, maximum and sum per row). Returns 0 when
 * num_splits <= 1, for invalid sizes, and when dtype != SQA_BF16.
 */
size_t sqa_attn_fwd_split_workspace_bytes(int64_t rows, int64_t d, int dtype, int64_t num_splits);

/*
 * sqa_attn_fwd_split / sqa_attn_fwd_varlen_split -- sqa_attn_fwd and
 * sqa_attn_fwd_varlen with the keys of each long sequence cut into
 * num_splits contiguous ranges computed by separate workgroups, whose
 * partial softmax states are merged afterwards (the streaming-softmax
 * recurrence applied once more across the ranges; the pages do not
 * describe a kernel, this is a scheduling choice). Same results as the
 * unsplit calls up to fp32 rounding order. At d = 64 a range holds at least
 * 1024 keys (an even number of 32-key tiles), at d = 16 and 32 at least 256
 * (64-key tiles), so a short sequence is computed unsplit or gets fewer
 * than num_splits ranges (d = 128: at least 1024 keys, 32-key tiles).
 * sqa_attn_fwd_num_splits only ever recommends splits at d = 64: at d = 16
 * under a causal mask (the SQAT-m layer's shape) and at d = 128 on a packed
 * batch, split launches measured slower.
 *
 *   num_splits 1..16; > 1 only for dtype SQA_BF16 (SQA_ERR_UNSUPPORTED
 *              otherwise). 1 behaves exactly as the unsplit call and
 *              ignores the workspace.
 *   workspace  device buffer of at least sqa_attn_fwd_split_workspace_bytes
 *              bytes, 16-byte aligned, owned by the caller, not overlapping
 *              any tensor argument; contents on return unspecified.
 *   every other argument: as sqa_attn_fwd / sqa_attn_fwd_varlen.
 * Errors: as those calls, plus SQA_ERR_WORKSPACE.
 */
sqa_status sqa_attn_fwd_split(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H_q,
                              int64_t H_kv, int64_t N, int64_t d, int dtype, float scale, int causal, float* lse,
                              int64_t num_splits, void* workspace, size_t workspace_bytes, void* stream);
sqa_status sqa_attn_fwd_varlen_split(const void* q, const void* k, const void* v, void* o,
                                     const int32_t* cu_seqlens, int64_t B, int64_t H_q, int64_t H_kv,
                                     int64_t T, int64_t max_seqlen, int64_t d, int dtype, float scale,
                                     int causal, float* lse, int64_t num_splits, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * sqa_attn_fwd_tail_splits / sqa_attn_fwd_tail_workspace_bytes /
 * sqa_attn_fwd_tail -- sqa_attn_fwd with a schedule for launches whose last
 * round of workgroups is mostly empty (a scheduling choice; the pages do
 * not describe a kernel). The forward's workgroups run in rounds of two per
 * compute unit. When the workgroups past the last whole round fill at most
 * half a round, each of them runs as S workgroups over S contiguous key
 * ranges (S = floor(slots / those workgroups), at most 16, each range at
 * least 1024 keys), whose partial softmax states are merged afterwards; so
 * the last round takes about 1/S of a workgroup's time instead of a whole
 * one. Same results as sqa_attn_fwd up to fp32 rounding order.
 * Planned only for dtype SQA_BF16, d = 64, causal == 0 and H_kv dividing
 * H_q; the plan depends on the current device's compute-unit count.
 *
 *   sqa_attn_fwd_tail_splits        S for these sizes (1: no tail split)
 *   sqa_attn_fwd_tail_workspace_bytes  device workspace sqa_attn_fwd_tail
 *                                   needs: S * units * 256 rows * (64 + 2)
 *                                   fp32 values (0 when S = 1)
 *   sqa_attn_fwd_tail               arguments as sqa_attn_fwd, plus the
 *                                   workspace (16-byte aligned, owned by the
 *                                   caller, not overlapping any tensor;
 *                                   contents on return unspecified). With
 *                                   S = 1 it is sqa_attn_fwd and ignores the
 *                                   workspace.
 * Errors: as sqa_attn_fwd, plus SQA_ERR_WORKSPACE.
 */
int64_t sqa_attn_fwd_tail_splits(int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t d, int dtype,
                                 int causal);
size_t sqa_attn_fwd_tail_workspace_bytes(int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t d, int dtype,
                                         int causal);
sqa_status sqa_attn_fwd_tail(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H_q,
                             int64_t H_kv, int64_t N, int64_t d, int dtype, float scale, int causal, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * sqa_attn_bwd_workspace_bytes -- bytes of device workspace sqa_attn_bwd
 * needs for these sizes: one fp32 pair (lse * log2(e), D_t) per query row,
 * with each (batch, query head)'s rows padded up to a multiple of 32, i.e.
 * 8 * B * H_q * ceil(N / 32) * 32 bytes. Returns 0 for invalid or zero
 * sizes, or when d / dtype are not supported by sqa_attn_bwd.
 */
size_t sqa_attn_bwd_workspace_bytes(int64_t B, int64_t H_q, int64_t N, int64_t d, int dtype);

/*
 * sqa_attn_bwd -- gradients of sqa_attn_fwd for an upstream gradient dout
 * (the backward pass of training, where the SQA abstract places SQA's gains:
 * pre-training and fine-tuning). With P the forward's attention
 * probabilities (same scale and causal mask) and j = floor(i * H_kv / H_q):
 *   D_t        = sum_c dout[b,i,t,c] * o[b,i,t,c]
 *   dS_tu      = P_tu * (sum_c dout[b,i,t,c] * v[b,j,u,c] - D_t)
 *   dq[b,i,t]  = scale * sum_u dS_tu * k[b,j,u]
 *   dk[b,j,u]  = scale * sum_{i in group j} sum_t dS_tu * q[b,i,t]
 *   dv[b,j,u]  = sum_{i in group j} sum_t P_tu * dout[b,i,t]
 * the exact derivative of the forward's definition (a textbook chain rule
 * through the softmax; the pages do not write it out).
 *
 *   q, o, dout [B, H_q, N, d]  inputs, bf16; o and lse as written by
 *                              sqa_attn_fwd on the same q, k, v, scale, causal
 *   k, v       [B, H_kv, N, d] inputs, bf16
 *   lse        [B, H_q, N]     input, fp32, natural log (sqa_attn_fwd's lse)
 *   dq         [B, H_q, N, d]  output, bf16, overwritten
 *   dk, dv     [B, H_kv, N, d] outputs, bf16, overwritten (group sums)
 *   workspace  device buffer of at least sqa_attn_bwd_workspace_bytes(...)
 *              bytes, owned by the caller; contents on return unspecified.
 *   d = 64 or 128 and dtype SQA_BF16 only (others: SQA_ERR_UNSUPPORTED).
 *   Arithmetic: P is recomputed from lse; scores and all sums are fp32, P and
 *   dS are rounded to bf16 (nearest even) for the matrix products, outputs
 *   are rounded to nearest-even bf16. Deterministic: no atomics.
 * Outputs must not overlap each other, an input or the workspace.
 * Errors: as sqa_attn_fwd, plus SQA_ERR_WORKSPACE.
 */
sqa_status sqa_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H_q,
                        int64_t H_kv, int64_t N, int64_t d, int dtype, float scale, int causal,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * sqa_attn_bwd_noalloc -- sqa_attn_bwd without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving or training loops, and harnesses that forbid allocation.
 * Same arguments (minus workspace) and the same kernels, so the same
 * results as sqa_attn_bwd bit for bit. The row terms go into a fixed
 * 32 MiB device buffer that the library holds on each GPU it runs on, from
 * the first call on that GPU until the process ends: the problem must
 * satisfy sqa_attn_bwd_workspace_bytes(B, H_q, N, d, dtype) <= 33554432
 * (8 B per query row, rows of each (batch, query head) padded to a multiple
 * of 32: about 4.19M rows, e.g. B*H_q = 16 heads at N = 262144), else
 * SQA_ERR_WORKSPACE and nothing is launched. Nothing in the buffer needs to
 * start at zero: every call writes all of the entries it reads. The call
 * allocates nothing and calls no allocating routine; its first call on a
 * device looks up the buffer's address (hipGetSymbolAddress).
 * Calls that overlap in time on one GPU (different streams, or different
 * host threads) share the buffer and race: serialise them.
 * Errors: as sqa_attn_bwd (SQA_ERR_WORKSPACE for problems over the limit;
 * SQA_ERR_HIP if the address lookup fails).
 */
sqa_status sqa_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H_q,
                                int64_t H_kv, int64_t N, int64_t d, int dtype, float scale, int causal,
                                void* stream);

/*
 * sqa_attn_bwd_varlen_workspace_bytes -- bytes of device workspace
 * sqa_attn_bwd_varlen needs: one fp32 pair (lse * log2(e), D_t) per packed
 * row plus 32 rows of padding per query head, 8 * H_q * (T + 32) bytes
 * rounded up to 256. Returns 0 for invalid or zero sizes, or when d / dtype
 * are not supported.
 */
size_t sqa_attn_bwd_varlen_workspace_bytes(int64_t B, int64_t H_q, int64_t T, int64_t d, int dtype);

/*
 * sqa_attn_bwd_varlen -- sqa_attn_bwd for a packed batch of variable-length
 * sequences, the layout of sqa_attn_fwd_varlen: per sequence the result
 * equals sqa_attn_bwd with B = 1 on that sequence's rows.
 *
 *   q, o, dout, dq [H_q,  T, d]  bf16 (dq output, overwritten)
 *   k, v, dk, dv   [H_kv, T, d]  bf16 (dk, dv outputs, overwritten)
 *   lse            [H_q, T]      fp32, sqa_attn_fwd_varlen's lse
 *   cu_seqlens     [B + 1]       DEVICE int32 offsets, as in sqa_attn_fwd_varlen
 *   workspace      at least sqa_attn_bwd_varlen_workspace_bytes(...) bytes
 *   d = 64 or 128, dtype SQA_BF16; head counts, scale, causal as sqa_attn_bwd.
 * Outputs must not overlap each other, an input (cu_seqlens included) or
 * the workspace. Errors: as sqa_attn_bwd.
 */
sqa_status sqa_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens,
                               int64_t B, int64_t H_q, int64_t H_kv, int64_t T, int64_t max_seqlen, int64_t d,
                               int dtype, float scale, int causal, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * sqa_attn_bwd_split / sqa_attn_bwd_varlen_split -- sqa_attn_bwd and
 * sqa_attn_bwd_varlen with the work of each long sequence cut into
 * num_splits ranges computed by separate workgroups: dQ over ranges of keys,
 * dK and dV over ranges of query rows. Each range leaves an fp32 partial
 * gradient in the workspace and the partials are summed (dQ, dK and dV are
 * plain sums over keys and queries; the pages do not describe a kernel, this
 * is a scheduling choice). Same results as the unsplit calls up to fp32
 * rounding order. Ranges hold at least 1024 rows (an even number of 32-row
 * tiles), so a sequence of at most 1024 tokens is computed unsplit.
 *
 *   num_splits 1..16; > 1 only with causal == 0 (SQA_ERR_UNSUPPORTED
 *              otherwise). 1 behaves exactly as the unsplit call.
 *   workspace  device buffer of at least sqa_attn_bwd_split_workspace_bytes
 *              (or the varlen variant) bytes, 16-byte aligned, owned by the
 *              caller: the row terms of the unsplit call followed by the
 *              partials; contents on return unspecified.
 *   every other argument: as sqa_attn_bwd / sqa_attn_bwd_varlen.
 * Errors: as those calls.
 */
sqa_status sqa_attn_bwd_split(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H_q,
                              int64_t H_kv, int64_t N, int64_t d, int dtype, float scale, int causal,
                              int64_t num_splits, void* workspace, size_t workspace_bytes, void* stream);
sqa_status sqa_attn_bwd_varlen_split(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                     const float* lse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens,
                                     int64_t B, int64_t H_q, int64_t H_kv, int64_t T, int64_t max_seqlen, int64_t d,
                                     int dtype, float scale, int causal, int64_t num_splits, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * sqa_attn_bwd_split_workspace_bytes / sqa_attn_bwd_varlen_split_workspace_bytes
 * -- workspace of a split backward: the unsplit call's row terms plus, when
 * num_splits > 1, num_splits * (rows_q + 2 * rows_kv) * d fp32 partials
 * (rows_q = B * H_q * N, rows_kv = B * H_kv * N; packed: H_q * T and
 * H_kv * T), each part rounded up to 256 bytes. Returns 0 for invalid sizes
 * or unsupported d / dtype.
 */
size_t sqa_attn_bwd_split_workspace_bytes(int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t d, int dtype,
                                          int64_t num_splits);
size_t sqa_attn_bwd_varlen_split_workspace_bytes(int64_t B, int64_t H_q, int64_t H_kv, int64_t T, int64_t d,
                                                 int dtype, int64_t num_splits);

/*
 * sqa_attn_bwd_num_splits -- the library's recommended num_splits for the
 * split backward on the current device. Dense (T = 0): 2 for an
 * encoder-style launch whose dK/dV or dQ workgroups fill under half a round
 * of the device's compute units, or whose rounds two splits cut by at least
 * 10 %. Packed (T > 0 tokens, N = max_seqlen): as sqa_attn_fwd_num_splits.
 * Otherwise, and always under a causal mask, 1. Returns 1 for invalid sizes.
 */
int64_t sqa_attn_bwd_num_splits(int64_t B, int64_t H_q, int64_t H_kv, int64_t N, int64_t d, int dtype,
                                int causal, int64_t T);

/*
 * sqa_layer_workspace_bytes -- bytes of device workspace sqa_layer_fwd needs
 * for these sizes: bf16 Q [B,H_q,N,d], K and V [B,H_kv,N,d] and the
 * attention output [B,H_q,N,d], each rounded up to 256 bytes. Returns 0 for
 * invalid or zero sizes.
 */
size_t sqa_layer_workspace_bytes(int64_t B, int64_t N, int64_t D, int64_t H,
                                 int64_t H_q, int64_t H_kv, int dtype);

/*
 * sqa_layer_fwd -- one SQA attention layer forward (SQAT-m model card,
 * "Architecture details" and "Model size difference"):
 *   Q = x W_q, K = x W_k, V = x W_v        (weights in [in, out] layout)
 *   Q, K <- RoPE (rotate-half pairs (c, c+d/2), angle t * rope_base^(-2c/d),
 *                 position t = 0..N-1 of each sequence)
 *   O = sqa_attn_fwd(Q, K, V, scale, causal)
 *   y = O_flat W_o,   O_flat[b, t, i*d + c] = O[b, i, t, c]
 * with d = D / H; head h owns projection columns [h*d, (h+1)*d). No biases,
 * norms or residual.
 *
 *   x   [B, N, D]        bf16 input
 *   w_q [D, H_q*d]       bf16      w_k, w_v [D, H_kv*d] bf16
 *   w_o [H_q*d, D]       bf16
 *   y   [B, N, D]        bf16 output; must not overlap x
 *   workspace            device buffer of at least
 *                        sqa_layer_workspace_bytes(...) bytes, owned by the
 *                        caller; its contents on return are unspecified.
 *   d = D / H must be 16 (the SQAT-m split) or 64, D a multiple of 16
 *   (other head dims: SQA_ERR_UNSUPPORTED); dtype must be SQA_BF16.
 * Errors: as sqa_attn_fwd, plus SQA_ERR_WORKSPACE.
 */
sqa_status sqa_layer_fwd(const void* x, const void* w_q, const void* w_k, const void* w_v,
                         const void* w_o, void* y, int64_t B, int64_t N, int64_t D,
                         int64_t H, int64_t H_q, int64_t H_kv, float rope_base, float scale,
                         int causal, int dtype, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * sqa_block_workspace_bytes -- bytes of device workspace sqa_block_fwd needs:
 * sqa_layer_workspace_bytes(...) plus bf16 buffers for the normalised input
 * [B, N, D], the residual stream after attention [B, N, D] and the SwiGLU
 * activations [B, N, F], each rounded up to 256 bytes. 0 for invalid sizes.
 */
size_t sqa_block_workspace_bytes(int64_t B, int64_t N, int64_t D, int64_t H, int64_t H_q,
                                 int64_t H_kv, int64_t F, int dtype);

/*
 * sqa_block_fwd -- one SQAT-m transformer block forward (SQAT-m model card,
 * "Architecture details": dim 256, RMS Norm, SwiGLU feed forward with 768
 * dim, RoPE; the card does not state the order, this is the pre-norm
 * residual block):
 *   h = x + layer(rms_norm(x, norm1))          (layer as sqa_layer_fwd)
 *   y = h + (silu(z W_gate) * (z W_up)) W_down,  z = rms_norm(h, norm2)
 *   rms_norm(x, g) = x / sqrt(mean_c x_c^2 + eps) * g,  silu(u) = u / (1 + e^-u)
 *
 *   x                [B, N, D]   bf16 input
 *   norm1, norm2     [D]         bf16 RMSNorm gains
 *   w_q, w_k, w_v, w_o           bf16, shapes as in sqa_layer_fwd
 *   w_gate, w_up     [D, F]      bf16      w_down [F, D] bf16
 *   y                [B, N, D]   bf16 output; must not overlap an input
 *   eps              RMSNorm epsilon, finite and >= 0
 *   workspace        at least sqa_block_workspace_bytes(...) bytes,
 *                    256-byte aligned, owned by the caller.
 *   Precision: norms, products and SwiGLU in fp32; the normalised input, the
 *   residual stream h, the activations and Q/K/V/O are stored as bf16.
 *   Layer constraints as sqa_layer_fwd; F a positive multiple of 16.
 * Errors: as sqa_layer_fwd.
 */
sqa_status sqa_block_fwd(const void* x, const void* norm1, const void* w_q, const void* w_k,
                         const void* w_v, const void* w_o, const void* norm2, const void* w_gate,
                         const void* w_up, const void* w_down, void* y, int64_t B, int64_t N,
                         int64_t D, int64_t H, int64_t H_q, int64_t H_kv, int64_t F,
                         float rope_base, float scale, float eps, int causal, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable name of a status code. Never NULL. */
const char* sqa_status_str(int status);

/* Detail of the last error raised on the calling thread ("" if none).
 * The pointer stays valid until the next libsqa call on that thread. */
const char* sqa_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int sqa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SQA_H_ */
