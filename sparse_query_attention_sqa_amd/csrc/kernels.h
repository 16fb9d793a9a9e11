// Internal launch interface between the C-ABI layer (sqa_api.cpp) and the
// HIP kernels. Not part of the public ABI; see include/sqa.h for that.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace sqa {

// SQA attention forward: q [B,Hq,N,D], k/v [B,Hkv,N,D], o [B,Hq,N,D],
// optional lse [B,Hq,N] fp32; 1 <= Hkv <= Hq (query head i reads K/V head
// floor(i*Hkv/Hq)). With cu_seqlens (device, B+1 int32 offsets) the tensors
// are packed instead: q/o [Hq,T,D], k/v [Hkv,T,D], lse [Hq,T], sequence b
// owning tokens cu[b] .. cu[b+1]-1, and N is the longest sequence. Sizes
// already validated.
struct AttnProblem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t B, Hq, Hkv, N, D;
  float scale;
  int causal;
  const int* cu_seqlens;  // nullptr: dense
  int64_t T;              // packed: total tokens
  // key-range splits (bf16, any supported d): nsplit > 1 needs split_ws of
  // attn_split_workspace_bytes(rows, D, nsplit) bytes, rows = B*Hq*N
  // (packed: Hq*T)
  int nsplit = 1;
  float* split_ws = nullptr;
  // tail split (d = 64, dense encoder-style, equal head groups, nsplit 1):
  // the last tail_units logical workgroups run as tail_split key ranges
  // each; tail_ws holds attn_tail_workspace_bytes(tail_units, tail_split)
  int tail_split = 0;
  int64_t tail_units = 0;
  float* tail_ws = nullptr;
  // dry_run: run every check of the launcher (sizes against the 32-bit
  // limits of grids, offsets and buffer descriptors) and launch nothing;
  // hipErrorInvalidValue then means the problem exceeds a launch limit
  bool dry_run = false;
};

size_t attn_split_workspace_bytes(int64_t rows, int64_t d, int nsplit);
// recommended nsplit for the d = 64 bf16 forward on a device with `cus` CUs
// (rows_per_wave: 64 for the d = 64 kernel, 32 for the d = 128 kernel; both
// run two 4-wave workgroups per CU over 32-key tiles)
int attn_fwd_auto_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t T, bool causal, int cus,
                         int rows_per_wave);
hipError_t launch_attn_fwd_bf16(const AttnProblem& p, hipStream_t stream);
// tail split plan of the d = 64 forward on a device with `cus` CUs: returns
// the key ranges per tail workgroup (0: none) and the tail workgroups
constexpr int kMaxTailSplit = 16;
int attn_fwd_tail_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, bool causal, int cus, int64_t* units);
size_t attn_tail_workspace_bytes(int64_t units, int S);
// head dim 16, unsplit, N*32 < 2^31 (attn_fwd_bf16_d16.hip)
hipError_t launch_attn_fwd_bf16_d16(const AttnProblem& p, hipStream_t stream);
// head dim 32, unsplit, N*64 < 2^31 (attn_fwd_bf16_d32.hip)
hipError_t launch_attn_fwd_bf16_d32(const AttnProblem& p, hipStream_t stream);
// head dim 64, software-pipelined (attn_fwd_bf16_d64.hip)
hipError_t launch_attn_fwd_bf16_d64(const AttnProblem& p, hipStream_t stream);
// head dim 128, software-pipelined (attn_fwd_bf16_d128.hip)
hipError_t launch_attn_fwd_bf16_d128(const AttnProblem& p, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const AttnProblem& p, hipStream_t stream);
// fp32, d = 16, dense (cu_seqlens == nullptr) on the fp32 matrix pipe
hipError_t launch_attn_fwd_f32_mfma16(const AttnProblem& p, hipStream_t stream);

// SQA attention backward (bf16, head dim 64 or 128): dq [B,Hq,N,D], dk/dv
// [B,Hkv,N,D] from q, k, v, the forward's o and lse, and dout (or the packed
// layouts with cu_seqlens, N the longest sequence). `rowterms` is device
// scratch of attn_bwd_rowterm_bytes(B, Hq, N) bytes (packed:
// attn_bwd_rowterm_bytes_packed(Hq, T)).
struct BwdProblem {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  void* rowterms;
  int64_t B, Hq, Hkv, N, D;
  float scale;
  int causal;
  const int* cu_seqlens;  // nullptr: dense; else packed as in AttnProblem
  int64_t T;              // packed: total tokens
  // range splits (encoder-style only): nsplit > 1 needs split_ws of
  // attn_bwd_split_bytes(q_rows, kv_rows, D, nsplit) bytes
  int nsplit = 1;
  float* split_ws = nullptr;
  bool dry_run = false;  // as in AttnProblem
};
size_t attn_bwd_split_bytes(int64_t q_rows, int64_t kv_rows, int64_t D, int nsplit);
// recommended nsplit for the backward on a device with `cus` CUs
int attn_bwd_auto_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t T, int64_t D, bool causal, int cus);
// packed batches: two splits when the longest sequence (N tokens of T) is long and holds a quarter of them
bool packed_wants_split(int64_t N, int64_t T);
size_t attn_bwd_rowterm_bytes(int64_t B, int64_t Hq, int64_t N);
size_t attn_bwd_rowterm_bytes_packed(int64_t Hq, int64_t T);
hipError_t launch_attn_bwd_bf16(const BwdProblem& p, hipStream_t stream);
// Fixed device buffer of the allocation-free backward: kNoAllocScratchBytes
// per GPU (room for the row terms of 4M padded query rows). noalloc_scratch
// returns its address on the current device.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void** ptr);

// Compute units of the current device (256 if the query fails), cached per
// device ordinal.
int device_cus();

// Projection + RoPE: x [M=B*N, Dm] bf16 times w_q [Dm,Hq*d] | w_k [Dm,Hkv*d] |
// w_v [Dm,Hkv*d]; writes q [B,Hq,N,d], k/v [B,Hkv,N,d] bf16 with RoPE applied
// to q and k.
struct QkvProblem {
  const void* x;
  const void* wq;
  const void* wk;
  const void* wv;
  void* q;
  void* k;
  void* v;
  int64_t B, N, Dm, Hq, Hkv, d;
  float rope_base;
  bool dry_run = false;  // as in AttnProblem
};
hipError_t launch_qkv_rope(const QkvProblem& p, hipStream_t stream);


// Output projection: y [B,N,Dm] = O_flat [B*N, Hq*d] times w_o [Hq*d, Dm],
// reading O from its [B,Hq,N,d] layout.
struct OprojProblem {
  const void* o;
  const void* wo;
  void* y;
  int64_t B, N, Dm, Hq, d;
  const void* resid;  // optional [B*N, Dm] added in the epilogue (nullptr: none)
  bool dry_run = false;  // as in AttnProblem
};
hipError_t launch_out_proj(const OprojProblem& p, hipStream_t stream);

// y [M, Ncols] = a [M, K] (row-major) times w [K, Ncols] (+ resid [M, Ncols]).
struct DenseProblem {
  const void* a;
  const void* w;
  const void* resid;  // nullable
  void* y;
  int64_t M, K, Ncols;
  bool dry_run = false;  // as in AttnProblem
};
hipError_t launch_dense_residual(const DenseProblem& p, hipStream_t stream);

// y = x / sqrt(mean(x^2) + eps) * g over rows of D (bf16 in/out).
hipError_t launch_rms_norm(const void* x, const void* g, void* y, int64_t M, int64_t D, float eps,
                           hipStream_t stream, bool dry_run = false);

// h [M, F] = silu(z w_gate) * (z w_up); z [M, K], w_gate / w_up [K, F].
struct GateUpProblem {
  const void* z;
  const void* w_gate;
  const void* w_up;
  void* h;
  int64_t M, K, F;
  bool dry_run = false;  // as in AttnProblem
};
hipError_t launch_gate_up(const GateUpProblem& p, hipStream_t stream);

}  // namespace sqa
