// SQA attention forward with fp32 inputs, outputs and arithmetic throughout
// (no reduced-precision step). Same operation as the bf16 kernels: query head
// i attends K/V head floor(i*H_kv/H_q) ("GQA ..." page, "The idea"; SQA paper
// abstract), encoder-style or causal.
//
// This path serves small fp32 workloads (the SQAT-m attention core: d = 16,
// N = 1024, 8 query heads), where one thread per query row would leave most
// of the GPU idle. A workgroup therefore takes RB query rows of one
// (batch, head) and splits each row's keys over S threads: thread
// (row r, split s) takes keys s, s + S, s + 2S, ... and runs an exact fp32
// streaming softmax over them (per key tile: scores, tile maximum, rescale,
// accumulate, IEEE expf); the S partial (max, sum, output) triples of a row
// are merged through LDS at the end. K/V stream through LDS in tiles of TK
// keys, loaded cooperatively (16 bytes per thread, one tile ahead in
// registers), so every key row is fetched once per workgroup and the
// threads wait on one load per tile instead of a chain of row loads.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"
#include "seq_groups.h"

namespace sqa {
namespace {

constexpr int kThreads = 256;
constexpr int kKeyTile = 16;

struct Args32 {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  const int* cu;  // packed sequence offsets (nullptr: dense)
  int64_t T;      // packed: total tokens
  int N, Hq, Hkv;
  int blocks_per_head;  // for the longest sequence
  float scale;
  int causal;
};

template <int D>
struct F32Tile {
  static constexpr int TK = D <= 32 ? 64 : 2048 / D;     // keys per tile
  static constexpr int kFloats = 2 * TK * D;                // K then V
  static constexpr int kLoads = kFloats / 4 / kThreads;     // float4 per thread
  static_assert(kFloats % (4 * kThreads) == 0, "whole float4 loads per thread");
};

template <int D, int S>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(Args32 a) {
  using T = F32Tile<D>;
  constexpr int TK = T::TK;
  constexpr int RB = kThreads / S;  // query rows per workgroup
  constexpr int KPT = TK / S;       // keys per thread and tile
  static_assert(TK % S == 0, "whole keys per thread");
  // the key tiles and, after the last one, the S partial states of each row
  constexpr int kTiles = 2 * T::kFloats, kPart = S * RB * (D + 2);
  __shared__ __attribute__((aligned(16))) float smem[kTiles > kPart ? kTiles : kPart];
  float* const tile0 = smem;
  float* const tile1 = smem + T::kFloats;
  auto part = [&](int x, int row) { return smem + ((size_t)x * RB + row) * (D + 2); };

  const int tid = threadIdx.x;
  const int r = tid % RB, sp = tid / RB;
  const int bh = blockIdx.x / a.blocks_per_head;  // b * Hq + h
  const int blk = blockIdx.x % a.blocks_per_head;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int kvh = (h * a.Hkv) / a.Hq;
  const SeqGeom sg = seq_geom(a.cu, a.T, a.N, b, a.Hq, a.Hkv);
  const int N = sg.n;
  if (blk * RB >= N) return;  // past this sequence's rows (whole workgroup)
  const int t = blk * RB + r;
  const bool valid = t < N;
  const int tq = min(t, N - 1);

  const int64_t qrow0 = sg.q_base + (int64_t)h * sg.stride;
  const int64_t kvrow0 = sg.kv_base + (int64_t)kvh * sg.stride;
  const float* qrow = a.q + ((size_t)qrow0 + tq) * D;
  const float* kbase = a.k + (size_t)kvrow0 * D;
  const float* vbase = a.v + (size_t)kvrow0 * D;

  float qv[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qv[c] = qrow[c];
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  // keys of this row: [0, kend); of the workgroup: [0, wend)
  const int kend = a.causal ? tq + 1 : N;
  const int wend = a.causal ? min(blk * RB + RB, N) : N;
  const int ntiles = (wend + TK - 1) / TK;

  // tile loads: float4 index e of a tile -> K (e < TK*D/4) or V, key row
  // clamped into [0, N)
  float4 stage[T::kLoads];
  auto load = [&](int key0) {
#pragma unroll
    for (int i = 0; i < T::kLoads; ++i) {
      const int e = tid + i * kThreads;
      const bool isv = e >= TK * D / 4;
      const int e2 = isv ? e - TK * D / 4 : e;
      const int key = min(key0 + e2 / (D / 4), N - 1);
      const float* src = (isv ? vbase : kbase) + (size_t)key * D + (e2 % (D / 4)) * 4;
      stage[i] = *reinterpret_cast<const float4*>(src);
    }
  };
  auto store = [&](float* dst) {
#pragma unroll
    for (int i = 0; i < T::kLoads; ++i)
      reinterpret_cast<float4*>(dst)[tid + i * kThreads] = stage[i];
  };
  load(0);
  store(tile0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int key0 = kt * TK;
    if (kt + 1 < ntiles) load(key0 + TK);
    const float* kt_k = (kt & 1) ? tile1 : tile0;
    const float* kt_v = kt_k + TK * D;
    float s[KPT];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int j = sp + i * S;  // key within the tile
      const float* kr = kt_k + j * D;
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(qv[c], kr[c], dot);
      s[i] = dot * a.scale;
      if (key0 + j < kend) mt = fmaxf(mt, s[i]);
    }
    if (mt != -INFINITY) {
      const float mnew = fmaxf(m, mt);
      const float alpha = (m == -INFINITY) ? 0.f : expf(m - mnew);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] *= alpha;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int j = sp + i * S;
        if (key0 + j < kend) {
          const float p = expf(s[i] - m);
          const float* vr = kt_v + j * D;
          l += p;
#pragma unroll
          for (int c = 0; c < D; ++c) acc[c] = fmaf(p, vr[c], acc[c]);
        }
      }
    }
    if (kt + 1 < ntiles) store((kt & 1) ? tile0 : tile1);
    __syncthreads();  // (after the last tile: the tiles are free for the merge)
  }

  // merge the S partial softmax states of each row
#pragma unroll
  for (int c = 0; c < D; ++c) part(sp, r)[c] = acc[c];
  part(sp, r)[D] = m;
  part(sp, r)[D + 1] = l;
  __syncthreads();
  if (sp != 0 || !valid) return;
  float M = -INFINITY;
#pragma unroll
  for (int x = 0; x < S; ++x) M = fmaxf(M, part(x, r)[D]);
  float L = 0.f;
  float out[D];
#pragma unroll
  for (int c = 0; c < D; ++c) out[c] = 0.f;
#pragma unroll
  for (int x = 0; x < S; ++x) {
    const float mx = part(x, r)[D];
    if (mx == -INFINITY) continue;  // empty split
    const float w = expf(mx - M);
    L = fmaf(part(x, r)[D + 1], w, L);
#pragma unroll
    for (int c = 0; c < D; ++c) out[c] = fmaf(part(x, r)[c], w, out[c]);
  }
  const float inv = 1.0f / L;
  float* orow = a.o + ((size_t)qrow0 + t) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) orow[c] = out[c] * inv;
  if (a.lse != nullptr) a.lse[(size_t)qrow0 + t] = M + logf(L);
}

template <int D, int S>
hipError_t launch_d(const AttnProblem& p, hipStream_t stream) {
  constexpr int RB = kThreads / S;
  Args32 a;
  a.q = static_cast<const float*>(p.q);
  a.k = static_cast<const float*>(p.k);
  a.v = static_cast<const float*>(p.v);
  a.o = static_cast<float*>(p.o);
  a.lse = p.lse;
  a.cu = p.cu_seqlens;
  a.T = p.T;
  a.N = (int)p.N;
  a.Hq = (int)p.Hq;
  a.Hkv = (int)p.Hkv;
  a.blocks_per_head = (int)((p.N + RB - 1) / RB);
  a.scale = p.scale;
  a.causal = p.causal;
  const int64_t nblk = (int64_t)a.blocks_per_head * p.B * p.Hq;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  if (p.dry_run) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, S>), dim3((unsigned)nblk), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_f32(const AttnProblem& p, hipStream_t stream) {
  if (p.tail_split > 1 || p.nsplit > 1) return hipErrorInvalidValue;
  // d = 16 packed batches: 16 splits per row (on the SQAT-m core, before it
  // moved to the matrix pipe, four waves per SIMD instead of one: 40 -> 36
  // us; 8 and 32 splits were slower)
  // d = 16 dense: the fp32 matrix pipe (SQAT-m core; attn_fwd_f32_mfma.hip)
  if (p.D == 16 && p.cu_seqlens == nullptr) return launch_attn_fwd_f32_mfma16(p, stream);
  if (p.D == 16) return launch_d<16, 16>(p, stream);
  if (p.D == 32) return launch_d<32, 8>(p, stream);
  if (p.D == 64) return launch_d<64, 4>(p, stream);
  if (p.D == 128) return launch_d<128, 4>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace sqa
