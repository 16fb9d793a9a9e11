// SQA attention forward with fp32 inputs, outputs and arithmetic throughout
// (no reduced-precision step). Same operation as the bf16 kernels: query head
// i attends K/V head floor(i*H_kv/H_q) ("GQA ..." page, "The idea"; SQA paper
// abstract), encoder-style or causal.
//
// This path serves small fp32 workloads (the SQAT-m attention core: d = 16,
// N = 1024, 8 query heads), where one thread per query row would leave most
// of the GPU idle. A workgroup therefore takes RB query rows of one
// (batch, head) and splits each row's key range over S threads: thread
// (row r, split s) runs an exact fp32 streaming softmax over its keys
// (16-key tiles: scores, tile maximum, rescale, accumulate, IEEE expf), then
// the S partial (max, sum, output) triples of a row are merged through LDS.
// K/V rows are read straight from global memory; all threads of a split read
// the same key at the same time, so those reads are broadcasts from cache.
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

template <int D, int S>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(Args32 a) {
  constexpr int RB = kThreads / S;  // query rows per workgroup
  __shared__ float part[S][RB][D + 2];

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

  // this thread's keys: [lo, hi)
  const int chunk = (N + S - 1) / S;
  const int kend = a.causal ? tq + 1 : N;
  const int lo = sp * chunk;
  const int hi = min(lo + chunk, kend);

  for (int key0 = lo; key0 < hi; key0 += kKeyTile) {
    const int cnt = min(kKeyTile, hi - key0);
    float s[kKeyTile];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeyTile; ++j) {
      const float* kr = kbase + (size_t)min(key0 + j, N - 1) * D;
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(qv[c], kr[c], dot);
      s[j] = dot * a.scale;
      if (j < cnt) mt = fmaxf(mt, s[j]);
    }
    const float mnew = fmaxf(m, mt);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - mnew);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeyTile; ++j) {
      if (j < cnt) {
        const float p = expf(s[j] - m);
        const float* vr = vbase + (size_t)(key0 + j) * D;
        l += p;
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] = fmaf(p, vr[c], acc[c]);
      }
    }
  }

  // merge the S partial softmax states of each row
#pragma unroll
  for (int c = 0; c < D; ++c) part[sp][r][c] = acc[c];
  part[sp][r][D] = m;
  part[sp][r][D + 1] = l;
  __syncthreads();
  if (sp != 0 || !valid) return;
  float M = -INFINITY;
#pragma unroll
  for (int x = 0; x < S; ++x) M = fmaxf(M, part[x][r][D]);
  float L = 0.f;
  float out[D];
#pragma unroll
  for (int c = 0; c < D; ++c) out[c] = 0.f;
#pragma unroll
  for (int x = 0; x < S; ++x) {
    const float mx = part[x][r][D];
    if (mx == -INFINITY) continue;  // empty split
    const float w = expf(mx - M);
    L = fmaf(part[x][r][D + 1], w, L);
#pragma unroll
    for (int c = 0; c < D; ++c) out[c] = fmaf(part[x][r][c], w, out[c]);
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
  // d = 16 (the SQAT-m core: N = 1024, 8 query heads): 16 splits per row put
  // four waves on each SIMD instead of one (40 -> 36 us; 8 and 32: slower)
  if (p.D == 16) return launch_d<16, 16>(p, stream);
  if (p.D == 32) return launch_d<32, 8>(p, stream);
  if (p.D == 64) return launch_d<64, 4>(p, stream);
  if (p.D == 128) return launch_d<128, 4>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace sqa
