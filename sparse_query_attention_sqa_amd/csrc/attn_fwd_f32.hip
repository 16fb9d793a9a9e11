// SQA attention forward with fp32 inputs, outputs and arithmetic throughout
// (no reduced-precision step). Same operation as the bf16 kernel: query head
// i attends K/V head floor(i*H_kv/H_q) ("GQA ..." page, "The idea"; SQA paper
// abstract), encoder-style or causal.
//
// One thread owns one query row; a workgroup is 256 consecutive positions of
// one (batch, query head). K/V are staged through LDS in 64-key tiles. For
// each tile a thread computes its 64 scores, raises its running maximum once,
// rescales its output accumulator, then accumulates exp(s - m) * v. This path
// serves the small fp32 configurations (d = 16 at N = 1024); it is VALU-bound
// by design and uses IEEE expf.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace sqa {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;

struct Args32 {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int N, Hq, Hkv, g;
  int blocks_per_head;
  float scale;
  int causal;
};

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(Args32 a) {
  __shared__ float ks[kTile][D];
  __shared__ float vs[kTile][D];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / a.blocks_per_head;       // b * Hq + h
  const int blk = blockIdx.x % a.blocks_per_head;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int kvh = h / a.g;
  const int N = a.N;
  const int t = blk * kThreads + tid;
  const bool valid = t < N;
  const int tq = min(t, N - 1);

  const float* qrow = a.q + ((size_t)bh * N + tq) * D;
  const float* kbase = a.k + ((size_t)b * a.Hkv + kvh) * (size_t)N * D;
  const float* vbase = a.v + ((size_t)b * a.Hkv + kvh) * (size_t)N * D;

  float qv[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qv[c] = qrow[c];
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  const int last_row = min(N - 1, blk * kThreads + kThreads - 1);
  const int nkeys = a.causal ? last_row + 1 : N;
  const int ntiles = (nkeys + kTile - 1) / kTile;
  const int my_end = a.causal ? tq + 1 : N;  // keys [0, my_end) are visible

  for (int kt = 0; kt < ntiles; ++kt) {
    const int key0 = kt * kTile;
    __syncthreads();
    for (int e = tid; e < kTile * D; e += kThreads) {
      const int r = e / D, c = e % D;
      const int row = min(key0 + r, N - 1);
      ks[r][c] = kbase[(size_t)row * D + c];
      vs[r][c] = vbase[(size_t)row * D + c];
    }
    __syncthreads();
    if (key0 >= my_end) continue;
    const int cnt = min(kTile, my_end - key0);

    float s[kTile];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(qv[c], ks[j][c], dot);
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
    for (int j = 0; j < kTile; ++j) {
      const float p = (j < cnt) ? expf(s[j] - m) : 0.f;
      l += p;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(p, vs[j][c], acc[c]);
    }
  }

  if (!valid) return;
  const float inv = 1.0f / l;
  float* orow = a.o + ((size_t)bh * N + t) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) orow[c] = acc[c] * inv;
  if (a.lse != nullptr) a.lse[(size_t)bh * N + t] = m + logf(l);
}

template <int D>
hipError_t launch_d(const AttnProblem& p, hipStream_t stream) {
  Args32 a;
  a.q = static_cast<const float*>(p.q);
  a.k = static_cast<const float*>(p.k);
  a.v = static_cast<const float*>(p.v);
  a.o = static_cast<float*>(p.o);
  a.lse = p.lse;
  a.N = (int)p.N;
  a.Hq = (int)p.Hq;
  a.Hkv = (int)p.Hkv;
  a.g = (int)(p.Hq / p.Hkv);
  a.blocks_per_head = (int)((p.N + kThreads - 1) / kThreads);
  a.scale = p.scale;
  a.causal = p.causal;
  const int64_t nblk = (int64_t)a.blocks_per_head * p.B * p.Hq;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_fwd_f32_kernel<D>, dim3((unsigned)nblk), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_f32(const AttnProblem& p, hipStream_t stream) {
  if (p.D == 16) return launch_d<16>(p, stream);
  if (p.D == 64) return launch_d<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace sqa
