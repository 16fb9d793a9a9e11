// SQA attention forward, fp32 in/out, head dim 16, dense batches: the
// matrix-pipe path of the fp32 attention (attn_fwd_f32.hip dispatches the
// SQAT-m attention core here). Same operation as every attention kernel:
// query head i attends K/V head floor(i*H_kv/H_q) ("GQA ..." page, "The
// idea"; SQA paper abstract), encoder-style or causal. It is a translation
// unit of its own: compiled next to the FMA-chain fp32 kernels, it changed
// the compiler's unrolling of those and made them twice as slow.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace sqa {
namespace {

struct Args32m {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int N, Hq, Hkv;
  int blocks_per_head;  // 32-row query blocks per (batch, head)
  float scale;
  int causal;
};

// d = 16, dense batches (the SQAT-m attention core): the dot products on the
// fp32 matrix pipe. v_mfma_f32_32x32x2_f32 forms exact fp32 products and
// adds them in fp32, so only the order of the additions differs from the
// FMA chains of attn_fwd_f32.hip. A workgroup takes 32 query rows of one (batch, head) and
// kMSplits waves; wave w streams key tiles w, w + kMSplits, ... of 32 keys
// (key rows read straight into the MFMA operand layout, one tile ahead),
// computes S^T = K Q^T (A = K, B = Q^T; lane l then holds 16 keys of query
// l % 32), an exact per-tile maximum and IEEE expf, and O^T += V^T P^T with
// P^T taken straight from the score accumulator (entry r of lane l is key
// 8(r/4) + 4(l/32) + r%4, so MFMA step r pairs keys 8(r/4) + r%4 and that
// plus 4). Head dims 16..31 of the 32-row O^T block are zero padding. The
// kMSplits partial (max, sum, O) states of each row are merged through LDS.
constexpr int kMSplits = 8;

__global__ __launch_bounds__(64 * kMSplits) void attn_fwd_f32_mfma16_kernel(Args32m a) {
  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  constexpr int D = 16;
  __shared__ float mrg[kMSplits][32][D + 2];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lg = lane >> 5;
  const int N = a.N;
  const int nqb = a.blocks_per_head;
  const int nbh = (int)(gridDim.x / nqb);
  // longest rows first under a causal mask: query block descending
  const int qb = a.causal ? nqb - 1 - (int)(blockIdx.x / nbh) : (int)(blockIdx.x % nqb);
  const int bh = a.causal ? (int)(blockIdx.x % nbh) : (int)(blockIdx.x / nqb);
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int kvh = (h * a.Hkv) / a.Hq;
  const int q0 = qb * 32;
  const int tq = min(q0 + l32, N - 1);  // this lane's query (rows past N: a copy of the last)

  // Q^T as B operand: step s of the d reduction takes dims 2s, 2s + 1;
  // lane l supplies Q[query][2s + l/32]
  float qv[8];
  {
    const f32x4_t* qr = reinterpret_cast<const f32x4_t*>(a.q + ((size_t)(b * a.Hq + h) * N + tq) * D);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4_t x = qr[c];
      qv[2 * c] = lg ? x[1] : x[0];
      qv[2 * c + 1] = lg ? x[3] : x[2];
    }
  }
  const float* kb = a.k + (size_t)(b * a.Hkv + kvh) * N * D;
  const float* vb = a.v + (size_t)(b * a.Hkv + kvh) * N * D;
  const int NT = (N + 31) / 32;
  const int nt = a.causal ? min(qb + 1, NT) : NT;

  // one tile's operands: K row of key key0 + l32 (A), and V[key(r)][l32] for
  // the 16 PV steps (A; zero for l32 >= 16)
  auto load = [&](int kt, float (&kv)[8], float (&vv)[16]) {
    const int key0 = kt * 32;
    const f32x4_t* kr = reinterpret_cast<const f32x4_t*>(kb + (size_t)min(key0 + l32, N - 1) * D);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4_t x = kr[c];
      kv[2 * c] = lg ? x[1] : x[0];
      kv[2 * c + 1] = lg ? x[3] : x[2];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = min(key0 + 8 * (r >> 2) + 4 * lg + (r & 3), N - 1);
      vv[r] = l32 < D ? vb[(size_t)key * D + l32] : 0.f;
    }
  };

  f32x16_t o;
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  float kv[8], vv[16], kn[8], vn[16];
  if (w < nt) load(w, kv, vv);
  for (int kt = w; kt < nt; kt += kMSplits) {
    if (kt + kMSplits < nt) load(kt + kMSplits, kn, vn);
    const int key0 = kt * 32;
    f32x16_t sc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st) sc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[st], qv[st], sc, 0, 0, 0);
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + 4 * lg + (r & 3);
      const bool ok = key < N && (!a.causal || key <= tq);
      sc[r] = ok ? sc[r] * a.scale : -INFINITY;
      mt = fmaxf(mt, sc[r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));  // the query's other 16 keys
    const float mnew = fmaxf(m, mt);      // finite: key0 <= tq is always visible
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - mnew);
    m = mnew;
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc[r] = expf(sc[r] - m);
      ps += sc[r];
    }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) o = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[r], sc[r], o, 0, 0, 0);
    if (kt + kMSplits < nt) {
#pragma unroll
      for (int c = 0; c < 8; ++c) kv[c] = kn[c];
#pragma unroll
      for (int r = 0; r < 16; ++r) vv[r] = vn[r];
    }
  }

  // this wave's partial state of query l32: O^T entry i is head dim
  // 8(i/4) + 4(l/32) + i%4 (entries 0..7 hold dims 0..15)
  const float ltot = lsum + __shfl_xor(lsum, 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) mrg[w][l32][8 * (i >> 2) + 4 * lg + (i & 3)] = o[i];
  if (lg == 0) {
    mrg[w][l32][D] = m;
    mrg[w][l32][D + 1] = ltot;
  }
  __syncthreads();
  // merge: one (query, head dim) per thread
  const int q = (int)threadIdx.x >> 4, d = (int)threadIdx.x & 15;
  if (q0 + q >= N) return;
  float M = -INFINITY;
#pragma unroll
  for (int x = 0; x < kMSplits; ++x) M = fmaxf(M, mrg[x][q][D]);
  float L = 0.f, acc = 0.f;
#pragma unroll
  for (int x = 0; x < kMSplits; ++x) {
    const float mx = mrg[x][q][D];
    if (mx == -INFINITY) continue;  // a wave with no key tile
    const float wt = expf(mx - M);
    L = fmaf(mrg[x][q][D + 1], wt, L);
    acc = fmaf(mrg[x][q][d], wt, acc);
  }
  const size_t row = (size_t)(b * a.Hq + h) * N + q0 + q;
  a.o[row * D + d] = acc / L;
  if (a.lse != nullptr && d == 0) a.lse[row] = M + logf(L);
}

}  // namespace

hipError_t launch_attn_fwd_f32_mfma16(const AttnProblem& p, hipStream_t stream) {
  Args32m a;
  a.q = static_cast<const float*>(p.q);
  a.k = static_cast<const float*>(p.k);
  a.v = static_cast<const float*>(p.v);
  a.o = static_cast<float*>(p.o);
  a.lse = p.lse;
  a.N = (int)p.N;
  a.Hq = (int)p.Hq;
  a.Hkv = (int)p.Hkv;
  a.blocks_per_head = (int)((p.N + 31) / 32);
  a.scale = p.scale;
  a.causal = p.causal;
  const int64_t nblk = (int64_t)a.blocks_per_head * p.B * p.Hq;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  if (p.dry_run) return hipSuccess;
  hipLaunchKernelGGL(attn_fwd_f32_mfma16_kernel, dim3((unsigned)nblk), dim3(64 * kMSplits), 0, stream, a);
  return hipGetLastError();
}


}  // namespace sqa
