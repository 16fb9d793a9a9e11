// SQA attention forward for head dim 64, bf16 in/out, gfx950: the
// software-pipelined kernel used for the long-sequence workloads.
//
// Same operation as attn_fwd_bf16.hip (query head i attends K/V head
// floor(i*H_kv/H_q), "GQA ..." page "The idea"; fewer query heads than the
// baseline, SQA paper abstract), same workgroup/slot decomposition and the
// same transposed MFMA formulation (S^T = K Q^T, O^T += V^T P^T with
// v_mfma_f32_32x32x16_bf16, K rows permuted in LDS, V stored transposed).
//
// What differs is the schedule. On gfx950 the softmax VALU work (one
// v_exp_f32 plus ~3 VALU ops per score) costs about as much issue time as the
// MFMA work per score at d = 64, and the two only overlap when independent
// VALU and MFMA instructions are interleaved in one instruction stream. Each
// wave's 64 query rows are therefore two 32-row halves h0/h1 in a two-phase
// pipeline over K/V tiles j:
//
//   phase A(j): MFMA  P(j-1,h1).V(j-1)   and  S(j,h1) = K(j).Q(h1)
//               VALU  softmax of S(j,h0)                 -> P(j,h0)
//   phase B(j): MFMA  P(j,h0).V(j)       and  S(j+1,h0) = K(j+1).Q(h0)
//               VALU  softmax of S(j,h1)                 -> P(j,h1)
//
// with 32-key tiles, so each phase has 8 MFMAs and the softmax of 32x32
// scores that do not depend on them. K/V tiles go HBM -> registers -> a
// 3-deep LDS ring with one barrier per tile; K(j) and V(j) fragments are read
// from LDS once per tile and kept in registers for both halves. The live set
// (~230 VGPRs) allows two waves per SIMD.
//
// The running maximum is raised lazily: probabilities are computed against
// the current maximum m, and only if a lane's sum of its 16 probabilities
// exceeds 2^20 (or is not finite -- always the case on the first tile, where
// m = -inf) is the exact row maximum taken, O and l rescaled and the tile's
// probabilities recomputed. Between refreshes every probability is <= 2^20,
// far inside the bf16/fp32 range, and the result equals the max-subtracted
// softmax up to rounding.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace sqa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int D = 64;
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 64;
constexpr int kTileKeys = 32;         // keys per K/V tile (one 32-row MFMA block)
constexpr int KROW = D + 8;            // bf16 elements per LDS row of K (144 B)
constexpr int VROW = kTileKeys + 8;    // bf16 elements per LDS row of V^T (80 B)
constexpr int KBUF = kTileKeys * KROW;
constexpr int VBUF = D * VROW;
constexpr int BUF = KBUF + VBUF;
constexpr int NBUF = 3;
constexpr int kXcds = 8;
constexpr float kSumLimit = 1048576.0f;  // 2^20
constexpr float kMaskedScore = -3.0e38f;
constexpr float kMinC = 1e-30f;          // |scale|*log2(e) is clamped up to this

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int N, Hq, Hkv, g;
  int TB;          // ceil(N / 64): 64-row query blocks per head
  int NT;          // ceil(N / 32): 32-key tiles
  int wg_per_bkv, n_bkv, nwg;
  float c;
  uint32_t qsign;
  int causal;
};

__device__ __forceinline__ int pi_inv(int p) { return ((p & 15) >> 2) * 8 + (p >> 4) * 4 + (p & 3); }
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

struct Staged {
  u32x4_t k;     // 8 d of one key
  u32x2_t v[2];  // 4 d of two consecutive keys
};

// HBM -> registers for tile kt (key rows clamped into [0, N)).
__device__ __forceinline__ void load_tile(Staged& r, const uint16_t* kbase, const uint16_t* vbase, int kt,
                                          int N, int tid) {
  const int key0 = kt * kTileKeys;
  {
    const int key = tid >> 3, dc = tid & 7;
    const int row = min(key0 + key, N - 1);
    r.k = *reinterpret_cast<const u32x4_t*>(kbase + (size_t)row * D + dc * 8);
  }
  const int kp = tid >> 4, dg = tid & 15;
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int row = min(key0 + 2 * kp + rr, N - 1);
    r.v[rr] = *reinterpret_cast<const u32x2_t*>(vbase + (size_t)row * D + dg * 4);
  }
}

// registers -> LDS: K rows under pi_inv; V transposed (2 keys x 4 d blocks).
__device__ __forceinline__ void store_tile(const Staged& r, uint16_t* buf, int tid) {
  uint16_t* ks = buf;
  uint16_t* vs = buf + KBUF;
  {
    const int key = tid >> 3, dc = tid & 7;
    *reinterpret_cast<u32x4_t*>(ks + pi_inv(key) * KROW + dc * 8) = r.k;
  }
  const int kp = tid >> 4, dg = tid & 15;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const int word = cc >> 1;
    const bool hi = cc & 1;
    const uint32_t e0 = hi ? (r.v[0][word] >> 16) : (r.v[0][word] & 0xffffu);
    const uint32_t e1 = hi ? (r.v[1][word] >> 16) : (r.v[1][word] & 0xffffu);
    const int d = dg * 4 + cc;
    const int lrow = (d & ~31) + pi_inv(d & 31);
    *reinterpret_cast<uint32_t*>(vs + lrow * VROW + 2 * kp) = e0 | (e1 << 16);
  }
}

// K(j) fragments (A operand of S^T): [ds]
__device__ __forceinline__ void read_k(const uint16_t* buf, u32x4_t (&kf)[4], int l32, int lg) {
#pragma unroll
  for (int ds = 0; ds < 4; ++ds)
    kf[ds] = *reinterpret_cast<const u32x4_t*>(buf + l32 * KROW + (ds * 2 + lg) * 8);
}

// V(j)^T fragments (A operand of O^T): [x][hh]
__device__ __forceinline__ void read_v(const uint16_t* buf, u32x4_t (&vf)[2][2], int l32, int lg) {
  const uint16_t* vs = buf + KBUF;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      vf[x][hh] = *reinterpret_cast<const u32x4_t*>(vs + (x * 32 + l32) * VROW + lg * 16 + hh * 8);
}

__device__ __forceinline__ void mfma_s(const u32x4_t (&kf)[4], const u32x4_t (&q)[4], f32x16_t& s) {
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int ds = 0; ds < 4; ++ds)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[ds]), as_bf16x8(q[ds]), acc, 0, 0, 0);
  s = acc;
}

__device__ __forceinline__ void mfma_pv(const u32x4_t (&vf)[2][2], const u32x4_t (&pk)[2], f32x16_t (&o)[2]) {
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int x = 0; x < 2; ++x)
      o[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[x][hh]), as_bf16x8(pk[hh]), o[x], 0, 0, 0);
}

// Scores of keys a query may not see (causal: key > t; ragged tail:
// key >= N) become kMaskedScore, whose probability underflows to exactly 0
// for any c >= kMinC. Only diagonal and tail tiles need this.
__device__ __forceinline__ void mask_scores(f32x16_t& s, int key0, int N, int causal, int t, int lg) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = key0 + lg * 16 + i;
    if (!(key < N && (!causal || key <= t))) s[i] = kMaskedScore;
  }
}

// probabilities of one 32-row half against the current maximum m, rounded to
// bf16 (nearest even) and packed as the B operand of O^T += V^T P^T; returns
// the lane's sum of its 16 rounded probabilities.
__device__ __forceinline__ float exp_half(const f32x16_t& s, u32x4_t (&pk)[2], float c, float m) {
  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  const float mneg = -m;
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * w], c, mneg));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * w + 1], c, mneg));
    const uint32_t pp = pack_bf16x2(p0, p1);
    pk[w >> 2][w & 3] = pp;
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp), ones, lsum, false);
  }
  return lsum;
}

// Finish the softmax of one half: if a lane's probabilities grew too large
// (or the running maximum was still -inf), take the exact row maximum,
// rescale O and l, and recompute the tile's probabilities.
__device__ __forceinline__ void finish_half(float lsum, const f32x16_t& s, u32x4_t (&pk)[2], float& m, float& l,
                                            f32x16_t (&o)[2], float c) {
  if (__ballot(!(lsum <= kSumLimit))) {
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    const float cand = mx * c;
    const float other = __shfl_xor(cand, 32);
    const float mnew = fmaxf(m, fmaxf(cand, other));
    const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[x][i] *= alpha;
    lsum = exp_half(s, pk, c, m);
  }
  l += lsum;
}

// Scheduling hints for one pipeline phase: 8 MFMAs, each followed by 6 VALU
// instructions of the independent softmax work.
__device__ __forceinline__ void interleave_phase() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
  }
}

__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_d64_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[NBUF * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lg = lane >> 5;

  int L;
  if (!a.causal) {
    const int bid = blockIdx.x;
    const int per = a.nwg / kXcds, rem = a.nwg % kXcds;
    const int x = bid % kXcds, i = bid / kXcds;
    L = x * per + min(x, rem) + i;
  } else {
    L = blockIdx.x;
  }
  int bkv, w_in;
  if (!a.causal) {
    bkv = L / a.wg_per_bkv;
    w_in = L % a.wg_per_bkv;
  } else {
    const int wr = L / a.n_bkv;
    bkv = L % a.n_bkv;
    w_in = a.wg_per_bkv - 1 - wr;
  }
  const int b = bkv / a.Hkv, kvh = bkv % a.Hkv;
  const int slot = w_in * kWaves + wave;
  const int tb = slot / a.g, jh = slot % a.g;
  const bool wave_valid = tb < a.TB;
  const int h = kvh * a.g + jh;
  const int N = a.N;
  // key tiles the workgroup streams, and the last one this wave computes
  // (-1: none). A causal wave's rows end at key tile 2*tb+1.
  const int maxtb = min((w_in * kWaves + kWaves - 1) / a.g, a.TB - 1);
  const int nt = a.causal ? min(2 * maxtb + 2, a.NT) : a.NT;
  const int last = !wave_valid ? -1 : (a.causal ? min(2 * tb + 1, a.NT - 1) : a.NT - 1);
  const int trow0 = tb * kRowsPerWave;

  const uint16_t* kbase = a.k + (size_t)bkv * N * D;
  const uint16_t* vbase = a.v + (size_t)bkv * N * D;
  const size_t qoff = ((size_t)b * a.Hq + h) * (size_t)N * D;

  u32x4_t qf[2][4];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int t = min(trow0 + qs * 32 + l32, N - 1);
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (wave_valid) x = *reinterpret_cast<const u32x4_t*>(a.q + qoff + (size_t)t * D + (ds * 2 + lg) * 8);
      x ^= a.qsign;
      qf[qs][ds] = x;
    }
  }

  f32x16_t acc_o[2][2];  // [half][x]
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_o[hh][x][i] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  const float c = a.c;
  const int t0 = trow0 + l32, t1 = trow0 + 32 + l32;

  // prologue: tiles 0 and 1 resident, tile 2 in flight, S(0,h0) issued
  Staged st;
  load_tile(st, kbase, vbase, 0, N, tid);
  store_tile(st, smem, tid);
  if (nt > 1) {
    load_tile(st, kbase, vbase, 1, N, tid);
    store_tile(st, smem + BUF, tid);
  }
  if (nt > 2) load_tile(st, kbase, vbase, 2, N, tid);
  __syncthreads();

  u32x4_t kf[4];
  u32x4_t vf[2][2];
  f32x16_t sA, sB;
  u32x4_t pk0[2], pk1[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    pk1[x] = u32x4_t{0u, 0u, 0u, 0u};  // P(-1,h1) = 0: the first phase A's P.V is a no-op
    vf[x][0] = u32x4_t{0u, 0u, 0u, 0u};
    vf[x][1] = u32x4_t{0u, 0u, 0u, 0u};
  }
  read_k(smem, kf, l32, lg);
  mfma_s(kf, qf[0], sB);

  for (int j = 0; j < nt; ++j) {
    const uint16_t* bj = smem + (j % NBUF) * BUF;
    const uint16_t* bn = smem + ((j + 1) % NBUF) * BUF;
    const int key0 = j * kTileKeys;
    const bool active = j <= last;
    const bool masked = (a.causal && j >= 2 * tb) || (key0 + kTileKeys > N);

    // ---------------- phase A(j)
    if (active) {
      if (masked) mask_scores(sB, key0, N, a.causal, t0, lg);
      mfma_pv(vf, pk1, acc_o[1]);    // P(j-1,h1) V(j-1)
      read_v(bj, vf, l32, lg);       // V(j), used from phase B on
      mfma_s(kf, qf[1], sA);         // S(j,h1); K(j) is in kf
      const float ls = exp_half(sB, pk0, c, m_run[0]);
      interleave_phase();
      finish_half(ls, sB, pk0, m_run[0], l_run[0], acc_o[0], c);
    }

    __syncthreads();  // every wave is done with tile j-1's buffer
    if (j + 2 < nt) {
      store_tile(st, smem + ((j + 2) % NBUF) * BUF, tid);
      if (j + 3 < nt) load_tile(st, kbase, vbase, j + 3, N, tid);
    }

    // ---------------- phase B(j); S(j+1,h0) is computed even past the
    // wave's last tile (then unused), so the phase stays branch-free.
    if (active) {
      if (masked) mask_scores(sA, key0, N, a.causal, t1, lg);
      read_k(bn, kf, l32, lg);       // K(j+1)
      mfma_pv(vf, pk0, acc_o[0]);    // P(j,h0) V(j)
      mfma_s(kf, qf[0], sB);         // S(j+1,h0)
      const float ls = exp_half(sA, pk1, c, m_run[1]);
      interleave_phase();
      finish_half(ls, sA, pk1, m_run[1], l_run[1], acc_o[1], c);
    }
  }
  if (last >= 0) mfma_pv(vf, pk1, acc_o[1]);  // drain P(last,h1) V(last)

  if (!wave_valid) return;

#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const float ltot = l_run[qs] + __shfl_xor(l_run[qs], 32);
    const float inv = 1.0f / ltot;
    const int t = trow0 + qs * 32 + l32;
    if (t < N) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int d0 = x * 32 + lg * 16;
        u32x4_t w0, w1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w0[e] = pack_bf16x2(acc_o[qs][x][2 * e] * inv, acc_o[qs][x][2 * e + 1] * inv);
          w1[e] = pack_bf16x2(acc_o[qs][x][8 + 2 * e] * inv, acc_o[qs][x][8 + 2 * e + 1] * inv);
        }
        uint16_t* dst = a.o + qoff + (size_t)t * D + d0;
        *reinterpret_cast<u32x4_t*>(dst) = w0;
        *reinterpret_cast<u32x4_t*>(dst + 8) = w1;
      }
      if (a.lse != nullptr && lg == 0)
        a.lse[((size_t)b * a.Hq + h) * (size_t)N + t] = (m_run[qs] + log2f(ltot)) * 0.69314718055994531f;
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16_d64(const AttnProblem& p, hipStream_t stream) {
  if (p.D != D) return hipErrorInvalidValue;
  Args a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.o = static_cast<uint16_t*>(p.o);
  a.lse = p.lse;
  a.N = (int)p.N;
  a.Hq = (int)p.Hq;
  a.Hkv = (int)p.Hkv;
  a.g = (int)(p.Hq / p.Hkv);
  a.TB = (int)((p.N + kRowsPerWave - 1) / kRowsPerWave);
  a.NT = (int)((p.N + kTileKeys - 1) / kTileKeys);
  const int64_t slots = (int64_t)a.TB * a.g;
  a.wg_per_bkv = (int)((slots + kWaves - 1) / kWaves);
  a.n_bkv = (int)(p.B * p.Hkv);
  const int64_t nwg = (int64_t)a.wg_per_bkv * a.n_bkv;
  if (nwg > 0x7fffffff) return hipErrorInvalidValue;
  a.nwg = (int)nwg;
  a.c = fmaxf(fabsf(p.scale) * 1.4426950408889634f, kMinC);
  a.qsign = (p.scale < 0.f) ? 0x80008000u : 0u;
  a.causal = p.causal;
  hipLaunchKernelGGL(attn_fwd_bf16_d64_kernel, dim3(a.nwg), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sqa
