// Issue-rate probes for gfx950: measurement aids, not part of the attention
// path. They bound what the d = 64 forward kernel (attn_fwd_bf16_d64.hip)
// can reach with its per-tile instruction mix by running that mix, or parts
// of it, from registers only -- no HBM traffic, no ring of K/V tiles, no
// barriers -- on every compute unit with the forward's occupancy (4-wave
// workgroups, two per CU, so two waves per SIMD).
//
//   kind 0  MFMA only: per iteration 16 v_mfma_f32_32x32x16_bf16 in the
//           forward's dependency pattern (two 4-deep score chains, two pairs
//           of output accumulators), no VALU work: the matrix pipe's rate at
//           the clock the chip runs under this load.
//   kind 1  the forward's two-phase step from registers: per phase 8 MFMAs
//           (P.V of one 32-row half, S = K.Q of the other) interleaved with
//           the softmax of the half whose scores are ready -- 16 v_fma_f32,
//           16 v_exp_f32, 8 v_cvt_pk_bf16_f32, 8 v_dot2c_f32_bf16 and the
//           running-sum update and range check -- under the same
//           sched_group_barrier hints (one MFMA, six VALU).
//   kind 2  kind 1 plus the forward's LDS fragment reads per phase pair
//           (4 ds_read_b128 for K, 8 ds_read_b64_tr_b16 for V) from a tile
//           written once.
//   kind 3  v_exp_f32 only: 16 independent exponentials per lane and
//           iteration.
//   kind 4  v_fma_f32 only: 16 independent FMAs per lane and iteration.
//
// Each lane folds its results into one float stored to out[global thread]
// so that nothing is optimised away; the stored values are meaningless.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sqa_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;
constexpr int kTileBytes = 32 * kRowBytes;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
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

// softmax of one 32-row half against a fixed maximum, as in the forward
__device__ __forceinline__ float exp_half(const f32x16_t& s, u32x4_t (&pk)[2], float c, float m) {
  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  const float mneg = -m;
  float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * w], c, mneg));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * w + 1], c, mneg));
    const uint32_t pp = pack_bf16x2(p0, p1);
    pk[w >> 2][w & 3] = pp;
    if (w & 1) ls1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp), ones, ls1, false);
    else ls0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp), ones, ls0, false);
  }
  return ls0 + ls1;
}

__device__ __forceinline__ void interleave_phase() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
  }
}

// Makes a register value opaque to the optimiser (no instruction), so that
// loop-invariant MFMA operands are not hoisted out of the probe loops.
__device__ __forceinline__ void opaque(u32x4_t& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ u32x4_t seed4(int lane, int i) {
  const uint32_t b = 0x3f803f80u ^ (uint32_t)((lane * 7 + i * 13) & 0x7f);
  return u32x4_t{b, b ^ 0x10u, b ^ 0x20u, b ^ 0x30u};
}

__global__ __launch_bounds__(kThreads, 2) void probe_mfma_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  u32x4_t q[2][4], kf[4], vf[2][2], pk[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q[0][i] = seed4(lane, i);
    q[1][i] = seed4(lane, i + 4);
    kf[i] = seed4(lane, i + 8);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    vf[i][0] = seed4(lane, 12 + i);
    vf[i][1] = seed4(lane, 14 + i);
    pk[i] = seed4(lane, 16 + i);
  }
  f32x16_t o[2][2], sA, sB;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[h][x][i] = 0.f;
  float chk = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      opaque(kf[i]);
      opaque(q[0][i]);
      opaque(q[1][i]);
    }
    mfma_pv(vf, pk, o[1]);
    mfma_s(kf, q[1], sA);
    mfma_pv(vf, pk, o[0]);
    mfma_s(kf, q[0], sB);
    chk += sA[it & 15] + sB[(it + 3) & 15];
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) chk += o[0][0][i] + o[0][1][i] + o[1][0][i] + o[1][1][i];
  out[blockIdx.x * kThreads + threadIdx.x] = chk;
}

template <bool LDS>
__global__ __launch_bounds__(kThreads, 2) void probe_mix_kernel(int iters, float c, float* out) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2 * kTileBytes];
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, lg = lane >> 5;
  if (LDS) {
    for (int e = threadIdx.x; e < 2 * kTileBytes / 16; e += kThreads)
      reinterpret_cast<u32x4_t*>(tile)[e] = seed4(e & 63, e >> 6);
    __syncthreads();
  }
  uint32_t koff[4], voffr[2];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds)
    koff[ds] = (uint32_t)(l32 * kRowBytes + ((ds * 2 + lg) ^ ((l32 & 7) ^ ((l32 >> 3) & 1))) * 16);
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int j16 = lane & 15, g1 = (lane >> 4) & 1, row = lg * 16 + (j16 >> 2);
    voffr[x] = (uint32_t)(row * kRowBytes + (((x * 4 + 2 * g1 + ((j16 & 3) >> 1)) ^ (2 * (row & 3))) * 16) +
                          (j16 & 1) * 8);
  }
  u32x4_t q[2][4], kf[4], vf[2][2], pk0[2], pk1[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q[0][i] = seed4(lane, i);
    q[1][i] = seed4(lane, i + 4);
    kf[i] = seed4(lane, i + 8);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    vf[i][0] = seed4(lane, 12 + i);
    vf[i][1] = seed4(lane, 14 + i);
    pk0[i] = seed4(lane, 16 + i);
    pk1[i] = seed4(lane, 18 + i);
  }
  f32x16_t o[2][2], sA, sB;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[h][x][i] = 0.f;
  mfma_s(kf, q[0], sB);
  float m0 = 0.5f, m1 = 0.25f, l0 = 0.f, l1 = 0.f;
  const float lim = 1048576.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!LDS) opaque(kf[i]);
      opaque(q[0][i]);
      opaque(q[1][i]);
    }
    // phase A: P(h1).V and S(h1) on the matrix pipe, softmax of S(h0)
    mfma_pv(vf, pk1, o[1]);
    if (LDS) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint8_t* p = tile + kTileBytes + voffr[x] + hh * 8 * kRowBytes;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * kRowBytes));
          const u32x2_t a = __builtin_bit_cast(u32x2_t, lo);
          const u32x2_t b = __builtin_bit_cast(u32x2_t, hi);
          vf[x][hh] = u32x4_t{a[0], a[1], b[0], b[1]};
        }
    }
    mfma_s(kf, q[1], sA);
    if (LDS) {
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) kf[ds] = *reinterpret_cast<const u32x4_t*>(tile + koff[ds]);
    }
    float ls = exp_half(sB, pk0, c, m0);
    interleave_phase();
    if (__ballot(!(ls <= lim))) m0 += 1.0f;  // the forward's range check (never taken here)
    l0 += ls;
    // phase B: P(h0).V and S(h0) on the matrix pipe, softmax of S(h1)
    mfma_pv(vf, pk0, o[0]);
    mfma_s(kf, q[0], sB);
    ls = exp_half(sA, pk1, c, m1);
    interleave_phase();
    if (__ballot(!(ls <= lim))) m1 += 1.0f;
    l1 += ls;
  }
  float chk = l0 + l1 + m0 + m1;
#pragma unroll
  for (int i = 0; i < 16; ++i) chk += o[0][0][i] + o[0][1][i] + o[1][0][i] + o[1][1][i];
  out[blockIdx.x * kThreads + threadIdx.x] = chk;
}

__global__ __launch_bounds__(kThreads, 2) void probe_exp_kernel(int iters, float* out) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = -0.001f * (float)(i + (threadIdx.x & 7));
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
  float chk = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) chk += x[i];
  out[blockIdx.x * kThreads + threadIdx.x] = chk;
}

__global__ __launch_bounds__(kThreads, 2) void probe_fma_kernel(int iters, float c, float* out) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = 0.001f * (float)(i + (threadIdx.x & 7));
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = __builtin_fmaf(x[i], c, -0.5f);
  float chk = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) chk += x[i];
  out[blockIdx.x * kThreads + threadIdx.x] = chk;
}

}  // namespace

extern "C" {

int sqa_probe_threads(int workgroups) { return workgroups * kThreads; }

int sqa_probe_run(int kind, int workgroups, int iters, float* out, void* stream) {
  if (workgroups < 1 || iters < 1 || out == nullptr) return (int)hipErrorInvalidValue;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)workgroups), block(kThreads);
  const float c = 0.18033688f;  // |scale| * log2(e) at scale 1/8
  switch (kind) {
    case 0: hipLaunchKernelGGL(probe_mfma_kernel, grid, block, 0, st, iters, out); break;
    case 1: hipLaunchKernelGGL(probe_mix_kernel<false>, grid, block, 0, st, iters, c, out); break;
    case 2: hipLaunchKernelGGL(probe_mix_kernel<true>, grid, block, 0, st, iters, c, out); break;
    case 3: hipLaunchKernelGGL(probe_exp_kernel, grid, block, 0, st, iters, out); break;
    case 4: hipLaunchKernelGGL(probe_fma_kernel, grid, block, 0, st, iters, c, out); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
