// Projection GEMMs of one SQA layer (SQAT-m model card, "Architecture
// details" and "Model size difference"): the query and output projections are
// H_q*d wide, the key/value projections H_kv*d wide, with d = d_model / H.
//
//   rope_table : (cos, sin) of t*base^(-2c/d) for every position t and pair c,
//              the angle formed and reduced modulo 2*pi in fp64.
//   qkv_rope : [B*N, Dm] x [W_q | W_k | W_v] -> Q [B,Hq,N,d], K/V [B,Hkv,N,d]
//              with rotary position embedding applied to Q and K in the
//              epilogue (rotate-half pairs (c, c+d/2)), reading the table.
//   out_proj : O_flat [B*N, Hq*d] x W_o -> Y [B, N, Dm], reading O in its
//              [B, Hq, N, d] attention layout (no separate transpose pass);
//              also a plain row-major A (the feed-forward down projection),
//              with an optional residual added in the epilogue.
//
// Block extras (SQAT-m card, "Architecture details": RMS Norm, SwiGLU feed
// forward with 768 dim):
//   rms_norm  : y = x / sqrt(mean(x^2) + eps) * g per row, fp32 math.
//   gate_up   : h = silu(z W_gate) * (z W_up), both products from one A tile
//               row block, the SwiGLU combination fused in the epilogue.
//
// Both are bf16 MFMA GEMMs (v_mfma_f32_32x32x16_bf16, fp32 accumulate) with a
// 64x64 output tile per 4-wave workgroup (2x2 waves of 32x32). The reduction
// runs in 64-wide chunks staged in LDS; the weight chunk is stored transposed
// so that both MFMA operands are single 16-byte LDS reads. Rows, columns and
// the reduction length are masked, so any B*N and any multiple of 16 for the
// widths work.
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

constexpr int kThreads = 256;
constexpr int BM = 64, BN = 64, KC = 64;
constexpr int PITCH = KC + 8;   // bf16 elements per LDS row (144 bytes)
constexpr int CPITCH = BN + 4;  // fp32 elements per epilogue row
constexpr int kMaxHalf = 32;    // d/2 <= 32

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

struct Theta {
  double v[kMaxHalf];
};

// Source of the A operand rows: either a row-major [M, K] matrix, or the
// attention output O [B, Hq, N, d] read as O_flat [B*N, Hq*d].
struct ASrc {
  const uint16_t* p;
  int64_t K;
  int gather;  // 1: O layout
  int64_t N, Hq, d;
  __device__ __forceinline__ const uint16_t* chunk(int64_t m, int64_t k) const {
    if (!gather) return p + m * K + k;
    const int64_t b = m / N, t = m % N;
    const int64_t h = k / d, c = k % d;
    return p + (((b * Hq + h) * N + t) * d + c);
  }
};

// Column n of the concatenated weight [W_q | W_k | W_v] (or of W_o).
struct WSrc {
  const uint16_t* w[3];
  int64_t ncol[3];  // columns of each part
  __device__ __forceinline__ uint32_t pair(int64_t k, int64_t n) const {
    // two adjacent columns n, n+1 (same part: parts have even widths)
    int part = 0;
    int64_t nn = n;
    if (nn >= ncol[0]) { nn -= ncol[0]; part = 1;
      if (nn >= ncol[1]) { nn -= ncol[1]; part = 2; } }
    return *reinterpret_cast<const uint32_t*>(w[part] + k * ncol[part] + nn);
  }
};

// Shared GEMM core: acc (per wave 32x32) for output tile (m0, n0).
__device__ __forceinline__ void gemm_tile(const ASrc& A, const WSrc& W, int64_t M, int64_t Ncols,
                                          int64_t K, int64_t m0, int64_t n0, uint16_t* as_,
                                          uint16_t* ws_, f32x16_t& acc) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lg = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

  for (int64_t k0 = 0; k0 < K; k0 += KC) {
    // A chunk [64 rows][64 k]: 512 chunks of 8 bf16
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = tid + it * kThreads;
      const int r = c >> 3, kc = c & 7;
      const int64_t m = min(m0 + r, M - 1);
      const int64_t k = k0 + kc * 8;
      u32x4_t val = {0u, 0u, 0u, 0u};
      if (k < K) val = *reinterpret_cast<const u32x4_t*>(A.chunk(m, k));
      *reinterpret_cast<u32x4_t*>(as_ + r * PITCH + kc * 8) = val;
    }
    // W chunk [64 k][64 n] -> LDS W^T [64 n][64 k] via 4x4 blocks
    {
      const int kb = tid >> 4, nb = tid & 15;  // 16 x 16 blocks
      uint32_t lo[4], hi[4];                    // row kk: cols (n,n+1), (n+2,n+3)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int64_t k = k0 + kb * 4 + kk;
        const int64_t n = n0 + nb * 4;
        lo[kk] = 0u;
        hi[kk] = 0u;
        if (k < K && n < Ncols) {
          lo[kk] = W.pair(k, n);
          hi[kk] = W.pair(k, n + 2);
        }
      }
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        uint32_t e[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint32_t wv = (cc < 2) ? lo[kk] : hi[kk];
          e[kk] = (cc & 1) ? (wv >> 16) : (wv & 0xffffu);
        }
        u32x2_t out;
        out[0] = e[0] | (e[1] << 16);
        out[1] = e[2] | (e[3] << 16);
        *reinterpret_cast<u32x2_t*>(ws_ + (nb * 4 + cc) * PITCH + kb * 4) = out;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KC; kk += 16) {
      const bf16x8_t af = as_bf16x8(*reinterpret_cast<const u32x4_t*>(as_ + (wm * 32 + l32) * PITCH + kk + lg * 8));
      const bf16x8_t bf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(ws_ + (wn * 32 + l32) * PITCH + kk + lg * 8));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
    }
    __syncthreads();
  }
}

// acc -> LDS fp32 tile [64][CPITCH]
__device__ __forceinline__ void spill_acc(const f32x16_t& acc, float* cs) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lg = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = wm * 32 + 8 * (i >> 2) + lg * 4 + (i & 3);
    cs[r * CPITCH + wn * 32 + l32] = acc[i];
  }
  __syncthreads();
}

struct QkvArgs {
  const float* cs;  // [N, d/2] (cos, sin)
  ASrc A;
  WSrc W;
  uint16_t* out[3];
  int64_t M, Ncols, K, N, Hq, Hkv, d;
  int nblk_n;
};

__global__ __launch_bounds__(kThreads) void qkv_rope_kernel(QkvArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t as_[BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t ws_[BN * PITCH];
  __shared__ __attribute__((aligned(16))) float cs[BM * CPITCH];
  const int64_t m0 = (int64_t)(blockIdx.x / a.nblk_n) * BM;
  const int64_t n0 = (int64_t)(blockIdx.x % a.nblk_n) * BN;
  f32x16_t acc;
  gemm_tile(a.A, a.W, a.M, a.Ncols, a.K, m0, n0, as_, ws_, acc);
  spill_acc(acc, cs);

  const int tid = threadIdx.x;
  const int r = tid >> 2, cq = tid & 3;
  const int64_t m = m0 + r;
  const int64_t nstart = n0 + cq * 16;
  if (m >= a.M || nstart >= a.Ncols) return;
  const int64_t d = a.d, half = d / 2;
  int part;
  int64_t nl;
  if (nstart < a.Hq * d) { part = 0; nl = nstart; }
  else if (nstart < (a.Hq + a.Hkv) * d) { part = 1; nl = nstart - a.Hq * d; }
  else { part = 2; nl = nstart - (a.Hq + a.Hkv) * d; }
  const int64_t head = nl / d, c0 = nl % d;
  const int64_t b = m / a.N, t = m % a.N;
  const int64_t nheads = (part == 0) ? a.Hq : a.Hkv;
  const int lc0 = (int)(nstart - n0);           // local column of c0
  const int lbase = lc0 - (int)c0;              // local column of the head start
  float y[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int c = (int)c0 + e;
    const float x = cs[r * CPITCH + lc0 + e];
    if (part == 2) {
      y[e] = x;
    } else {
      const int kpair = c % (int)half;
      const float2 csv = *reinterpret_cast<const float2*>(a.cs + 2 * (t * half + kpair));
      const float cn = csv.x, sn = csv.y;
      if (c < half) {
        const float xp = cs[r * CPITCH + lbase + c + (int)half];
        y[e] = x * cn - xp * sn;
      } else {
        const float xp = cs[r * CPITCH + lbase + c - (int)half];
        y[e] = xp * sn + x * cn;
      }
    }
  }
  u32x4_t w0, w1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w0[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
    w1[e] = pack_bf16x2(y[8 + 2 * e], y[8 + 2 * e + 1]);
  }
  uint16_t* dst = a.out[part] + (((b * nheads + head) * a.N + t) * d + c0);
  *reinterpret_cast<u32x4_t*>(dst) = w0;
  *reinterpret_cast<u32x4_t*>(dst + 8) = w1;
}

struct OprojArgs {
  ASrc A;
  WSrc W;
  const uint16_t* resid;  // [M, Ncols] added before rounding, or nullptr
  uint16_t* y;
  int64_t M, Ncols, K;
  int nblk_n;
};

__global__ __launch_bounds__(kThreads) void out_proj_kernel(OprojArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t as_[BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t ws_[BN * PITCH];
  __shared__ __attribute__((aligned(16))) float cs[BM * CPITCH];
  const int64_t m0 = (int64_t)(blockIdx.x / a.nblk_n) * BM;
  const int64_t n0 = (int64_t)(blockIdx.x % a.nblk_n) * BN;
  f32x16_t acc;
  gemm_tile(a.A, a.W, a.M, a.Ncols, a.K, m0, n0, as_, ws_, acc);
  spill_acc(acc, cs);
  const int tid = threadIdx.x;
  const int r = tid >> 2, cq = tid & 3;
  const int64_t m = m0 + r;
  const int64_t n = n0 + cq * 16;
  if (m >= a.M || n >= a.Ncols) return;
  float yv[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) yv[e] = cs[r * CPITCH + cq * 16 + e];
  if (a.resid != nullptr) {
    const u32x4_t* rp = reinterpret_cast<const u32x4_t*>(a.resid + m * a.Ncols + n);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4_t rv = rp[h];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t pr = rv[e];
        yv[8 * h + 2 * e] += __builtin_bit_cast(float, pr << 16);
        yv[8 * h + 2 * e + 1] += __builtin_bit_cast(float, pr & 0xffff0000u);
      }
    }
  }
  u32x4_t w0, w1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w0[e] = pack_bf16x2(yv[2 * e], yv[2 * e + 1]);
    w1[e] = pack_bf16x2(yv[8 + 2 * e], yv[8 + 2 * e + 1]);
  }
  uint16_t* dst = a.y + m * a.Ncols + n;
  *reinterpret_cast<u32x4_t*>(dst) = w0;
  *reinterpret_cast<u32x4_t*>(dst + 8) = w1;
}

// ---------------------------------------------------------------- RMSNorm
struct NormArgs {
  const uint16_t* x;
  const uint16_t* g;
  uint16_t* y;
  int64_t M;
  int D;
  float eps;
};

// 32 lanes per row (8 rows per workgroup), 8 bf16 per lane per pass; the
// sum of squares is reduced with lane shuffles inside the 32-lane half.
__global__ __launch_bounds__(kThreads) void rms_norm_kernel(NormArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  const int l = threadIdx.x & 31;
  if (row >= a.M) return;  // whole 32-lane halves leave together
  const uint16_t* xr = a.x + row * a.D;
  float ss = 0.f;
  for (int c = l * 8; c < a.D; c += 256) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(xr + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t pr = v[e];
      const float lo = __builtin_bit_cast(float, pr << 16), hi = __builtin_bit_cast(float, pr & 0xffff0000u);
      ss = fmaf(lo, lo, fmaf(hi, hi, ss));
    }
  }
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) ss += __shfl_xor(ss, off);
  const float r = 1.0f / sqrtf(ss / (float)a.D + a.eps);
  uint16_t* yr = a.y + row * a.D;
  for (int c = l * 8; c < a.D; c += 256) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(xr + c);
    const u32x4_t gv = *reinterpret_cast<const u32x4_t*>(a.g + c);
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t pr = v[e], gr = gv[e];
      const float x0 = __builtin_bit_cast(float, pr << 16), x1 = __builtin_bit_cast(float, pr & 0xffff0000u);
      const float g0 = __builtin_bit_cast(float, gr << 16), g1 = __builtin_bit_cast(float, gr & 0xffff0000u);
      o[e] = pack_bf16x2(x0 * r * g0, x1 * r * g1);
    }
    *reinterpret_cast<u32x4_t*>(yr + c) = o;
  }
}

// ---------------------------------------------------------------- SwiGLU
struct GateUpArgs {
  ASrc A;
  WSrc Wg, Wu;
  uint16_t* h;
  int64_t M, F, K;
  int nblk_n;
};

__global__ __launch_bounds__(kThreads) void gate_up_kernel(GateUpArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t as_[BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t ws_[BN * PITCH];
  __shared__ __attribute__((aligned(16))) float cg[BM * CPITCH];
  __shared__ __attribute__((aligned(16))) float cu[BM * CPITCH];
  const int64_t m0 = (int64_t)(blockIdx.x / a.nblk_n) * BM;
  const int64_t n0 = (int64_t)(blockIdx.x % a.nblk_n) * BN;
  f32x16_t acc;
  gemm_tile(a.A, a.Wg, a.M, a.F, a.K, m0, n0, as_, ws_, acc);
  spill_acc(acc, cg);
  gemm_tile(a.A, a.Wu, a.M, a.F, a.K, m0, n0, as_, ws_, acc);
  spill_acc(acc, cu);
  const int tid = threadIdx.x;
  const int r = tid >> 2, cq = tid & 3;
  const int64_t m = m0 + r;
  const int64_t n = n0 + cq * 16;
  if (m >= a.M || n >= a.F) return;
  float hv[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float g = cg[r * CPITCH + cq * 16 + e];
    const float u = cu[r * CPITCH + cq * 16 + e];
    hv[e] = g / (1.0f + expf(-g)) * u;  // silu(g) * u
  }
  u32x4_t w0, w1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w0[e] = pack_bf16x2(hv[2 * e], hv[2 * e + 1]);
    w1[e] = pack_bf16x2(hv[8 + 2 * e], hv[8 + 2 * e + 1]);
  }
  uint16_t* dst = a.h + m * a.F + n;
  *reinterpret_cast<u32x4_t*>(dst) = w0;
  *reinterpret_cast<u32x4_t*>(dst + 8) = w1;
}

struct RopeArgs {
  float* cs;
  int64_t N, half;
  Theta theta;
};

__global__ __launch_bounds__(kThreads) void rope_table_kernel(RopeArgs a) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= a.N * a.half) return;
  const int64_t t = i / a.half, c = i % a.half;
  const double twopi = 6.283185307179586476925286766559;
  double ang = (double)t * a.theta.v[c];
  ang -= twopi * floor(ang / twopi);  // reduce to [0, 2*pi) in fp64
  float sn, cn;
  sincosf((float)ang, &sn, &cn);
  a.cs[2 * i] = cn;
  a.cs[2 * i + 1] = sn;
}

}  // namespace

hipError_t launch_rope_table(float* cs, int64_t N, int64_t d, float rope_base, hipStream_t stream) {
  if (d % 2 != 0 || d / 2 > kMaxHalf) return hipErrorInvalidValue;
  RopeArgs a;
  a.cs = cs;
  a.N = N;
  a.half = d / 2;
  for (int i = 0; i < kMaxHalf; ++i)
    a.theta.v[i] = (i < d / 2) ? pow((double)rope_base, -2.0 * i / (double)d) : 0.0;
  const int64_t n = N * a.half;
  const int64_t nblk = (n + kThreads - 1) / kThreads;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)nblk), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_qkv_rope(const QkvProblem& p, hipStream_t stream) {
  if (p.d / 2 > kMaxHalf || p.d % 16 != 0 || p.Dm % 16 != 0) return hipErrorInvalidValue;
  QkvArgs a;
  a.A.p = static_cast<const uint16_t*>(p.x);
  a.A.K = p.Dm;
  a.A.gather = 0;
  a.A.N = p.N;
  a.A.Hq = p.Hq;
  a.A.d = p.d;
  a.W.w[0] = static_cast<const uint16_t*>(p.wq);
  a.W.w[1] = static_cast<const uint16_t*>(p.wk);
  a.W.w[2] = static_cast<const uint16_t*>(p.wv);
  a.W.ncol[0] = p.Hq * p.d;
  a.W.ncol[1] = p.Hkv * p.d;
  a.W.ncol[2] = p.Hkv * p.d;
  a.out[0] = static_cast<uint16_t*>(p.q);
  a.out[1] = static_cast<uint16_t*>(p.k);
  a.out[2] = static_cast<uint16_t*>(p.v);
  a.M = p.B * p.N;
  a.Ncols = (p.Hq + 2 * p.Hkv) * p.d;
  a.K = p.Dm;
  a.N = p.N;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.d = p.d;
  a.cs = p.rope_cs;
  a.nblk_n = (int)((a.Ncols + BN - 1) / BN);
  const int64_t nblk = ((a.M + BM - 1) / BM) * a.nblk_n;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(qkv_rope_kernel, dim3((unsigned)nblk), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_out_proj(const OprojProblem& p, hipStream_t stream) {
  if (p.d % 16 != 0 || p.Dm % 16 != 0) return hipErrorInvalidValue;
  OprojArgs a;
  a.A.p = static_cast<const uint16_t*>(p.o);
  a.A.K = p.Hq * p.d;
  a.A.gather = 1;
  a.A.N = p.N;
  a.A.Hq = p.Hq;
  a.A.d = p.d;
  a.W.w[0] = static_cast<const uint16_t*>(p.wo);
  a.W.w[1] = a.W.w[0];
  a.W.w[2] = a.W.w[0];
  a.W.ncol[0] = p.Dm;
  a.W.ncol[1] = 0;
  a.W.ncol[2] = 0;
  a.resid = static_cast<const uint16_t*>(p.resid);
  a.y = static_cast<uint16_t*>(p.y);
  a.M = p.B * p.N;
  a.Ncols = p.Dm;
  a.K = p.Hq * p.d;
  a.nblk_n = (int)((a.Ncols + BN - 1) / BN);
  const int64_t nblk = ((a.M + BM - 1) / BM) * a.nblk_n;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(out_proj_kernel, dim3((unsigned)nblk), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dense_residual(const DenseProblem& p, hipStream_t stream) {
  if (p.K % 16 != 0 || p.Ncols % 16 != 0) return hipErrorInvalidValue;
  OprojArgs a;
  a.A.p = static_cast<const uint16_t*>(p.a);
  a.A.K = p.K;
  a.A.gather = 0;
  a.A.N = 1;
  a.A.Hq = 1;
  a.A.d = 1;
  a.W.w[0] = static_cast<const uint16_t*>(p.w);
  a.W.w[1] = a.W.w[0];
  a.W.w[2] = a.W.w[0];
  a.W.ncol[0] = p.Ncols;
  a.W.ncol[1] = 0;
  a.W.ncol[2] = 0;
  a.resid = static_cast<const uint16_t*>(p.resid);
  a.y = static_cast<uint16_t*>(p.y);
  a.M = p.M;
  a.Ncols = p.Ncols;
  a.K = p.K;
  a.nblk_n = (int)((a.Ncols + BN - 1) / BN);
  const int64_t nblk = ((a.M + BM - 1) / BM) * a.nblk_n;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(out_proj_kernel, dim3((unsigned)nblk), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_rms_norm(const void* x, const void* g, void* y, int64_t M, int64_t D, float eps,
                           hipStream_t stream) {
  if (D % 8 != 0 || D > (int64_t(1) << 20)) return hipErrorInvalidValue;
  NormArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.g = static_cast<const uint16_t*>(g);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.D = (int)D;
  a.eps = eps;
  const int64_t nblk = (M + 7) / 8;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rms_norm_kernel, dim3((unsigned)nblk), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gate_up(const GateUpProblem& p, hipStream_t stream) {
  if (p.K % 16 != 0 || p.F % 16 != 0) return hipErrorInvalidValue;
  GateUpArgs a;
  a.A.p = static_cast<const uint16_t*>(p.z);
  a.A.K = p.K;
  a.A.gather = 0;
  a.A.N = 1;
  a.A.Hq = 1;
  a.A.d = 1;
  for (int i = 0; i < 3; ++i) {
    a.Wg.w[i] = static_cast<const uint16_t*>(p.w_gate);
    a.Wu.w[i] = static_cast<const uint16_t*>(p.w_up);
  }
  a.Wg.ncol[0] = p.F;
  a.Wg.ncol[1] = 0;
  a.Wg.ncol[2] = 0;
  a.Wu.ncol[0] = p.F;
  a.Wu.ncol[1] = 0;
  a.Wu.ncol[2] = 0;
  a.h = static_cast<uint16_t*>(p.h);
  a.M = p.M;
  a.F = p.F;
  a.K = p.K;
  a.nblk_n = (int)((a.F + BN - 1) / BN);
  const int64_t nblk = ((a.M + BM - 1) / BM) * a.nblk_n;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gate_up_kernel, dim3((unsigned)nblk), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sqa
