// Row-wise helper of the SQAT-m block (SQAT-m model card, "Architecture
// details": RMS Norm):
//   rms_norm : y = x / sqrt(mean(x^2) + eps) * g per row, fp32 math.
// The projection GEMMs (with the RoPE epilogue) live in gemm_bf16.hip.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace sqa {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
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

}  // namespace

hipError_t launch_rms_norm(const void* x, const void* g, void* y, int64_t M, int64_t D, float eps,
                           hipStream_t stream, bool dry_run) {
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
  if (dry_run) return hipSuccess;
  hipLaunchKernelGGL(rms_norm_kernel, dim3((unsigned)nblk), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sqa
