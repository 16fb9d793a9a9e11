// Merge of key-range splits of the attention forward (shared by the d = 64
// kernel and the d = 16/32 kernel). Each range of a query row left its
// unnormalised output O_s, running maximum m_s (log2 units) and sum l_s in
// fp32; the streaming-softmax merge is M = max m_s,
// O = sum 2^(m_s - M) O_s / sum 2^(m_s - M) l_s, LSE = (M + log2 L) ln 2.
// Range s is part of row t when it holds a key tile of the sequence and,
// under a causal mask, starts at or before t; rows of sequences that were
// not split were finished by the attention kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "seq_groups.h"

namespace sqa {
namespace {

struct SplitMergeArgs {
  const float* part;  // [nsplit][rows][D] O, then [nsplit][rows][2] (m, l)
  uint16_t* o;
  float* lse;
  const int* cu;  // packed sequence offsets (nullptr: dense)
  int64_t T, rows;
  int N, B, nsplit, causal;
  int tile_keys, min_tiles, even;  // the attention kernel's key tile and split_chunk rule
};

// D/4 lanes per query row, lane j holding head dims 4j..4j+3.
template <int D>
__global__ __launch_bounds__(256) void attn_split_merge_kernel(SplitMergeArgs a) {
  typedef float f4_t __attribute__((ext_vector_type(4)));
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  constexpr int kLanes = D / 4, kRowsPerBlock = 256 / kLanes;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanes;
  const int j = threadIdx.x % kLanes;
  if (r >= a.rows) return;
  int t, n;
  if (a.cu == nullptr) {
    t = (int)(r % a.N);
    n = a.N;
  } else {
    // token p of some head; its sequence is the last b with start(b) <= p,
    // offsets clamped into [0, T] as the attention kernels clamp them
    const int64_t p = r % a.T;
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      int64_t st = a.cu[mid];
      st = st < 0 ? 0 : (st > a.T ? a.T : st);
      if (st <= p) lo = mid; else hi = mid - 1;
    }
    int64_t st = a.cu[lo], en = a.cu[lo + 1];
    st = st < 0 ? 0 : (st > a.T ? a.T : st);
    en = en < st ? st : (en > a.T ? a.T : en);
    if (p < st || p >= en) return;
    t = (int)(p - st);
    n = (int)(en - st < (int64_t)a.N ? en - st : (int64_t)a.N);
  }
  if (t >= n) return;
  const int NT = (n + a.tile_keys - 1) / a.tile_keys;
  const int chunk = split_chunk(NT, a.nsplit, a.min_tiles, a.even != 0);
  if (NT <= chunk) return;
  const float* pml = a.part + (size_t)a.nsplit * a.rows * D;
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) {
    const int kt0 = s * chunk;
    if (kt0 >= NT || (a.causal && kt0 * a.tile_keys > t)) break;
    M = fmaxf(M, pml[((size_t)s * a.rows + r) * 2]);
  }
  float L = 0.f;
  f4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.nsplit; ++s) {
    const int kt0 = s * chunk;
    if (kt0 >= NT || (a.causal && kt0 * a.tile_keys > t)) break;
    const f2_t ml = *reinterpret_cast<const f2_t*>(pml + ((size_t)s * a.rows + r) * 2);
    const float wgt = __builtin_amdgcn_exp2f(ml[0] - M);
    L += wgt * ml[1];
    acc += wgt * *reinterpret_cast<const f4_t*>(a.part + ((size_t)s * a.rows + r) * D + 4 * j);
  }
  const float inv = 1.0f / L;
  const b2_t lo2 = __builtin_convertvector((f2_t){acc[0] * inv, acc[1] * inv}, b2_t);
  const b2_t hi2 = __builtin_convertvector((f2_t){acc[2] * inv, acc[3] * inv}, b2_t);
  uint32_t* dst = reinterpret_cast<uint32_t*>(a.o + (size_t)r * D + 4 * j);
  dst[0] = __builtin_bit_cast(uint32_t, lo2);
  dst[1] = __builtin_bit_cast(uint32_t, hi2);
  if (a.lse != nullptr && j == 0) a.lse[r] = (M + log2f(L)) * 0.69314718055994531f;
}

template <int D>
hipError_t launch_split_merge(const SplitMergeArgs& m, hipStream_t stream, bool dry_run) {
  constexpr int kRowsPerBlock = 256 / (D / 4);
  const int64_t blocks = (m.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (dry_run) return hipSuccess;
  hipLaunchKernelGGL((attn_split_merge_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, stream, m);
  return hipGetLastError();
}

}  // namespace
}  // namespace sqa
