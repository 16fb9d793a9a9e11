// SQA attention forward for head dim 32, bf16 in/out, gfx950: dense and
// packed variable-length batches without key-range splits.
//
// Operation: query head i attends K/V head floor(i*H_kv/H_q) (contiguous
// query-head groups, "GQA ..." page, "The idea") with fewer query heads than
// the baseline (SQA paper abstract); encoder-style or causal.
//
// The design of the d = 16 kernel (attn_fwd_bf16_d16.hip) with every operand
// in two 16-dim halves. At d = 32 a score costs one 16x16x32 MFMA k-step of
// S and one of P.V, still less issue time than its v_exp_f32 and the rest of
// the softmax, so the kernel is bound by VALU issue and trades matrix work
// for VALU work as the d = 16 one does:
//   * Each query row is multiplied by c = scale*log2(e) in fp32 and split into
//     two bf16 parts, x = hi + lo (|x - hi - lo| <= 2^-18 |x|); per 16-key
//     block the score chain is two v_mfma_f32_16x16x32_bf16, one per dim
//     half, each with K rows twice against hi then lo, the first starting
//     from the C operand -m. The accumulator holds s*c - m and a probability
//     is one v_exp_f32 of it.
//   * O^T (two 16-dim halves x 16 queries) += V^T P^T over 32 keys is one
//     MFMA per dim half, P^T taken straight from the score accumulators.
//
// Decomposition: a workgroup is 4 waves sharing one (batch, K/V head); each
// wave owns 32 query rows of one query head (slots ordered by position block,
// then head-in-group, as the other forward kernels). K/V stream in 64-key
// tiles straight from HBM to LDS (buffer_load ... lds, two 1 KB DMAs per wave
// and tile: waves 0, 1 K keys 32w .. 32w+31, waves 2, 3 V keys
// 32(w-2) ..) through a 4-slot ring, one barrier per tile. Rows are 64 B;
// K rows hold their four 16-byte chunks at position c ^ ((key >> 2) & 3) and
// V rows their two 32-byte halves swapped when (key >> 2) & 1, so the
// fragment reads (16-byte reads of 16 rows, transposed 8-byte reads of 8
// rows) spread over all LDS banks; V reaches the P.V MFMA through
// ds_read_b64_tr_b16. The score MFMA's k-groups run hi and lo of one
// 16-byte chunk before the other chunk's (G = 2*chunk + part): a 16-byte LDS
// read is served in passes of 32 lanes x 8 bytes, so lanes 0-31 must not
// touch two chunks of one row (SQ_LDS_BANK_CONFLICT 2 per LDS instruction
// with hi/lo as the high k-group bit, 0 with this order).
//
// Schedule: a wave's 32 rows are two 16-row halves in the two-phase pipeline
// of the d = 16 kernel:
//   phase A(kt): MFMA P(kt-1,h1).V(kt-1), S(kt,h1)    VALU softmax S(kt,h0)
//   phase B(kt): MFMA P(kt,h0).V(kt),   S(kt+1,h0)    VALU softmax S(kt,h1)
// Softmax: probabilities against the running maximum as it stands; a wave's
// first tile takes its exact row maximum, later tiles raise it only when a
// lane's sum of its 16 rounded probabilities exceeds 2^20 (or is not finite),
// then rescale O and l and recompute the tile. Masked scores (causal key > t,
// key >= N) become -inf, on the causal diagonal tile and the ragged last tile
// only.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"
#include "seq_groups.h"

namespace sqa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int D = 32;
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kTileKeys = 64;
constexpr int kRowBytes = D * 2;                   // 64 B per key row
constexpr int kPartBytes = 16 * kRowBytes;         // 16 keys: 1 KB, one DMA instruction
constexpr int kVOffset = kTileKeys * kRowBytes;    // V after the tile's 64 K rows
constexpr int kSlotBytes = 2 * kVOffset;           // K and V of 64 keys: 8 KB
constexpr int kDma = 2;                            // DMA instructions per wave and tile
constexpr int NBUF = 4;                            // ring slots
constexpr int kXcds = 8;
constexpr float kSumLimit = 1048576.0f;            // 2^20
constexpr float kMinC = 1e-30f;                    // |scale|*log2(e) is clamped up to this
constexpr int kBufferWord3 = 0x00020000;           // raw buffer descriptor flags (gfx9)

struct Args32 {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int* cu;        // packed sequence offsets (nullptr: dense)
  int64_t T;            // packed: total tokens
  int N, Hq, Hkv;       // N: the (longest) sequence length
  int wg_per_bkv, n_bkv, nwg;
  int spread;           // packed, or uneven groups under a causal mask: spread_coords order
  int spread_block;
  int exact_per_batch;  // > 0: dense uneven groups, encoder-style: exact_coords order
  int pair_major;       // packed encoder-style: pair_major_coords order
  int snake;            // dense causal, even groups: the CU count (order reversed in every other round)
  float c;              // scale * log2(e), |c| clamped up to kMinC
  int causal;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// MFMA lane layout (v_mfma_f32_16x16x32_bf16): A lane l -> row l%16,
// k = (l/16)*8 + 0..7; B lane l -> column l%16, same k; accumulator entry i
// of lane l -> row (l/16)*4 + i, column l%16.
__device__ __forceinline__ f32x4_t mfma(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Wait for this wave's LDS reads and for its DMAs of every tile but the
// `pending` newest, then synchronise the workgroup.
template <int PENDING>
__device__ __forceinline__ void wait_vm_then_barrier() {
  static_assert(PENDING == 1 || PENDING == 2, "pending tiles");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(PENDING == 2 ? (0x0070 | (2 * kDma)) : (0x0070 | kDma));  // vmcnt lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Separate __shared__ objects per slot, so that the compiler can tell an LDS
// read of one slot from a DMA in flight into another.
struct Ring {
  uint8_t* p[NBUF];
};

struct Lane {
  uint32_t dma_src;  // source byte offset within the tile of this lane's 16-byte chunk (first DMA; +1 KB the second)
  uint32_t kro[2];   // per dim half: K fragment offset within a slot (+ 16-key block * 1 KB)
  uint32_t vro[2];   // per dim half: V transposed-read offset within a slot (+ 32-key range * 2 KB, + 1 KB)
};

struct Ctx {
  Ring ring;
  const uint16_t* kvbase;  // K (waves 0, 1) or V (waves 2, 3) of this (batch, K/V head)
  int N, nt, last, causal;
  uint32_t dst;            // LDS offset of this wave's DMA parts within a slot
  int lim[2];              // per half: last visible key minus this lane's first key of a block, at tile 0
};

struct WaveState {
  u32x4_t qf[2][2];  // [half][dim half]: c*q as the B operand, k-group G: hi (G even) or lo (G odd) of dims 8(G>>1)..
  f32x4_t negm[2];   // per half: -m in every entry, the C operand of each score chain
  f32x4_t o[2][2];   // [half][dim half]: O^T entries, dims 16*dh + 4G .. +3 of query l%16
  float l[2];        // per half: this lane's share of the row sum
  u32x4_t kf[4][2];  // K fragments of the tile whose scores come next, per 16-key block and dim half
  u32x4_t vf[2][2];  // V^T fragments of the tile whose P.V comes next, per 32-key range and dim half
  f32x4_t s[2][4];   // per half, per 16-key block: scores (keys 16*blk + 4G + i)
  u32x4_t pk[2][2];  // per half, per 32-key range: P^T as the B operand
};

// DMA this wave's two 1 KB parts of tile kt into ring slot SLOT; keys at or
// past N are zero-filled by the descriptor's range check, without any memory
// access. Every wave issues its DMAs for every tile step, also past the last
// tile, so that the count of VMEM operations in flight is the same on every
// path and the compiler's own waits before LDS reads of a slot stay exact.
template <int SLOT>
__device__ __forceinline__ void issue_tile(const Ctx& cx, const Lane& ln, int kt) {
  const bool live = kt < cx.nt;
  const int key0 = live ? kt * kTileKeys : 0;
  const int rem = live ? max(cx.N - key0, 0) * kRowBytes : 0;
  __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(cx.kvbase + (size_t)key0 * D), (short)0, rem, kBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(cx.ring.p[SLOT] + cx.dst), 16, ln.dma_src, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(cx.ring.p[SLOT] + cx.dst + kPartBytes), 16,
                                           ln.dma_src + kPartBytes, 0, 0, 0);
}

template <int SLOT>
__device__ __forceinline__ void read_k(const Ctx& cx, const Lane& ln, u32x4_t (&kf)[4][2]) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int dh = 0; dh < 2; ++dh)
      kf[kb][dh] = *reinterpret_cast<const u32x4_t*>(cx.ring.p[SLOT] + ln.kro[dh] + kb * kPartBytes);
}

// V^T fragments per 32-key range j and dim half dh: dims 16*dh + l%16 against
// keys 32j + 4G + 0..3 (k positions 8G + 0..3) and 32j + 16 + 4G + 0..3
// (8G + 4..7).
template <int SLOT>
__device__ __forceinline__ void read_v(const Ctx& cx, const Lane& ln, u32x4_t (&vf)[2][2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) {
      const uint8_t* p = cx.ring.p[SLOT] + ln.vro[dh] + j * 2 * kPartBytes;
      const u32x2_t a = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
      const u32x2_t b =
          __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + kPartBytes)));
      vf[j][dh] = u32x4_t{a[0], a[1], b[0], b[1]};
    }
}

// S'^T = [K K].[hi lo]^T - m of half h for the four 16-key blocks in kf: per
// block a chain over the two dim halves.
__device__ __forceinline__ void mfma_s(WaveState& w, int h) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) w.s[h][kb] = mfma(w.kf[kb][1], w.qf[h][1], mfma(w.kf[kb][0], w.qf[h][0], w.negm[h]));
}

// O^T(h) += V^T P^T(h) over the 64 keys of the tile in vf.
__device__ __forceinline__ void mfma_pv(WaveState& w, int h) {
#pragma unroll
  for (int dh = 0; dh < 2; ++dh)
#pragma unroll
    for (int j = 0; j < 2; ++j) w.o[h][dh] = mfma(w.vf[j][dh], w.pk[h][j], w.o[h][dh]);
}

// Keys past `lim` (relative to this lane's first key of each block) become -inf.
__device__ __forceinline__ void mask_half(f32x4_t (&s)[4], int lim) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (kb * 16 + i > lim) s[kb][i] = -INFINITY;
}

// Probabilities 2^s of one half, rounded to bf16 and packed as the P^T B
// operand of each 32-key range; returns the lane's sum of its 16 rounded
// probabilities.
__device__ __forceinline__ float exp_pack(const f32x4_t (&s)[4], u32x4_t (&pk)[2]) {
  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x4_t& b = s[2 * j + (w >> 1)];
      const uint32_t pp =
          pack_bf16x2(__builtin_amdgcn_exp2f(b[2 * (w & 1)]), __builtin_amdgcn_exp2f(b[2 * (w & 1) + 1]));
      pk[j][w] = pp;
      if (w & 1) l1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp), ones, l1, false);
      else l0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp), ones, l0, false);
    }
  return l0 + l1;
}

// Largest of a half's row scores in this tile (all four lane groups).
__device__ __forceinline__ float row_max(const f32x4_t (&s)[4]) {
  float mx = s[0][0];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  return fmaxf(mx, __shfl_xor(mx, 32));
}

// Softmax of half h's scores: the first tile takes the exact row maximum
// (every row sees key 0); later tiles raise m only when a probability grew
// past the safe range, rescaling O and l and recomputing.
template <bool FIRST>
__device__ __forceinline__ void softmax_half(WaveState& w, int h) {
  if constexpr (FIRST) {
    const float mx = row_max(w.s[h]);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) w.s[h][kb][i] -= mx;
#pragma unroll
    for (int i = 0; i < 4; ++i) w.negm[h][i] = -mx;
    w.l[h] = exp_pack(w.s[h], w.pk[h]);
  } else {
    float ls = exp_pack(w.s[h], w.pk[h]);
    if (__ballot(!(ls <= kSumLimit))) {
      const float dm = fmaxf(row_max(w.s[h]), 0.f);  // never lower m
      const float alpha = __builtin_amdgcn_exp2f(-dm);
      w.l[h] *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w.o[h][0][i] *= alpha;
        w.o[h][1][i] *= alpha;
        w.negm[h][i] -= dm;
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) w.s[h][kb][i] -= dm;
      ls = exp_pack(w.s[h], w.pk[h]);
    }
    w.l[h] += ls;
  }
}

// Scheduling hints for a phase: each of its 12 MFMAs followed by 3 VALU
// instructions of the other half's softmax.
__device__ __forceinline__ void interleave_phase() {
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
  }
}

// One tile kt in ring slot SLOT: phase A(kt), the barrier that makes tile
// kt+1 resident and frees tile kt-1's slot for tile kt+3, phase B(kt).
template <int SLOT, bool FIRST>
__device__ __forceinline__ void step(const Ctx& cx, const Lane& ln, WaveState& w, int kt) {
  constexpr int NEXT = (SLOT + 1) % NBUF;
  constexpr int ISSUE = (SLOT + NBUF - 1) % NBUF;
  const bool active = kt <= cx.last;
  const int key0 = kt * kTileKeys;
  const bool masked = (cx.causal && kt == cx.last) || (key0 + kTileKeys > cx.N);

  // ---- phase A(kt): P(kt-1,h1).V(kt-1), S(kt,h1) || softmax S(kt,h0)
  if (active) {
    if (masked) mask_half(w.s[0], cx.lim[0] - key0);
    mfma_pv(w, 1);
    mfma_s(w, 1);
    softmax_half<FIRST>(w, 0);
    interleave_phase();
  }

  wait_vm_then_barrier<1>();
  issue_tile<ISSUE>(cx, ln, kt + NBUF - 1);

  // ---- phase B(kt): P(kt,h0).V(kt), S(kt+1,h0) || softmax S(kt,h1)
  if (active) {
    read_v<SLOT>(cx, ln, w.vf);
    read_k<NEXT>(cx, ln, w.kf);
    if (masked) mask_half(w.s[1], cx.lim[1] - key0);
    mfma_pv(w, 0);
    mfma_s(w, 0);
    softmax_half<FIRST>(w, 1);
    interleave_phase();
  }
}

__global__ __launch_bounds__(kThreads, 3) void attn_fwd_bf16_d32_kernel(Args32 a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring0[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[kSlotBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, G = lane >> 4;

  // ---- workgroup -> (batch*Hkv, workgroup index within it)
  const int wid = (int)blockIdx.x;
  if (wid >= a.nwg) return;
  int bkv, w_in;
  if (a.pair_major) {
    if (!pair_major_coords(wid, a.n_bkv, a.wg_per_bkv, bkv, w_in)) return;
  } else if (a.spread) {
    spread_coords(wid, a.n_bkv, a.wg_per_bkv, a.causal != 0, a.spread_block, bkv, w_in);
  } else if (a.exact_per_batch > 0) {  // XCD-contiguous, exact counts per group
    const int per = a.nwg / kXcds, rem = a.nwg % kXcds;
    const int x = wid % kXcds, i = wid / kXcds;
    exact_coords(x * per + min(x, rem) + i, a.exact_per_batch, a.Hq, a.Hkv,
                 (a.N + kRowsPerWave - 1) / kRowsPerWave, kWaves, bkv, w_in);
  } else if (!a.causal) {
    // consecutive logical workgroups (same K/V head) on one XCD, whose L2
    // they share (the hardware deals blockIdx round-robin over the XCDs)
    const int per = a.nwg / kXcds, rem = a.nwg % kXcds;
    const int x = wid % kXcds, i = wid / kXcds;
    const int L = x * per + min(x, rem) + i;
    bkv = L / a.wg_per_bkv;
    w_in = L % a.wg_per_bkv;
  } else {
    // longest (largest position block) first, the order reversed in every
    // other full round of `snake` workgroups, so that the CUs that took the
    // longest blocks of one round take the shortest of the next
    int L = wid;
    if (a.snake > 0) {
      const int r = L / a.snake, c = L % a.snake;
      if ((r & 1) && (int64_t)(r + 1) * a.snake <= a.nwg) L = r * a.snake + (a.snake - 1 - c);
    }
    const int wr = L / a.n_bkv;
    bkv = L % a.n_bkv;
    w_in = a.wg_per_bkv - 1 - wr;
  }
  const int b = bkv / a.Hkv, kvh = bkv % a.Hkv;
  const HeadGroup hg = head_group(kvh, a.Hq, a.Hkv);
  const SeqGeom sg = seq_geom(a.cu, a.T, a.N, b, a.Hq, a.Hkv);
  const int N = sg.n, g = hg.count;
  const int TB = (N + kRowsPerWave - 1) / kRowsPerWave;
  const int NT = (N + kTileKeys - 1) / kTileKeys;
  if (w_in * kWaves >= TB * g) return;  // past this group's rows
  const int slot = w_in * kWaves + wave;
  const int tb = slot / g, jh = slot % g;
  const bool wave_valid = tb < TB;
  const int h = hg.first + jh;

  Ctx cx;
  cx.ring.p[0] = ring0;
  cx.ring.p[1] = ring1;
  cx.ring.p[2] = ring2;
  cx.ring.p[3] = ring3;
  cx.N = N;
  cx.causal = a.causal;
  const int maxtb = min((w_in * kWaves + kWaves - 1) / g, TB - 1);
  cx.nt = a.causal ? min((maxtb * kRowsPerWave + kRowsPerWave - 1) / kTileKeys + 1, NT) : NT;
  cx.last = !wave_valid ? -1 : (a.causal ? min((tb * kRowsPerWave + kRowsPerWave - 1) / kTileKeys, NT - 1) : NT - 1);
  cx.dst = (uint32_t)(wave * 2 * kPartBytes);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int t = tb * kRowsPerWave + hf * 16 + c16;
    cx.lim[hf] = (a.causal ? min(t, N - 1) : N - 1) - 4 * G;
  }
  const int64_t kvrow0 = sg.kv_base + (int64_t)kvh * sg.stride;
  const int64_t qrow0 = sg.q_base + (int64_t)h * sg.stride;
  cx.kvbase = (wave < 2 ? a.k : a.v) + (size_t)kvrow0 * D;

  // DMA lane i of a 1 KB part writes LDS bytes 16i: row r = i >> 2 of the
  // part's 16 keys, position p = i & 3; it reads the row's chunk stored there
  Lane ln;
  {
    const int r = lane >> 2, p = lane & 3;
    const int key = (wave & 1) * 32 + r;  // within the tile (second DMA: + 16 keys, same swizzle)
    const int ch = wave < 2 ? (p ^ ((r >> 2) & 3)) : (p ^ (((r >> 2) & 1) << 1));
    ln.dma_src = (uint32_t)(key * kRowBytes + ch * 16);
  }
#pragma unroll
  for (int dh = 0; dh < 2; ++dh) {
    ln.kro[dh] = (uint32_t)(c16 * kRowBytes + (((2 * dh + (G >> 1)) ^ ((c16 >> 2) & 3)) * 16));
    ln.vro[dh] = (uint32_t)(kVOffset + (4 * G + (c16 >> 2)) * kRowBytes + ((dh ^ (G & 1)) * 32) + (c16 & 3) * 8);
  }

  // ---- Q loads, on every wave (one past the last row block reads row N-1 of
  // its head): a load under a branch would be waited for inside it, before
  // the first DMA is issued. The split into hi/lo follows the DMA issue.
  u32x4_t qraw[2][2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int t = min(tb * kRowsPerWave + hf * 16 + c16, N - 1);
#pragma unroll
    for (int dh = 0; dh < 2; ++dh)
      qraw[hf][dh] = *reinterpret_cast<const u32x4_t*>(a.q + ((size_t)qrow0 + t) * D + dh * 16 + (G >> 1) * 8);
  }

  // ---- prologue: tiles 0..2 in flight; tile 0 landed; S(0,h0)
  issue_tile<0>(cx, ln, 0);
  issue_tile<1>(cx, ln, 1);
  issue_tile<2>(cx, ln, 2);
  __builtin_amdgcn_sched_barrier(0);

  WaveState w;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = bf16_lo(qraw[hf][dh][e]) * a.c, x1 = bf16_hi(qraw[hf][dh][e]) * a.c;
        const uint32_t hi = pack_bf16x2(x0, x1);
        w.qf[hf][dh][e] = (G & 1) ? pack_bf16x2(x0 - bf16_lo(hi), x1 - bf16_hi(hi)) : hi;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) w.o[hf][dh][i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) w.negm[hf][i] = 0.f;
    w.l[hf] = 0.f;
    w.pk[hf][0] = w.pk[hf][1] = u32x4_t{0u, 0u, 0u, 0u};  // P(-1,h1) = 0: the first P.V is a no-op
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) w.vf[j][0] = w.vf[j][1] = u32x4_t{0u, 0u, 0u, 0u};

  wait_vm_then_barrier<2>();
  if (cx.last >= 0) {
    read_k<0>(cx, ln, w.kf);
    mfma_s(w, 0);
  }

  // whole turns of the ring: steps past the last tile only barrier and issue
  // their (empty) DMAs, so that every path issues the same VMEM sequence
  step<0, true>(cx, ln, w, 0);
  for (int kt = 1; kt < cx.nt; kt += NBUF) {
    step<1, false>(cx, ln, w, kt);
    step<2, false>(cx, ln, w, kt + 1);
    step<3, false>(cx, ln, w, kt + 2);
    step<0, false>(cx, ln, w, kt + 3);
  }
  if (cx.last >= 0) mfma_pv(w, 1);  // drain P(last,h1) V(last)

  // no DMA may still write this workgroup's LDS once its waves have ended
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  if (!wave_valid) return;
  // ---- epilogue: O = O^T / l (bf16, nearest even), LSE = m ln2 + ln l;
  // lane group G holds dims 16*dh + 4G .. +3 of query l%16 of each half
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    float ltot = w.l[hf] + __shfl_xor(w.l[hf], 16);
    ltot += __shfl_xor(ltot, 32);
    const int t = tb * kRowsPerWave + hf * 16 + c16;
    if (t < N) {
      const float inv = 1.0f / ltot;
#pragma unroll
      for (int dh = 0; dh < 2; ++dh) {
        const u32x2_t out = {pack_bf16x2(w.o[hf][dh][0] * inv, w.o[hf][dh][1] * inv),
                             pack_bf16x2(w.o[hf][dh][2] * inv, w.o[hf][dh][3] * inv)};
        // non-temporal: no dirty L2 line left to write back at the end
        __builtin_nontemporal_store(out, reinterpret_cast<u32x2_t*>(a.o + ((size_t)qrow0 + t) * D + dh * 16 + 4 * G));
      }
      if (a.lse != nullptr && G == 0)
        a.lse[(size_t)qrow0 + t] = (log2f(ltot) - w.negm[hf][0]) * 0.69314718055994531f;
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16_d32(const AttnProblem& p, hipStream_t stream) {
  if (p.D != D || p.nsplit > 1 || p.tail_split > 1) return hipErrorInvalidValue;
  // the DMA descriptors count a sequence's bytes from a tile on in 32 bits
  if (p.N * kRowBytes >= 0x7fffffffLL) return hipErrorInvalidValue;
  Args32 a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.o = static_cast<uint16_t*>(p.o);
  a.lse = p.lse;
  a.cu = p.cu_seqlens;
  a.T = p.T;
  a.N = (int)p.N;
  a.Hq = (int)p.Hq;
  a.Hkv = (int)p.Hkv;
  const bool packed = p.cu_seqlens != nullptr;
  const bool uneven = p.Hq % p.Hkv != 0;
  a.spread = (packed || (uneven && p.causal)) ? 1 : 0;
  a.spread_block = spread_block(packed, p.B * p.Hkv);
  const int64_t TB = (p.N + kRowsPerWave - 1) / kRowsPerWave;
  const int64_t wg_per_bkv = (TB * max_group(a.Hq, a.Hkv) + kWaves - 1) / kWaves;
  if (wg_per_bkv > 0x7fffffff || p.B * p.Hkv > 0x7fffffff || TB * p.Hq > 0x7fffffff) return hipErrorInvalidValue;
  a.wg_per_bkv = (int)wg_per_bkv;
  a.n_bkv = (int)(p.B * p.Hkv);
  int64_t nwg = (int64_t)a.wg_per_bkv * a.n_bkv;
  a.exact_per_batch = 0;
  if (uneven && !a.spread) {
    int64_t per = 0;
    for (int j = 0; j < a.Hkv; ++j) per += group_wgs(j, a.Hq, a.Hkv, (int)TB, kWaves);
    if (per > 0x7fffffff) return hipErrorInvalidValue;
    a.exact_per_batch = (int)per;
    nwg = per * p.B;
  }
  a.pair_major = (packed && !p.causal) ? 1 : 0;
  if (a.pair_major) nwg = pair_major_nwg(a.n_bkv, a.wg_per_bkv);
  if (nwg > 0x7fffffff) return hipErrorInvalidValue;
  a.nwg = (int)nwg;
  a.snake = (!p.dry_run && p.causal && !a.spread && a.exact_per_batch == 0 && !a.pair_major) ? device_cus() : 0;
  const float cabs = fmaxf(fabsf(p.scale) * 1.4426950408889634f, kMinC);
  a.c = p.scale < 0.f ? -cabs : cabs;
  a.causal = p.causal;
  if (p.dry_run) return hipSuccess;
  hipLaunchKernelGGL(attn_fwd_bf16_d32_kernel, dim3((unsigned)a.nwg), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sqa
