// SQA attention forward for head dim 16, bf16 in/out, gfx950: dense and
// packed variable-length batches without key-range splits (the attention core
// of the SQAT-m layer: B16, N1024, (8,4), causal).
//
// Operation: query head i attends K/V head floor(i*H_kv/H_q) (contiguous
// query-head groups, "GQA ..." page, "The idea") with fewer query heads than
// the baseline (SQA paper abstract); encoder-style or causal.
//
// At d = 16 each score costs one MFMA k-step but the softmax spends a
// v_exp_f32 and a handful of other VALU instructions on it, so this kernel
// is bound by VALU issue, not by the matrix pipe. It trades matrix work for
// VALU work wherever it can:
//   * The scale and the running maximum are folded into the score MFMAs.
//     Each query row is multiplied by c = scale*log2(e) in fp32 and split
//     into two bf16 parts, x = hi + lo (|x - hi - lo| <= 2^-18 |x|), and the
//     score chain S'^T = K.hi^T + K.lo^T starts from the C operand -m (m the
//     row's running maximum, in every accumulator entry). The accumulator then
//     holds s*c - m, and a probability is one v_exp_f32 of it.
//   * V^T rows 16..31 of the 32-row P.V MFMA (which d = 16 leaves over) read
//     the same V rows with the head dims rotated by 4, so each lane-half ends
//     with all 16 dims of its row and stores 8 of them as one 16-byte write.
// What is left per score: v_exp_f32, half a v_cvt_pk_bf16_f32 and half a
// v_dot2c_f32_bf16 (the row sum of the rounded probabilities).
//
// Decomposition: a workgroup is 4 waves sharing one (batch, K/V head); each
// wave owns 32 query rows of one query head (slots ordered by position block,
// then head-in-group, as the other forward kernels; groups may differ in size
// by one head and packed sequences in length, and workgroups with no rows
// leave at once). K/V stream in 64-key
// tiles straight from HBM to LDS (buffer_load ... lds, one 1 KB DMA per wave
// and tile: K keys 0-31, K keys 32-63, V keys 0-31, V keys 32-63) through a
// 4-slot ring with one barrier per tile. K rows sit in LDS under the
// permutation pi (accumulator entry i of lane-half lg is then key lg*16 + i,
// the B-operand order of P^T) with their two 16-byte chunks swapped on rows
// 8-15 and 24-31 (conflict-free fragment reads); V rows are in key order and
// reach the P.V MFMA through ds_read_b64_tr_b16.
//
// Softmax: probabilities against the running maximum as it stands; a wave's
// first tile takes its exact row maximum, later tiles raise it only when a
// lane's sum of its 32 rounded probabilities exceeds 2^20 (or is not finite),
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
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int D = 16;
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kTileKeys = 64;
constexpr int kRowBytes = D * 2;                   // 32 B per key row
constexpr int kBlockBytes = 32 * kRowBytes;        // 32 keys: 1 KB, one DMA per wave
constexpr int kSlotBytes = 4 * kBlockBytes;        // K keys 0-31, K 32-63, V 0-63
constexpr int kVOffset = 2 * kBlockBytes;
constexpr int NBUF = 4;                            // ring slots
constexpr int kXcds = 8;
constexpr float kSumLimit = 1048576.0f;            // 2^20
constexpr float kMinC = 1e-30f;                    // |scale|*log2(e) is clamped up to this
constexpr int kBufferWord3 = 0x00020000;           // raw buffer descriptor flags (gfx9)

struct Args16 {
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

__device__ __forceinline__ int pi_row(int r) { return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ f32x16_t mfma(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Wait for this wave's LDS reads and for its DMAs of every tile but the two
// newest, then synchronise the workgroup.
__device__ __forceinline__ void wait_vm_then_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0072);  // vmcnt(2) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Separate __shared__ objects per slot, so that the compiler can tell an LDS
// read of one slot from a DMA in flight into another.
struct Ring {
  uint8_t* p[NBUF];
};

struct Lane {
  uint32_t dma_src;  // source byte offset within the tile of this lane's 16-byte DMA chunk
  uint32_t kro[2];   // K fragment offsets (32-key block 0, 1) within a slot
  uint32_t vro;      // V transposed-read offset within a slot (+ block*1 KB + hh*256 + hi*128)
};

struct Ctx {
  Ring ring;
  const uint16_t* kvbase;  // K (waves 0, 1) or V (waves 2, 3) of this (batch, K/V head)
  int N, nt, last, causal, wave;
  int vis;                 // last key this lane's row may see
  int lg;
};

struct WaveState {
  u32x4_t qh, ql;   // c*q split into two bf16 parts (B operand, k = head dims)
  f32x16_t negm;    // -m in every entry: the C operand of each score chain
  f32x16_t o;       // O^T (rows 0-15: dims 0-15; rows 16-31: dims rotated by 4)
  float l;          // this lane's share of the row sum
};

// DMA wave `wave`'s 1 KB part of tile kt into ring slot SLOT; keys at or past
// N are zero-filled by the descriptor's range check, without any memory
// access (a tile past the last is all zeros). Every wave issues one DMA per
// tile step, also past the last tile, so that the count of VMEM operations
// in flight is the same on every path: the compiler's own waits before LDS
// reads of a slot are then exact instead of a wait for every DMA (measured
// as an s_waitcnt vmcnt(0) before the reads of one slot in four).
template <int SLOT>
__device__ __forceinline__ void issue_tile(const Ctx& cx, const Lane& ln, int kt) {
  const int key0 = kt * kTileKeys;
  const int rem = max(cx.N - key0, 0) * kRowBytes;
  __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(cx.kvbase + (size_t)key0 * D), (short)0, rem, kBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(cx.ring.p[SLOT] + cx.wave * kBlockBytes), 16, ln.dma_src,
                                           0, 0, 0);
}

// S'^T = K.hi^T + K.lo^T + C for both 32-key blocks of the tile in slot SLOT.
template <int SLOT>
__device__ __forceinline__ void scores(const Ctx& cx, const Lane& ln, const WaveState& w, const f32x16_t& cinit,
                                       f32x16_t (&s)[2]) {
#pragma unroll
  for (int kx = 0; kx < 2; ++kx) {
    const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(cx.ring.p[SLOT] + ln.kro[kx]);
    s[kx] = mfma(kf, w.qh, cinit);
    s[kx] = mfma(kf, w.ql, s[kx]);
  }
}

// Keys past `lim` (relative to the block's first key of this lane-half)
// become -inf.
__device__ __forceinline__ void mask_tile(f32x16_t (&s)[2], int lim) {
#pragma unroll
  for (int kx = 0; kx < 2; ++kx)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i > lim - kx * 32) s[kx][i] = -INFINITY;
}

// Probabilities 2^s, rounded to bf16 and packed as the P^T B operand
// [block][hh]; returns the lane's sum of its 32 rounded probabilities.
__device__ __forceinline__ float exp_pack(const f32x16_t (&s)[2], u32x4_t (&pk)[2][2]) {
  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int kx = 0; kx < 2; ++kx)
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t pp =
          pack_bf16x2(__builtin_amdgcn_exp2f(s[kx][2 * w]), __builtin_amdgcn_exp2f(s[kx][2 * w + 1]));
      pk[kx][w >> 2][w & 3] = pp;
      if (w & 1) l1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp), ones, l1, false);
      else l0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp), ones, l0, false);
    }
  return l0 + l1;
}

// Largest of the row's scores in this tile (both lane-halves).
__device__ __forceinline__ float row_max(const f32x16_t (&s)[2]) {
  float mx = s[0][0];
#pragma unroll
  for (int kx = 0; kx < 2; ++kx)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kx][i]);
  return fmaxf(mx, __shfl_xor(mx, 32));
}

// O^T += V^T P^T over the tile in slot SLOT.
template <int SLOT>
__device__ __forceinline__ void pv(const Ctx& cx, const Lane& ln, const u32x4_t (&pk)[2][2], f32x16_t& o) {
#pragma unroll
  for (int kx = 0; kx < 2; ++kx)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint8_t* p = cx.ring.p[SLOT] + ln.vro + kx * kBlockBytes + hh * 8 * kRowBytes;
      const u32x2_t a = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
      const u32x2_t b =
          __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * kRowBytes)));
      o = mfma(u32x4_t{a[0], a[1], b[0], b[1]}, pk[kx][hh], o);
    }
}

// One tile: wait for it (and free the slot three tiles on), then, if the
// wave has rows that see it, scores, softmax and P.V.
template <int SLOT, bool FIRST>
__device__ __forceinline__ void step(const Ctx& cx, const Lane& ln, WaveState& w, int kt) {
  wait_vm_then_barrier();
  issue_tile<(SLOT + NBUF - 1) % NBUF>(cx, ln, kt + NBUF - 1);
  if (kt > cx.last) return;

  const int key0 = kt * kTileKeys;
  const bool masked = (cx.causal && kt == cx.last) || (key0 + kTileKeys > cx.N);
  const int lim = cx.vis - key0 - cx.lg * 16;
  f32x16_t s[2];
  u32x4_t pk[2][2];
  if constexpr (FIRST) {
    // the wave's first tile: its exact row maximum (every row sees key 0)
    f32x16_t zero;
#pragma unroll
    for (int i = 0; i < 16; ++i) zero[i] = 0.f;
    scores<SLOT>(cx, ln, w, zero, s);
    if (masked) mask_tile(s, lim);
    const float mx = row_max(s);
#pragma unroll
    for (int kx = 0; kx < 2; ++kx)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kx][i] -= mx;
#pragma unroll
    for (int i = 0; i < 16; ++i) w.negm[i] = -mx;
    w.l = exp_pack(s, pk);
  } else {
    scores<SLOT>(cx, ln, w, w.negm, s);
    if (masked) mask_tile(s, lim);
    float ls = exp_pack(s, pk);
    if (__ballot(!(ls <= kSumLimit))) {
      // a probability grew past the safe range: raise m by the tile's
      // maximum over it (never lower it), rescale O and l, recompute
      const float dm = fmaxf(row_max(s), 0.f);
      const float alpha = __builtin_amdgcn_exp2f(-dm);
      w.l *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        w.o[i] *= alpha;
        w.negm[i] -= dm;
      }
#pragma unroll
      for (int kx = 0; kx < 2; ++kx)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kx][i] -= dm;
      ls = exp_pack(s, pk);
    }
    w.l += ls;
  }
  pv<SLOT>(cx, ln, pk, w.o);
}

__global__ __launch_bounds__(kThreads, 4) void attn_fwd_bf16_d16_kernel(Args16 a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring0[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[kSlotBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lg = lane >> 5;

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
  cx.wave = wave;
  cx.lg = lg;
  const int maxtb = min((w_in * kWaves + kWaves - 1) / g, TB - 1);
  cx.nt = a.causal ? min((maxtb * kRowsPerWave + kRowsPerWave - 1) / kTileKeys + 1, NT) : NT;
  cx.last = !wave_valid ? -1 : (a.causal ? min((tb * kRowsPerWave + kRowsPerWave - 1) / kTileKeys, NT - 1) : NT - 1);
  const int t = tb * kRowsPerWave + l32;
  cx.vis = a.causal ? min(t, N - 1) : N - 1;
  const int64_t kvrow0 = sg.kv_base + (int64_t)kvh * sg.stride;
  const int64_t qrow0 = sg.q_base + (int64_t)h * sg.stride;
  cx.kvbase = (wave < 2 ? a.k : a.v) + (size_t)kvrow0 * D;

  Lane ln;
  if (wave < 2) {  // K keys 32*wave + pi(r), 16-byte chunk c at position c ^ ((r >> 3) & 1)
    const int r = lane >> 1, cp = lane & 1;
    ln.dma_src = (uint32_t)((wave * 32 + pi_row(r)) * kRowBytes + ((cp ^ ((r >> 3) & 1)) * 16));
  } else {         // V keys 32*(wave-2) .. +31 in order
    ln.dma_src = (uint32_t)((wave - 2) * kBlockBytes + lane * 16);
  }
#pragma unroll
  for (int kx = 0; kx < 2; ++kx)
    ln.kro[kx] = (uint32_t)(kx * kBlockBytes + l32 * kRowBytes + ((lg ^ ((l32 >> 3) & 1)) * 16));
  {
    // lanes 16-31 of each half read dims 4.. with a rotation by 4, so that
    // accumulator rows 16-31 hold dims (r - 12) mod 16
    const int j16 = lane & 15, g1 = (lane >> 4) & 1;
    ln.vro = (uint32_t)(kVOffset + (lg * 16 + (j16 >> 2)) * kRowBytes + ((((j16 & 3) + g1) & 3) * 8));
  }

  // ---- Q: c*q in fp32, split into bf16 hi + lo (B operand, dims lg*8 .. +8)
  WaveState w;
  {
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (wave_valid) x = *reinterpret_cast<const u32x4_t*>(a.q + ((size_t)qrow0 + min(t, N - 1)) * D + lg * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = bf16_lo(x[e]) * a.c, x1 = bf16_hi(x[e]) * a.c;
      const uint32_t hi = pack_bf16x2(x0, x1);
      w.qh[e] = hi;
      w.ql[e] = pack_bf16x2(x0 - bf16_lo(hi), x1 - bf16_hi(hi));
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    w.o[i] = 0.f;
    w.negm[i] = 0.f;
  }
  w.l = 0.f;

  // ---- prologue: tiles 0..2 in flight, then one tile per step
  issue_tile<0>(cx, ln, 0);
  issue_tile<1>(cx, ln, 1);
  issue_tile<2>(cx, ln, 2);
  // whole turns of the ring: steps past the last tile only wait, barrier and
  // issue their (empty) DMA, so that every path issues the same VMEM sequence
  step<0, true>(cx, ln, w, 0);
  for (int kt = 1; kt < cx.nt; kt += NBUF) {
    step<1, false>(cx, ln, w, kt);
    step<2, false>(cx, ln, w, kt + 1);
    step<3, false>(cx, ln, w, kt + 2);
    step<0, false>(cx, ln, w, kt + 3);
  }

  // no DMA may still write this workgroup's LDS once its waves have ended
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  if (!wave_valid) return;
  // ---- epilogue: O = O^T / l (bf16, nearest even), LSE = m ln2 + ln l.
  // Lane-half 0 holds dims 0-3 in entries 0-3 and 4-7 in entries 8-11;
  // lane-half 1 holds dims 8-11 in entries 8-11 and 12-15 in entries 4-7.
  const float ltot = w.l + __shfl_xor(w.l, 32);
  if (t < N) {
    const float inv = 1.0f / ltot;
    u32x4_t out;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float a0 = lg ? w.o[8 + 2 * e] : w.o[2 * e];
      const float a1 = lg ? w.o[9 + 2 * e] : w.o[2 * e + 1];
      const float b0 = lg ? w.o[4 + 2 * e] : w.o[8 + 2 * e];
      const float b1 = lg ? w.o[5 + 2 * e] : w.o[9 + 2 * e];
      out[e] = pack_bf16x2(a0 * inv, a1 * inv);
      out[2 + e] = pack_bf16x2(b0 * inv, b1 * inv);
    }
    // non-temporal: no dirty L2 line left to write back at the end
    __builtin_nontemporal_store(out, reinterpret_cast<u32x4_t*>(a.o + ((size_t)qrow0 + t) * D + lg * 8));
    if (a.lse != nullptr && lg == 0) a.lse[(size_t)qrow0 + t] = (log2f(ltot) - w.negm[0]) * 0.69314718055994531f;
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16_d16(const AttnProblem& p, hipStream_t stream) {
  if (p.D != D || p.nsplit > 1 || p.tail_split > 1) return hipErrorInvalidValue;
  // the DMA descriptors count a sequence's bytes from a tile on in 32 bits
  if (p.N * kRowBytes >= 0x7fffffffLL) return hipErrorInvalidValue;
  Args16 a;
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
  hipLaunchKernelGGL(attn_fwd_bf16_d16_kernel, dim3((unsigned)a.nwg), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sqa
