// SQA attention forward for head dim 16, bf16 in/out, gfx950: dense and
// packed variable-length batches without key-range splits (the attention core
// of the SQAT-m layer: B16, N1024, (8,4), causal).
//
// Operation: query head i attends K/V head floor(i*H_kv/H_q) (contiguous
// query-head groups, "GQA ..." page, "The idea") with fewer query heads than
// the baseline (SQA paper abstract); encoder-style or causal.
//
// At d = 16 each score costs half an MFMA k-step but the softmax spends a
// v_exp_f32 and a few other VALU instructions on it, so this kernel is bound
// by VALU issue, not by the matrix pipe. It trades matrix work for VALU work:
//   * The scale and the running maximum are folded into the score MFMAs.
//     Each query row is multiplied by c = scale*log2(e) in fp32 and split
//     into two bf16 parts, x = hi + lo (|x - hi - lo| <= 2^-18 |x|), which
//     fill the 32-deep k of v_mfma_f32_16x16x32_bf16 (K rows twice against
//     hi then lo), and the chain starts from the C operand -m (m the row's
//     running maximum). The accumulator then holds s*c - m, and a probability
//     is one v_exp_f32 of it.
//   * 16x16 tiles fit d = 16 exactly: O^T (16 dims x 16 queries) += V^T P^T
//     over 32 keys is one MFMA with no padded rows.
// What is left per score: v_exp_f32, half a v_cvt_pk_bf16_f32 and half a
// v_dot2c_f32_bf16 (the row sum of the rounded probabilities).
//
// Decomposition: a workgroup is 4 row waves sharing one (batch, K/V head);
// each owns 32 query rows of one query head (slots ordered by position block,
// then head-in-group, as the other forward kernels; groups may differ in size
// by one head and packed sequences in length, and workgroups with no rows
// leave at once). On grids too small to fill the device the workgroup has 8
// waves: the row waves twice, over two key ranges (the first ceil(nt/2) of
// its nt tiles and the rest) in lockstep on one ring with two tiles a slot,
// the two partial softmax results (O, l, m) combined through LDS at the end
// (the rescaling of partial results by exp(m_part - m), as in the online
// softmax itself). K/V stream in 64-key tiles straight from HBM to LDS
// (buffer_load ... lds, one 1 KB DMA per wave and tile: K keys 0-31, K keys
// 32-63, V keys 0-31, V keys 32-63) through a 4-slot ring, one barrier per
// tile. K and V rows are in key order (32 B), the K rows' two 16-byte chunks
// swapped on rows 8-15 of every 16; V reaches the P.V MFMA through
// ds_read_b64_tr_b16. The score MFMA's k-groups run hi and lo of one chunk
// before the other chunk's (G = 2*chunk + part), so that lanes 0-31 of a K
// fragment read share 16 chunks: a 16-byte LDS read is served in passes of
// 32 lanes x 8 bytes, and two chunks per row in one pass met in the same
// banks (SQ_LDS_BANK_CONFLICT about 2 per LDS instruction before, 0 after).
//
// Schedule: a wave's 32 rows are two 16-row halves in a two-phase pipeline
// over the tiles kt (as the d = 64 kernel's):
//   phase A(kt): MFMA P(kt-1,h1).V(kt-1), S(kt,h1)    VALU softmax S(kt,h0)
//   phase B(kt): MFMA P(kt,h0).V(kt),   S(kt+1,h0)    VALU softmax S(kt,h1)
// so the MFMAs of one half run under the exponentials of the other and a
// wave's chain of tiles is not a sequence of MFMA and VALU latencies.
//
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

constexpr int D = 16;
constexpr int kWaves = 4;                          // row waves per key-range part
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
  static_assert(PENDING == 1 || PENDING == 2, "pending DMAs");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(PENDING == 2 ? 0x0072 : 0x0071);  // vmcnt(PENDING) lgkmcnt(0)
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
  uint32_t kro;      // K fragment offset within a slot (+ 16-key block * 512 B)
  uint32_t vro;      // V transposed-read offset within a slot (+ 32-key range * 1 KB + half * 512 B)
};

struct Ctx {
  Ring ring;
  const uint16_t* kvbase;  // K (row waves 0, 1) or V (row waves 2, 3) of this (batch, K/V head)
  int N, causal;
  int kbase, kend;         // this wave's key-range part: step j takes tile kbase + j, tiles below kend
  int last;                // last tile this wave computes (below kbase: none)
  int diag;                // causal: the tile that holds the diagonal of this wave's rows
  uint32_t dst;            // LDS offset of this wave's DMA part within a slot
  int lim[2];              // per half: last visible key minus this lane's first key of a block, at tile 0
};

struct WaveState {
  u32x4_t qf[2];     // per half: c*q as the B operand, k-group G: hi (G even) or lo (G odd) of dims 8(G>>1)..
  f32x4_t negm[2];   // per half: -m in every entry, the C operand of each score chain
  f32x4_t o[2];      // per half: O^T entries, dims 4G .. 4G+3 of query l%16
  float l[2];        // per half: this lane's share of the row sum
  u32x4_t kf[4];     // K fragments of the tile whose scores come next, per 16-key block
  u32x4_t vf[2];     // V^T fragments of the tile whose P.V comes next, per 32-key range
  f32x4_t s[2][4];   // per half, per 16-key block: scores (keys 16*blk + 4G + i)
  u32x4_t pk[2][2];  // per half, per 32-key range: P^T as the B operand
};

// DMA wave `wave`'s 1 KB part of tile kt into ring slot SLOT; keys at or past
// N are zero-filled by the descriptor's range check, without any memory
// access (a tile past the last is all zeros). Every wave issues one DMA per
// tile, also past the last tile, so that the count of VMEM operations in
// flight is the same on every path: the compiler's own waits before LDS reads
// of a slot are then exact instead of a wait for every DMA in flight.
template <int SLOT>
__device__ __forceinline__ void issue_tile(const Ctx& cx, const Lane& ln, int j) {
  const int kt = cx.kbase + j;
  const bool live = kt < cx.kend;
  const int key0 = live ? kt * kTileKeys : 0;
  const int rem = live ? max(cx.N - key0, 0) * kRowBytes : 0;
  __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(cx.kvbase + (size_t)key0 * D), (short)0, rem, kBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(cx.ring.p[SLOT] + cx.dst), 16, ln.dma_src, 0, 0, 0);
}

template <int SLOT>
__device__ __forceinline__ void read_k(const Ctx& cx, const Lane& ln, u32x4_t (&kf)[4]) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    kf[kb] = *reinterpret_cast<const u32x4_t*>(cx.ring.p[SLOT] + ln.kro + kb * 16 * kRowBytes);
}

// V^T fragments per 32-key range j: dims l%16 against keys 32j + 4G + 0..3
// (k positions 8G + 0..3) and 32j + 16 + 4G + 0..3 (8G + 4..7).
template <int SLOT>
__device__ __forceinline__ void read_v(const Ctx& cx, const Lane& ln, u32x4_t (&vf)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint8_t* p = cx.ring.p[SLOT] + ln.vro + j * kBlockBytes;
    const u32x2_t a = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
    const u32x2_t b =
        __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 16 * kRowBytes)));
    vf[j] = u32x4_t{a[0], a[1], b[0], b[1]};
  }
}

// S'^T = [K K].[hi lo]^T - m of half h for the four 16-key blocks in kf.
__device__ __forceinline__ void mfma_s(WaveState& w, int h) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) w.s[h][kb] = mfma(w.kf[kb], w.qf[h], w.negm[h]);
}

// O^T(h) += V^T P^T(h) over the 64 keys of the tile in vf.
__device__ __forceinline__ void mfma_pv(WaveState& w, int h) {
#pragma unroll
  for (int j = 0; j < 2; ++j) w.o[h] = mfma(w.vf[j], w.pk[h][j], w.o[h]);
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
        w.o[h][i] *= alpha;
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

// Scheduling hints for a phase: each of its 6 MFMAs followed by 5 VALU
// instructions of the other half's softmax.
__device__ __forceinline__ void interleave_phase() {
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
  }
}

// Step j (tile kt = kbase + j) in ring slot SLOT: phase A(kt), the barrier
// that makes step j+1's tile resident and frees step j-1's slot for step
// j+3's, phase B(kt).
template <int SLOT, bool FIRST>
__device__ __forceinline__ void step(const Ctx& cx, const Lane& ln, WaveState& w, int j) {
  constexpr int NEXT = (SLOT + 1) % NBUF;
  constexpr int ISSUE = (SLOT + NBUF - 1) % NBUF;
  const int kt = cx.kbase + j;
  const bool active = kt <= cx.last;
  const int key0 = kt * kTileKeys;
  const bool masked = (cx.causal && kt == cx.diag) || (key0 + kTileKeys > cx.N);

  // ---- phase A(kt): P(kt-1,h1).V(kt-1), S(kt,h1) || softmax S(kt,h0)
  if (active) {
    if (masked) mask_half(w.s[0], cx.lim[0] - key0);
    mfma_pv(w, 1);
    mfma_s(w, 1);
    softmax_half<FIRST>(w, 0);
    interleave_phase();
  }

  wait_vm_then_barrier<1>();
  issue_tile<ISSUE>(cx, ln, j + NBUF - 1);

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

// KSPLIT: eight waves, the workgroup's tiles split in two key-range parts
// (row waves 0-3 the first ceil(nt/2) tiles, 4-7 the rest) run side by side
// over the same rows, their partial results combined through LDS at the end.
template <bool KSPLIT>
__global__ __launch_bounds__(KSPLIT ? 512 : 256, 4) void attn_fwd_bf16_d16_kernel(Args16 a) {
  constexpr int kParts = KSPLIT ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t ring0[kParts * kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[kParts * kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[kParts * kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[kParts * kSlotBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rw = wave & (kWaves - 1);         // row wave
  const int kh = KSPLIT ? wave / kWaves : 0;  // key-range part
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
  const int slot = w_in * kWaves + rw;
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
  const int nt = a.causal ? min((maxtb * kRowsPerWave + kRowsPerWave - 1) / kTileKeys + 1, NT) : NT;
  // steps of the ring; the second key-range part starts at tile ns, where
  // every row of a wave that computes any of its tiles sees the tile's first
  // key (a wave's 32 rows lie in one 64-key window), as the first part's
  // rows all see key 0: the first tile's exact row maximum is defined
  const int ns = KSPLIT ? (nt + 1) / 2 : nt;
  cx.kbase = kh * ns;
  cx.kend = (KSPLIT && kh == 0) ? ns : nt;
  cx.diag = !wave_valid ? -1 : (a.causal ? min((tb * kRowsPerWave + kRowsPerWave - 1) / kTileKeys, NT - 1) : NT - 1);
  cx.last = min(cx.diag, cx.kend - 1);
  cx.dst = (uint32_t)(kh * kSlotBytes + rw * kBlockBytes);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int t = tb * kRowsPerWave + hf * 16 + c16;
    cx.lim[hf] = (a.causal ? min(t, N - 1) : N - 1) - 4 * G;
  }
  const int64_t kvrow0 = sg.kv_base + (int64_t)kvh * sg.stride;
  const int64_t qrow0 = sg.q_base + (int64_t)h * sg.stride;
  cx.kvbase = (rw < 2 ? a.k : a.v) + (size_t)kvrow0 * D;

  Lane ln;
  if (rw < 2) {  // K keys 32*rw + r, 16-byte chunk c at position c ^ ((r >> 3) & 1)
    const int r = lane >> 1, cp = lane & 1;
    ln.dma_src = (uint32_t)((rw * 32 + r) * kRowBytes + ((cp ^ ((r >> 3) & 1)) * 16));
  } else {       // V keys 32*(rw-2) .. +31
    ln.dma_src = (uint32_t)((rw - 2) * kBlockBytes + lane * 16);
  }
  ln.kro = (uint32_t)(kh * kSlotBytes + c16 * kRowBytes + (((G >> 1) ^ (c16 >> 3)) * 16));
  ln.vro = (uint32_t)(kh * kSlotBytes + kVOffset + (4 * G + (c16 >> 2)) * kRowBytes + (c16 & 3) * 8);

  // ---- Q loads, on every wave (one past the last row block reads row N-1 of
  // its head): a load under a branch would be waited for inside it, before
  // the first DMA is issued. The split into hi/lo follows the DMA issue.
  u32x4_t qraw[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int t = min(tb * kRowsPerWave + hf * 16 + c16, N - 1);
    qraw[hf] = *reinterpret_cast<const u32x4_t*>(a.q + ((size_t)qrow0 + t) * D + (G >> 1) * 8);
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
    for (int e = 0; e < 4; ++e) {
      const float x0 = bf16_lo(qraw[hf][e]) * a.c, x1 = bf16_hi(qraw[hf][e]) * a.c;
      const uint32_t hi = pack_bf16x2(x0, x1);
      w.qf[hf][e] = (G & 1) ? pack_bf16x2(x0 - bf16_lo(hi), x1 - bf16_hi(hi)) : hi;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w.o[hf][i] = 0.f;
      w.negm[hf][i] = 0.f;
    }
    w.l[hf] = 0.f;
    w.pk[hf][0] = w.pk[hf][1] = u32x4_t{0u, 0u, 0u, 0u};  // P(-1,h1) = 0: the first P.V is a no-op
  }
  w.vf[0] = w.vf[1] = u32x4_t{0u, 0u, 0u, 0u};

  wait_vm_then_barrier<2>();
  if (cx.last >= cx.kbase) {
    read_k<0>(cx, ln, w.kf);
    mfma_s(w, 0);
  }

  // whole turns of the ring: steps past the last tile only barrier and issue
  // their (empty) DMA, so that every path issues the same VMEM sequence
  step<0, true>(cx, ln, w, 0);
  for (int j = 1; j < ns; j += NBUF) {
    step<1, false>(cx, ln, w, j);
    step<2, false>(cx, ln, w, j + 1);
    step<3, false>(cx, ln, w, j + 2);
    step<0, false>(cx, ln, w, j + 3);
  }
  if (cx.last >= cx.kbase) mfma_pv(w, 1);  // drain P(last,h1) V(last)

  // no DMA may still write this workgroup's LDS once its waves have ended
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  float ltot[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    ltot[hf] = w.l[hf] + __shfl_xor(w.l[hf], 16);
    ltot[hf] += __shfl_xor(ltot[hf], 32);
  }
  if constexpr (KSPLIT) {
    // the second part hands O^T, l and m (per lane, as held) to the row wave
    // of the first part through the ring's first two slots; a part that
    // computed no tile has l = 0 and adds nothing. Both parts' m are finite.
    f32x4_t* ob = reinterpret_cast<f32x4_t*>(ring0);
    f32x2_t* lb = reinterpret_cast<f32x2_t*>(ring1);
    __syncthreads();  // every wave is past its last read of the ring
    if (kh == 1) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        ob[(rw * 2 + hf) * 64 + lane] = w.o[hf];
        lb[(rw * 2 + hf) * 64 + lane] = f32x2_t{ltot[hf], w.negm[hf][0]};
      }
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4_t o1 = ob[(rw * 2 + hf) * 64 + lane];
      const f32x2_t lm = lb[(rw * 2 + hf) * 64 + lane];
      if (lm[0] > 0.f) {
        const float m = fmaxf(-w.negm[hf][0], -lm[1]);
        const float a0 = __builtin_amdgcn_exp2f(-w.negm[hf][0] - m), a1 = __builtin_amdgcn_exp2f(-lm[1] - m);
#pragma unroll
        for (int i = 0; i < 4; ++i) w.o[hf][i] = w.o[hf][i] * a0 + o1[i] * a1;
        ltot[hf] = ltot[hf] * a0 + lm[0] * a1;
        w.negm[hf][0] = -m;
      }
    }
  }
  if (!wave_valid) return;
  // ---- epilogue: O = O^T / l (bf16, nearest even), LSE = m ln2 + ln l;
  // lane group G holds dims 4G .. 4G+3 of query l%16 of each half
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int t = tb * kRowsPerWave + hf * 16 + c16;
    if (t < N) {
      const float inv = 1.0f / ltot[hf];
      const u32x2_t out = {pack_bf16x2(w.o[hf][0] * inv, w.o[hf][1] * inv),
                           pack_bf16x2(w.o[hf][2] * inv, w.o[hf][3] * inv)};
      // non-temporal: no dirty L2 line left to write back at the end
      __builtin_nontemporal_store(out, reinterpret_cast<u32x2_t*>(a.o + ((size_t)qrow0 + t) * D + 4 * G));
      if (a.lse != nullptr && G == 0)
        a.lse[(size_t)qrow0 + t] = (log2f(ltot[hf]) - w.negm[hf][0]) * 0.69314718055994531f;
    }
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
  // key-range parts when the eight-wave workgroups all fit on the device at
  // once (two per CU at four waves per SIMD): the waves' tile chains halve
  // and twice the waves hide each other's latency. With more workgroups
  // they would run in two rounds, slower than the four-wave kernel in one.
  if ((int64_t)a.nwg <= 2LL * device_cus())
    hipLaunchKernelGGL(attn_fwd_bf16_d16_kernel<true>, dim3((unsigned)a.nwg), dim3(2 * kWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_d16_kernel<false>, dim3((unsigned)a.nwg), dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sqa
