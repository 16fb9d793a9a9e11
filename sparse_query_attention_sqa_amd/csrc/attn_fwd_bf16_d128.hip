// SQA attention forward for head dim 128, bf16 in/out, gfx950.
//
// Operation: query head i attends K/V head floor(i*H_kv/H_q) (contiguous
// query-head groups, "GQA ..." page, "The idea"), with fewer query heads than
// the baseline (SQA paper abstract); encoder-style or causal; dense
// [B, H, N, d] tensors or packed variable-length sequences.
//
// Decomposition: a workgroup is 4 waves that share one (batch, K/V head);
// each wave owns 32 query positions of one query head of the group (slots
// ordered by position block, then head-in-group), so one K/V tile in LDS
// feeds 128 query rows. On request (nsplit > 1) each row block's keys are
// cut into ranges computed by separate workgroups, merged afterwards
// (split_merge.h).
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
// (A = K tile from LDS, B = Q in registers, 8 k-steps over d = 128); the
// accumulator layout is the B operand of O^T += V^T P^T (4 output tiles of
// 32 head dims), so probabilities never leave registers.
//
// Schedule. At d = 128 a tile of 32 keys x 32 rows costs 16 MFMAs (8 for S,
// 8 for P.V) against one softmax of 16 scores per lane, so the MFMA pipe,
// not the VALU, sets the pace -- provided MFMA and softmax work of
// independent tiles are interleaved. Each wave runs a one-stage pipeline over
// 32-key tiles j:
//
//   phase j: MFMA  P(j-1).V(j-1)  and  S(j+1) = K(j+1).Q
//            VALU  softmax of S(j)                  -> P(j)
//
// with sched_group_barrier hints alternating one MFMA with four VALU ops.
// The fragments the next phase multiplies (V(j), K(j+2)) are read from LDS
// during this phase, after the MFMAs that consumed the previous ones.
//
// Data movement. K and V tiles go straight from HBM to LDS with
// buffer_load ... lds into a 5-slot ring (tile j+4 is issued in phase j; one
// barrier per tile). A 32 x 128 tile is stored as two 32 x 64 halves (head
// dims 0-63 and 64-127), each in the layout of the head-dim-64 kernel: K rows
// under the permutation pi with an XOR swizzle, read as 16-byte
// ds_read_b128; V rows natural with a swizzle, read with the transposing
// ds_read_b64_tr_b16. The descriptor's range check zero-fills keys past the
// sequence end.
//
// Softmax: fp32, base-2 exponentials of s*c - m (c = |scale|*log2 e), bf16
// probabilities whose row sum adds the same rounded values, and a lazily
// raised maximum (a tile is recomputed against the exact row maximum only
// when a lane's probability sum exceeds 2^20 or is not finite). Masked
// scores (causal key > t, tail key >= N) take a large negative value on the
// diagonal and tail tiles only.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"
#include "seq_groups.h"
#include "split_merge.h"

namespace sqa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int D = 128;
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kTileKeys = 32;
constexpr int kRowBytes = D * 2;                  // 256 B per row in HBM
constexpr int kHalfRowBytes = 128;                // one head-dim half of a row
constexpr int kHalfBytes = kTileKeys * kHalfRowBytes;  // 4 KB: one half-tile in LDS
constexpr int kSlotBytes = 4 * kHalfBytes;        // K lo | K hi | V lo | V hi
constexpr int NBUF = 5;                           // ring slots
constexpr int kDmaPerTile = 4;                    // DMA instructions per wave per tile
constexpr int kXcds = 8;
constexpr float kSumLimit = 1048576.0f;           // 2^20
constexpr float kMaskedScore = -3.0e38f;
constexpr float kMinC = 1e-30f;
constexpr int kBufferWord3 = 0x00020000;          // raw buffer descriptor flags (gfx9)

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int* cu;  // packed sequence offsets (nullptr: dense)
  int64_t T;      // packed: total tokens
  int N, Hq, Hkv;
  int wg_per_bkv, n_bkv, nwg;  // sized for the longest sequence and the largest head group
  int spread;                  // 1: spread_coords order (packed sequences, causal uneven groups)
  int spread_block;   // rotation block of the spread order
  int exact_per_batch;         // > 0: exact_coords order with this many workgroups per batch
  int pair_major;  // packed encoder-style: pair_major_coords order
  float c;
  uint32_t qsign;
  int causal;
  int nsplit;    // key-range splits (1: none)
  float* part;   // nsplit > 1: [nsplit][rows][128] unnormalised O, then [nsplit][rows][2] (m, l)
  int64_t rows;  // query rows: B*Hq*N (packed: Hq*T)
};

__device__ __forceinline__ int pi_row(int r) { return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3); }
__device__ __forceinline__ int swz_k(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_v(int r) { return 2 * (r & 3); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// s_waitcnt immediate (gfx9 encoding): vmcnt vm, expcnt 7, lgkmcnt 0.
constexpr int waitcnt_vm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

// Wait until at most VM of this wave's DMAs are in flight and its LDS reads
// are done, then synchronise the workgroup.
template <int VM>
__device__ __forceinline__ void barrier_vm() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct Ring {
  uint8_t* p[NBUF];
};

struct Lane {
  int l32, lg;
  uint32_t voff_k, voff_v;  // DMA source offsets within a tile (bytes), low head-dim half
  uint32_t koff[4];         // K fragment LDS offsets within a half-tile
  uint32_t voffr[2];        // V^T transposed-read LDS offsets within a half-tile
};

struct WaveState {
  u32x4_t qf[8];         // Q rows as B operands, k-steps over d
  f32x16_t acc_o[4];     // O^T, head dims x*32 .. x*32+31
  float m_run, l_run;
  u32x4_t kf[8];         // K fragments of the next S
  u32x4_t vf[4][2];      // V^T fragments of the next P.V
  f32x16_t s[2];         // scores of tiles j (s[j&1]) and j+1
  u32x4_t pk[2][2];      // probabilities of tiles j-1 and j (pk[j&1])
};

// DMA K/V tile kt into ring slot SLOT: per wave 8 rows of each half-tile.
// Rows at or past nlim are zero-filled by the descriptor range check without
// any memory access, so tiles past the last one are issued as empty DMAs.
template <int SLOT>
__device__ __forceinline__ void issue_tile(const Ring& ring, const uint16_t* kbase, const uint16_t* vbase, int kt,
                                           int nlim, int wave, const Lane& ln) {
  const int key0 = kt * kTileKeys;
  const int rem = max(nlim - key0, 0) * kRowBytes;
  __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (size_t)key0 * D), (short)0, rem, kBufferWord3);
  __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (size_t)key0 * D), (short)0, rem, kBufferWord3);
  uint8_t* slot = ring.p[SLOT] + wave * 1024;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)slot, 16, ln.voff_k, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(slot + kHalfBytes), 16, ln.voff_k + kHalfRowBytes, 0,
                                           0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(slot + 2 * kHalfBytes), 16, ln.voff_v, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(slot + 3 * kHalfBytes), 16, ln.voff_v + kHalfRowBytes,
                                           0, 0, 0);
}

// K fragments (A operand, M = 32 keys) for k-steps ds = 0..7 (head dims
// ds*16 .. ds*16+15): steps 0-3 from the low half-tile, 4-7 from the high.
template <int SLOT>
__device__ __forceinline__ void read_k(const Ring& ring, const Lane& ln, u32x4_t (&kf)[8]) {
#pragma unroll
  for (int ds = 0; ds < 8; ++ds)
    kf[ds] = *reinterpret_cast<const u32x4_t*>(ring.p[SLOT] + (ds >> 2) * kHalfBytes + ln.koff[ds & 3]);
}

// V^T fragments [x][hh]: keys lg*16 + hh*8 + 0..7 of head dim x*32 + l32, as
// two transposed 4-key reads; x = 0, 1 from the low half-tile, 2, 3 from the
// high one.
template <int SLOT>
__device__ __forceinline__ void read_v(const Ring& ring, const Lane& ln, u32x4_t (&vf)[4][2]) {
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint8_t* p =
          ring.p[SLOT] + (2 + (x >> 1)) * kHalfBytes + ln.voffr[x & 1] + hh * 8 * kHalfRowBytes;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * kHalfRowBytes));
      const u32x2_t a = __builtin_bit_cast(u32x2_t, lo);
      const u32x2_t b = __builtin_bit_cast(u32x2_t, hi);
      vf[x][hh] = u32x4_t{a[0], a[1], b[0], b[1]};
    }
}

__device__ __forceinline__ void mfma_s(const u32x4_t (&kf)[8], const u32x4_t (&q)[8], f32x16_t& s) {
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int ds = 0; ds < 8; ++ds)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[ds]), as_bf16x8(q[ds]), acc, 0, 0, 0);
  s = acc;
}

__device__ __forceinline__ void mfma_pv(const u32x4_t (&vf)[4][2], const u32x4_t (&pk)[2], f32x16_t (&o)[4]) {
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int x = 0; x < 4; ++x)
      o[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[x][hh]), as_bf16x8(pk[hh]), o[x], 0, 0, 0);
}

__device__ __forceinline__ void mask_scores(f32x16_t& s, int key0, int n, int causal, int t, int lg) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = key0 + lg * 16 + i;
    if (!(key < n && (!causal || key <= t))) s[i] = kMaskedScore;
  }
}

// Probabilities of a tile against the current maximum m, rounded to bf16 and
// packed as the B operand of O^T += V^T P^T; returns the lane's sum of its 16
// rounded probabilities.
__device__ __forceinline__ float exp_tile(const f32x16_t& s, u32x4_t (&pk)[2], float c, float m) {
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

// If a lane's probabilities grew too large (or m was still -inf), take the
// exact row maximum, rescale O and l and recompute the tile's probabilities.
__device__ __forceinline__ void finish_tile(float lsum, const f32x16_t& s, u32x4_t (&pk)[2], float& m, float& l,
                                            f32x16_t (&o)[4], float c) {
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
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[x][i] *= alpha;
    lsum = exp_tile(s, pk, c, m);
  }
  l += lsum;
}

// Scheduling hints for one phase: 16 MFMAs, each followed by 4 VALU
// instructions of the independent softmax work.
__device__ __forceinline__ void interleave_phase() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
  }
}

struct Ctx {
  Ring ring;
  const uint16_t* kbase;
  const uint16_t* vbase;
  int n, nlim, last, tb, causal, wave, t;
  float c;
};

// Phase j: tile j sits in ring slot SLOT = j % NBUF; P = j & 1 selects the
// score and probability registers.
template <int SLOT, int P>
__device__ __forceinline__ void phase(const Ctx& cx, const Lane& ln, WaveState& w, int j) {
  constexpr int AHEAD = (SLOT + 4) % NBUF;
  constexpr int KNEXT = (SLOT + 2) % NBUF;
  // tile j+2 has landed (tile j+3 may still be in flight); every wave is done
  // with tile j-1, whose slot receives tile j+4
  barrier_vm<kDmaPerTile>();
  issue_tile<AHEAD>(cx.ring, cx.kbase, cx.vbase, j + 4, cx.nlim, cx.wave, ln);
  if (j > cx.last) return;

  const int key0 = j * kTileKeys;
  const bool masked = (cx.causal && j == cx.tb) || (key0 + kTileKeys > cx.n);
  if (masked) mask_scores(w.s[P], key0, cx.n, cx.causal, cx.t, ln.lg);
  mfma_pv(w.vf, w.pk[P ^ 1], w.acc_o);   // P(j-1) V(j-1)
  read_v<SLOT>(cx.ring, ln, w.vf);        // V(j), multiplied next phase
  mfma_s(w.kf, w.qf, w.s[P ^ 1]);        // S(j+1); K(j+1) is in kf
  read_k<KNEXT>(cx.ring, ln, w.kf);       // K(j+2)
  const float ls = exp_tile(w.s[P], w.pk[P], cx.c, w.m_run);
  interleave_phase();
  finish_tile(ls, w.s[P], w.pk[P], w.m_run, w.l_run, w.acc_o, cx.c);
}

__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_d128_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring0[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring4[kSlotBytes];
  Ring ring;
  ring.p[0] = ring0;
  ring.p[1] = ring1;
  ring.p[2] = ring2;
  ring.p[3] = ring3;
  ring.p[4] = ring4;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- workgroup -> (batch*Hkv, slot range)
  // key-range split: runs of 8 consecutive workgroups take one split index,
  // so that the splits of logical workgroup wid run on XCD wid % 8
  const int g8 = (int)(blockIdx.x >> 3), x8 = (int)(blockIdx.x & 7);
  const int split = g8 % a.nsplit;
  const int wid = (g8 / a.nsplit) * 8 + x8;
  if (wid >= a.nwg) return;
  int bkv, w_in;
  if (a.pair_major) {
    if (!pair_major_coords(wid, a.n_bkv, a.wg_per_bkv, bkv, w_in)) return;
  } else if (a.spread) {
    spread_coords(wid, a.n_bkv, a.wg_per_bkv, a.causal != 0, a.spread_block, bkv, w_in);
  } else if (a.exact_per_batch > 0 || !a.causal) {  // XCD-contiguous (shared L2)
    const int bid = wid;
    const int per = a.nwg / kXcds, rem = a.nwg % kXcds;
    const int x = bid % kXcds, i = bid / kXcds;
    const int L = x * per + min(x, rem) + i;
    if (a.exact_per_batch > 0) {
      exact_coords(L, a.exact_per_batch, a.Hq, a.Hkv, (a.N + kRowsPerWave - 1) / kRowsPerWave, kWaves, bkv, w_in);
    } else {
      bkv = L / a.wg_per_bkv;
      w_in = L % a.wg_per_bkv;
    }
  } else {  // causal: longest (largest position block) first
    const int L = wid;
    const int wr = L / a.n_bkv;
    bkv = L % a.n_bkv;
    w_in = a.wg_per_bkv - 1 - wr;
  }
  const int b = bkv / a.Hkv, kvh = bkv % a.Hkv;
  const HeadGroup hg = head_group(kvh, a.Hq, a.Hkv);
  const SeqGeom sg = seq_geom(a.cu, a.T, a.N, b, a.Hq, a.Hkv);
  const int n = sg.n, g = hg.count;
  const int TB = (n + kRowsPerWave - 1) / kRowsPerWave;  // 32-row query blocks
  const int NT = (n + kTileKeys - 1) / kTileKeys;        // 32-key tiles
  if (w_in * kWaves >= TB * g) return;  // no rows for this workgroup (whole workgroup)
  const int slot = w_in * kWaves + wave;
  const int tb = slot / g, jh = slot % g;
  const bool wave_valid = tb < TB;
  const int h = hg.first + jh;
  const int maxtb = min((w_in * kWaves + kWaves - 1) / g, TB - 1);
  const int nt_all = a.causal ? min(maxtb + 1, NT) : NT;
  const int last_all = !wave_valid ? -1 : (a.causal ? tb : NT - 1);
  // Key-range split: key tiles [kt0, kt0 + chunk) of the workgroup's rows,
  // with tiles, keys, n and the causal positions counted from kt0 below. A
  // causal wave (32 rows, diagonal tile tb) sees a key of every row in a
  // range starting at or before tb and none in a later one.
  const int chunk = split_chunk(NT, a.nsplit, kMinSplitTiles, false);
  const bool split_rows = NT > chunk;
  const int kt0 = split * chunk;
  if (kt0 >= nt_all) return;
  const int nt = min(nt_all - kt0, chunk);
  const int last = last_all < kt0 ? -1 : min(last_all - kt0, chunk - 1);
  const int key_shift = kt0 * kTileKeys;
  const int trow0 = tb * kRowsPerWave;

  Lane ln;
  ln.l32 = lane & 31;
  ln.lg = lane >> 5;
  {
    const int r = wave * 8 + (lane >> 3), s = lane & 7;
    ln.voff_k = (uint32_t)(pi_row(r) * kRowBytes + ((s ^ swz_k(r)) * 16));
    ln.voff_v = (uint32_t)(r * kRowBytes + ((s ^ swz_v(r)) * 16));
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
      ln.koff[ds] = (uint32_t)(ln.l32 * kHalfRowBytes + (((ds * 2 + ln.lg) ^ swz_k(ln.l32)) * 16));
    const int j16 = lane & 15, g1 = (lane >> 4) & 1;
    const int row = ln.lg * 16 + (j16 >> 2);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int c16 = x * 4 + 2 * g1 + ((j16 & 3) >> 1);
      ln.voffr[x] = (uint32_t)(row * kHalfRowBytes + ((c16 ^ swz_v(row)) * 16) + (j16 & 1) * 8);
    }
  }

  const int64_t kvrow0 = sg.kv_base + (int64_t)kvh * sg.stride;
  const int64_t qrow0 = sg.q_base + (int64_t)h * sg.stride;
  const uint16_t* kbase = a.k + (size_t)(kvrow0 + key_shift) * D;
  const uint16_t* vbase = a.v + (size_t)(kvrow0 + key_shift) * D;
  const int nk = n - key_shift;  // keys of this sequence from the range start on

  WaveState w;
  {
    const int t = min(trow0 + ln.l32, n - 1);
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (wave_valid)
        x = *reinterpret_cast<const u32x4_t*>(a.q + ((size_t)qrow0 + t) * D + (ds * 2 + ln.lg) * 8);
      x ^= a.qsign;
      w.qf[ds] = x;
    }
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
#pragma unroll
    for (int i = 0; i < 16; ++i) w.acc_o[x][i] = 0.f;
    w.vf[x][0] = u32x4_t{0u, 0u, 0u, 0u};  // V(-1) = 0 and P(-1) = 0: the first P.V is a no-op
    w.vf[x][1] = u32x4_t{0u, 0u, 0u, 0u};
  }
  w.pk[1][0] = u32x4_t{0u, 0u, 0u, 0u};
  w.pk[1][1] = u32x4_t{0u, 0u, 0u, 0u};
  w.m_run = -INFINITY;
  w.l_run = 0.f;

  // zero the ring once so that no LDS byte is ever uninitialised
#pragma unroll
  for (int sl = 0; sl < NBUF; ++sl)
    for (int e = tid; e < kSlotBytes / 16; e += kThreads)
      reinterpret_cast<u32x4_t*>(ring.p[sl])[e] = u32x4_t{0u, 0u, 0u, 0u};
  barrier_vm<0>();

  // prologue: tiles 0..3 in flight (empty ranges past the end), wait for
  // tiles 0..2, S(0), then K(1) into kf
  const int nlim = min(nk, nt * kTileKeys);  // keys the workgroup streams
  issue_tile<0>(ring, kbase, vbase, 0, nlim, wave, ln);
  issue_tile<1>(ring, kbase, vbase, 1, nlim, wave, ln);
  issue_tile<2>(ring, kbase, vbase, 2, nlim, wave, ln);
  issue_tile<3>(ring, kbase, vbase, 3, nlim, wave, ln);
  barrier_vm<kDmaPerTile>();
  read_k<0>(ring, ln, w.kf);
  mfma_s(w.kf, w.qf, w.s[0]);
  read_k<1>(ring, ln, w.kf);

  Ctx cx;
  cx.ring = ring;
  cx.kbase = kbase;
  cx.vbase = vbase;
  cx.n = nk;
  cx.nlim = nlim;
  cx.last = last;
  cx.tb = tb - kt0;
  cx.causal = a.causal;
  cx.wave = wave;
  cx.t = trow0 + ln.l32 - key_shift;
  cx.c = a.c;

  // ten phases per round (ring slots repeat every 5, register parity every
  // 2); whole rounds first, so that every path to the loop back-edge has
  // issued the same DMAs and the compiler's wait bookkeeping stays exact
  int j = 0;
  for (; j + 2 * NBUF <= nt; j += 2 * NBUF) {
    phase<0, 0>(cx, ln, w, j);
    phase<1, 1>(cx, ln, w, j + 1);
    phase<2, 0>(cx, ln, w, j + 2);
    phase<3, 1>(cx, ln, w, j + 3);
    phase<4, 0>(cx, ln, w, j + 4);
    phase<0, 1>(cx, ln, w, j + 5);
    phase<1, 0>(cx, ln, w, j + 6);
    phase<2, 1>(cx, ln, w, j + 7);
    phase<3, 0>(cx, ln, w, j + 8);
    phase<4, 1>(cx, ln, w, j + 9);
  }
  if (j < nt) phase<0, 0>(cx, ln, w, j);
  if (j + 1 < nt) phase<1, 1>(cx, ln, w, j + 1);
  if (j + 2 < nt) phase<2, 0>(cx, ln, w, j + 2);
  if (j + 3 < nt) phase<3, 1>(cx, ln, w, j + 3);
  if (j + 4 < nt) phase<4, 0>(cx, ln, w, j + 4);
  if (j + 5 < nt) phase<0, 1>(cx, ln, w, j + 5);
  if (j + 6 < nt) phase<1, 0>(cx, ln, w, j + 6);
  if (j + 7 < nt) phase<2, 1>(cx, ln, w, j + 7);
  if (j + 8 < nt) phase<3, 0>(cx, ln, w, j + 8);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  if (last < 0) return;
  // drain P(last) V(last)
  if (last & 1) mfma_pv(w.vf, w.pk[1], w.acc_o);
  else mfma_pv(w.vf, w.pk[0], w.acc_o);

  const float ltot = w.l_run + __shfl_xor(w.l_run, 32);
  const int t = trow0 + ln.l32;
  if (split_rows) {
    // ---- split epilogue: unnormalised O^T, m and l of this key range (fp32)
    if (t < n) {
      float* po = a.part + ((size_t)split * a.rows + qrow0 + t) * D;
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int ab = 0; ab < 4; ++ab) {
          const f32x4_t v4 = {w.acc_o[x][4 * ab], w.acc_o[x][4 * ab + 1], w.acc_o[x][4 * ab + 2],
                              w.acc_o[x][4 * ab + 3]};
          *reinterpret_cast<f32x4_t*>(po + x * 32 + 8 * ab + 4 * ln.lg) = v4;
        }
      if (ln.lg == 0)
        *reinterpret_cast<f32x2_t*>(a.part + (size_t)a.nsplit * a.rows * D + ((size_t)split * a.rows + qrow0 + t) * 2) =
            f32x2_t{w.m_run, ltot};
    }
    return;
  }

  // ---- epilogue: O = O^T / l (bf16, nearest even); LSE = m ln2 + ln l
  const float inv = 1.0f / ltot;
  if (t < n) {
    uint16_t* orow = a.o + ((size_t)qrow0 + t) * D;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int ab = 0; ab < 4; ++ab) {
        // accumulator entries 4ab..4ab+3 are head dims x*32 + 8ab + 4lg + 0..3
        u32x2_t wv;
        wv[0] = pack_bf16x2(w.acc_o[x][4 * ab] * inv, w.acc_o[x][4 * ab + 1] * inv);
        wv[1] = pack_bf16x2(w.acc_o[x][4 * ab + 2] * inv, w.acc_o[x][4 * ab + 3] * inv);
        *reinterpret_cast<u32x2_t*>(orow + x * 32 + 8 * ab + 4 * ln.lg) = wv;
      }
    if (a.lse != nullptr && ln.lg == 0) a.lse[(size_t)qrow0 + t] = (w.m_run + log2f(ltot)) * 0.69314718055994531f;
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16_d128(const AttnProblem& p, hipStream_t stream) {
  if (p.D != D) return hipErrorInvalidValue;
  if (p.N * kRowBytes > 0x7fffffffLL) return hipErrorInvalidValue;  // buffer descriptor range
  Args a;
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
  const bool uneven = p.Hq % p.Hkv != 0;
  a.spread = (p.cu_seqlens != nullptr || (uneven && p.causal)) ? 1 : 0;
  a.spread_block = spread_block(p.cu_seqlens != nullptr, p.B * p.Hkv);
  const int TB = (int)((p.N + kRowsPerWave - 1) / kRowsPerWave);
  const int64_t slots = (int64_t)TB * max_group(a.Hq, a.Hkv);
  const int64_t wg_per_bkv = (slots + kWaves - 1) / kWaves;
  if (wg_per_bkv > 0x7fffffff || p.B * p.Hkv > 0x7fffffff || (int64_t)TB * p.Hq > 0x7fffffff)
    return hipErrorInvalidValue;
  a.wg_per_bkv = (int)wg_per_bkv;
  a.n_bkv = (int)(p.B * p.Hkv);
  int64_t nwg = (int64_t)a.wg_per_bkv * a.n_bkv;
  a.exact_per_batch = 0;
  if (uneven && !a.spread) {
    int64_t per = 0;
    for (int j = 0; j < a.Hkv; ++j) per += group_wgs(j, a.Hq, a.Hkv, TB, kWaves);
    if (per > 0x7fffffff) return hipErrorInvalidValue;
    a.exact_per_batch = (int)per;
    nwg = per * p.B;
  }
  a.pair_major = (p.cu_seqlens != nullptr && !p.causal) ? 1 : 0;  // as the d = 64 kernel
  if (a.pair_major) nwg = pair_major_nwg(a.n_bkv, a.wg_per_bkv);
  if (nwg > 0x7fffffff) return hipErrorInvalidValue;
  a.nwg = (int)nwg;
  a.c = fmaxf(fabsf(p.scale) * 1.4426950408889634f, kMinC);
  a.qsign = (p.scale < 0.f) ? 0x80008000u : 0u;
  a.causal = p.causal;
  a.nsplit = p.nsplit < 1 ? 1 : p.nsplit;
  a.part = p.split_ws;
  a.rows = p.cu_seqlens != nullptr ? p.Hq * p.T : p.B * p.Hq * p.N;
  if (a.nsplit > 1 && a.part == nullptr) return hipErrorInvalidValue;
  // with splits the grid covers whole runs of 8 (see the kernel's decode)
  const int64_t grid = a.nsplit == 1 ? a.nwg : ((int64_t)a.nwg + 7) / 8 * 8 * a.nsplit;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (!p.dry_run) {
    hipLaunchKernelGGL(attn_fwd_bf16_d128_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.nsplit == 1) return hipSuccess;
  SplitMergeArgs m;
  m.part = a.part;
  m.o = a.o;
  m.lse = a.lse;
  m.cu = a.cu;
  m.T = a.T;
  m.rows = a.rows;
  m.N = a.N;
  m.B = (int)p.B;
  m.nsplit = a.nsplit;
  m.causal = a.causal;
  m.tile_keys = kTileKeys;
  m.min_tiles = kMinSplitTiles;
  m.even = 0;
  return launch_split_merge<D>(m, stream, p.dry_run);
}

}  // namespace sqa
