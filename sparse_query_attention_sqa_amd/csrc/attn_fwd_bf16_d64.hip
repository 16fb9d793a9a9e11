// SQA attention forward for head dim 64, bf16 in/out, gfx950: the
// software-pipelined kernel used for the long-sequence workloads.
//
// Operation: query head i attends K/V head floor(i*H_kv/H_q) (contiguous
// query-head groups, "GQA ..." page, "The idea"), with fewer query heads than
// the baseline (SQA paper abstract); encoder-style or causal.
//
// Decomposition: a workgroup is 4 waves that share one (batch, K/V head);
// each wave owns 64 query positions of one query head of the group (slots
// ordered by position block, then head-in-group), so one K/V tile in LDS
// feeds 256 query rows, and for groups of g >= 2 heads those rows come from
// different query heads -- the reuse the grouping offers. Groups may differ
// in size by one head (H_kv need not divide H_q) and packed batches have
// sequences of different lengths: the grid is sized for the largest group
// and the longest sequence, and workgroups with no rows leave at once.
// With key-range splits (nsplit > 1) each row block's keys are cut into
// ranges of an even number of tiles, one workgroup per range; a range's
// workgroup runs the same pipeline on shifted pointers and leaves fp32
// partial softmax states that attn_split_merge_kernel (split_merge.h)
// combines.
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
// (A = K tile from LDS, B = Q in registers), so the score accumulator already
// is the B operand of O^T += V^T P^T and probabilities never leave registers.
// K rows sit in LDS under the permutation pi, making each lane's 16 scores 16
// consecutive keys.
//
// Schedule. At d = 64 the softmax VALU work per score (one v_exp_f32 at half
// rate plus ~2.5 other VALU ops) costs about as much issue time as the MFMA
// work per score, and the two overlap only when independent MFMA and VALU
// instructions are interleaved. Each wave's 64 rows are two 32-row halves in
// a two-phase pipeline over 32-key tiles j:
//
//   phase A(j): MFMA  P(j-1,h1).V(j-1)  and  S(j,h1) = K(j).Q(h1)
//               VALU  softmax of S(j,h0)                -> P(j,h0)
//   phase B(j): MFMA  P(j,h0).V(j)      and  S(j+1,h0) = K(j+1).Q(h0)
//               VALU  softmax of S(j,h1)                -> P(j,h1)
//
// with sched_group_barrier hints alternating one MFMA with six VALU ops.
//
// Data movement. K and V tiles go straight from HBM to LDS with
// buffer_load ... lds (no register staging), into a 6-slot ring with one
// barrier per two tiles: at the barrier of odd tile j every wave has read
// tile j and everything before it, tiles up to j+3 have landed, and tiles
// j+5 and j+6 are issued into the two slots just freed (tile j+4 is still in
// flight). Measured against one barrier per tile (5 slots): 1045 -> 1065
// TFLOP/s encoder-style and 946 -> 961 causal at N = 32768, (8,4), on one
// box; packed batches unchanged. The buffer descriptor's range
// check zero-fills keys past N. Both tiles are stored row-major (128 B rows)
// with an XOR swizzle of their 16-byte chunks; K fragments are 16-byte
// ds_read_b128, and V^T fragments come from ds_read_b64_tr_b16, whose
// 16-lane transpose hands each lane 4 consecutive keys of one head-dim
// column. K(j+1) is already resident during phase A(j), so its fragments are
// read there, ahead of the MFMAs of phase B(j) that use them. With the loop
// unrolled over the ring slots every LDS address is a per-lane register plus
// an immediate, so the barrier block has no VALU work.
//
// Softmax. fp32, base-2 exponentials of s*c - m with c = |scale|*log2(e);
// probabilities are rounded to bf16 (nearest even) for the P.V MFMA and the
// row sum adds the same rounded values (v_dot2c_f32_bf16, two partial sums).
// The running
// maximum m is raised lazily: probabilities are computed against the current
// m and only if a lane's sum of its 16 probabilities exceeds 2^20 (or is not
// finite, as on the first tile where m = -inf) is the exact row maximum
// taken, O and l rescaled and the tile recomputed; between refreshes every
// probability is <= 2^20, far inside the bf16/fp32 range. Masked scores
// (causal key > t, tail key >= N) are replaced by a large negative value,
// only on diagonal and tail tiles, so one branch-free phase body serves all
// tiles.
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

constexpr int D = 64;
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 64;
constexpr int kTileKeys = 32;                      // keys per K/V tile
constexpr int kRowBytes = D * 2;                   // 128 B per key row
constexpr int kTileBytes = kTileKeys * kRowBytes;  // 4 KB (K or V)
constexpr int kSlotBytes = 2 * kTileBytes;         // K then V
constexpr int NBUF = 6;                            // ring slots
constexpr int kXcds = 8;
constexpr float kSumLimit = 1048576.0f;            // 2^20
constexpr float kMaskedScore = -3.0e38f;
constexpr float kMinC = 1e-30f;                    // |scale|*log2(e) is clamped up to this
constexpr int kBufferWord3 = 0x00020000;           // raw buffer descriptor flags (gfx9)

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
  int pair_major;              // packed encoder-style: pair_major_coords order
  float c;
  uint32_t qsign;
  int causal;
  int nsplit;    // key-range splits per workgroup's rows (1: none)
  float* part;   // nsplit > 1: [nsplit][rows][64] unnormalised O, then [nsplit][rows][2] (m, l)
  int64_t rows;  // query rows: B*Hq*N (packed: Hq*T)
  // tail split (dense encoder-style, nsplit == 1): logical workgroups from
  // tail_start on run as tail_split workgroups each, one per key range,
  // leaving partial states in tail_part ([tail_split][units*256][64], then
  // [tail_split][units*256][2]) for attn_tail_merge_kernel
  int tail_start, tail_split;
  float* tail_part;
};

// MFMA row r of a K tile holds key pi(r), so that S^T entry i of lane-half lg
// is key lg*16 + i.
__device__ __forceinline__ int pi_row(int r) { return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3); }
// 16-byte chunk swizzles of the K and V tiles (bank-conflict-free reads)
__device__ __forceinline__ int swz_k(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_v(int r) { return 2 * (r & 3); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Wait for this wave's LDS reads and for all but the newest tile's DMA (or
// for every DMA), then synchronise the workgroup.
__device__ __forceinline__ void wait_vm_then_barrier(bool keep_one_tile) {
  asm volatile("" ::: "memory");
  if (keep_one_tile)
    __builtin_amdgcn_s_waitcnt(0x0072);  // vmcnt(2) lgkmcnt(0)
  else
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The ring slots are separate __shared__ objects so that the compiler can
// tell an LDS read of one slot from the DMA still in flight into another.
struct Ring {
  uint8_t* p[NBUF];
};

struct Lane {
  int l32, lg;
  uint32_t voff_k, voff_v;  // DMA source offsets within a tile (bytes)
  uint32_t koff[4];         // K fragment LDS offsets within a slot
  uint32_t voffr[2];        // V^T transposed-read LDS offsets within a slot (x = 0, 1)
};

struct WaveState {
  u32x4_t qf[2][4];
  f32x16_t acc_o[2][2];  // [half][x]
  float m_run[2], l_run[2];
  u32x4_t kf[4];
  u32x4_t vf[2][2];
  f32x16_t sA, sB;
  u32x4_t pk0[2], pk1[2];
};

// DMA K/V tile kt into ring slot SLOT: one 16-byte chunk per lane of each.
template <int SLOT>
__device__ __forceinline__ void issue_tile(const Ring& ring, const uint16_t* kbase, const uint16_t* vbase, int kt,
                                           int N, int wave, const Lane& ln) {
  const int key0 = kt * kTileKeys;
  const int rem = max(N - key0, 0) * kRowBytes;  // bytes of this head from key0 on
  __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (size_t)key0 * D), (short)0, rem, kBufferWord3);
  __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (size_t)key0 * D), (short)0, rem, kBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(ring.p[SLOT] + wave * 1024), 16, ln.voff_k, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(ring.p[SLOT] + kTileBytes + wave * 1024), 16,
                                           ln.voff_v, 0, 0, 0);
}

template <int SLOT>
__device__ __forceinline__ void read_k(const Ring& ring, const Lane& ln, u32x4_t (&kf)[4]) {
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) kf[ds] = *reinterpret_cast<const u32x4_t*>(ring.p[SLOT] + ln.koff[ds]);
}

// V^T fragments [x][hh]: the 8 keys lg*16 + hh*8 + 0..7 of head-dim row
// x*32 + l32, as two transposed 4-key reads.
template <int SLOT>
__device__ __forceinline__ void read_v(const Ring& ring, const Lane& ln, u32x4_t (&vf)[2][2]) {
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint8_t* p = ring.p[SLOT] + kTileBytes + ln.voffr[x] + hh * 8 * kRowBytes;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * kRowBytes));
      const u32x2_t a = __builtin_bit_cast(u32x2_t, lo);
      const u32x2_t b = __builtin_bit_cast(u32x2_t, hi);
      vf[x][hh] = u32x4_t{a[0], a[1], b[0], b[1]};
    }
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

// Scores of keys a query may not see (causal: key > t; tail: key >= N)
// become kMaskedScore, whose probability underflows to exactly 0 for any
// c >= kMinC. Only diagonal and tail tiles need this.
__device__ __forceinline__ void mask_scores(f32x16_t& s, int key0, int N, int causal, int t, int lg) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = key0 + lg * 16 + i;
    if (!(key < N && (!causal || key <= t))) s[i] = kMaskedScore;
  }
}

// probabilities of one 32-row half against the current maximum m, rounded to
// bf16 and packed as the B operand of O^T += V^T P^T; returns the lane's sum
// of its 16 rounded probabilities.
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

// Finish the softmax of one half: if a lane's probabilities grew too large
// (or m was still -inf), take the exact row maximum, rescale O and l and
// recompute the tile's probabilities.
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

struct Ctx {
  Ring ring;
  const uint16_t* kbase;
  const uint16_t* vbase;
  int N, nt, last, diag0, causal, wave;
  int t0, t1;
  float c;
};

// One pipeline step over tile j, whose K/V sit in ring slot SLOT = j % NBUF;
// BAR (odd j) steps hold the workgroup barrier, the others a scheduling
// barrier in its place so that both phases keep their own regions.
template <int SLOT, bool BAR>
__device__ __forceinline__ void step(const Ctx& cx, const Lane& ln, WaveState& w, int j) {
  constexpr int NEXT = (SLOT + 1) % NBUF;
  constexpr int PREV = (SLOT + NBUF - 1) % NBUF;
  const int key0 = j * kTileKeys;
  const bool active = j <= cx.last;
  const bool masked = (cx.causal && j >= cx.diag0) || (key0 + kTileKeys > cx.N);

  // ---------------- phase A(j)
  if (active) {
    if (masked) mask_scores(w.sB, key0, cx.N, cx.causal, cx.t0, ln.lg);
    mfma_pv(w.vf, w.pk1, w.acc_o[1]);  // P(j-1,h1) V(j-1)
    read_v<SLOT>(cx.ring, ln, w.vf);   // V(j), used from phase B on
    mfma_s(w.kf, w.qf[1], w.sA);       // S(j,h1); K(j) is in kf
    read_k<NEXT>(cx.ring, ln, w.kf);   // K(j+1), resident since the last barrier
    const float ls = exp_half(w.sB, w.pk0, cx.c, w.m_run[0]);
    interleave_phase();
    finish_half(ls, w.sB, w.pk0, w.m_run[0], w.l_run[0], w.acc_o[0], cx.c);
  }

  // BAR: tiles up to j+3 must have landed (tile j+4 may still be in flight),
  // for the reads of phases A(j+1) and A(j+2); every wave is done with tiles
  // j-1 and j, whose slots receive tiles j+5 and j+6.
  if (BAR) {
    wait_vm_then_barrier(true);
    issue_tile<PREV>(cx.ring, cx.kbase, cx.vbase, j + 5, cx.N, cx.wave, ln);
    issue_tile<SLOT>(cx.ring, cx.kbase, cx.vbase, j + 6, cx.N, cx.wave, ln);
  } else {
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---------------- phase B(j)
  if (active) {
    if (masked) mask_scores(w.sA, key0, cx.N, cx.causal, cx.t1, ln.lg);
    mfma_pv(w.vf, w.pk0, w.acc_o[0]);  // P(j,h0) V(j)
    mfma_s(w.kf, w.qf[0], w.sB);       // S(j+1,h0)
    const float ls = exp_half(w.sA, w.pk1, cx.c, w.m_run[1]);
    interleave_phase();
    finish_half(ls, w.sA, w.pk1, w.m_run[1], w.l_run[1], w.acc_o[1], cx.c);
  }
}

__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_d64_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring0[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring4[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ring5[kSlotBytes];
  Ring ring;
  ring.p[0] = ring0;
  ring.p[1] = ring1;
  ring.p[2] = ring2;
  ring.p[3] = ring3;
  ring.p[4] = ring4;
  ring.p[5] = ring5;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- workgroup -> (key-range split, batch*Hkv, slot range)
  // The hardware deals workgroups round-robin over the 8 XCDs. Runs of 8
  // consecutive workgroups take one split index, cycling over the splits, so
  // that the splits of logical workgroup wid all run on XCD wid % 8, close
  // together in time (a split index tied to blockIdx % nsplit would put, for
  // two splits, every first range -- under a causal mask most of the work --
  // on the even XCDs). With one split wid = blockIdx.x.
  // Tail split: blocks from tail_start on are the key ranges of the
  // logical workgroups past the last full round; the blocks before it map
  // the whole workgroups below tail_start as an unsplit launch would.
  const bool tail = a.tail_split > 1 && (int)blockIdx.x >= a.tail_start;
  const int nsplit = tail ? a.tail_split : a.nsplit;
  const int nwg_map = a.tail_split > 1 ? a.tail_start : a.nwg;
  const int g8 = (int)(blockIdx.x >> 3), x8 = (int)(blockIdx.x & 7);
  const int split = tail ? ((int)blockIdx.x - a.tail_start) % a.tail_split : g8 % a.nsplit;
  const int wid = tail ? a.tail_start + ((int)blockIdx.x - a.tail_start) / a.tail_split : (g8 / a.nsplit) * 8 + x8;
  if (wid >= a.nwg) return;
  int bkv, w_in;
  if (tail) {  // one logical workgroup per tail unit, in (batch*Hkv, index) order
    bkv = wid / a.wg_per_bkv;
    w_in = wid % a.wg_per_bkv;
  } else if (a.pair_major) {
    if (!pair_major_coords(wid, a.n_bkv, a.wg_per_bkv, bkv, w_in)) return;
  } else if (a.spread) {  // packed sequences, or uneven groups under a causal mask
    spread_coords(wid, a.n_bkv, a.wg_per_bkv, a.causal != 0, a.spread_block, bkv, w_in);
  } else if (a.exact_per_batch > 0) {  // uneven groups, encoder-style: XCD-contiguous, exact counts
    const int bid = wid;
    const int per = a.nwg / kXcds, rem = a.nwg % kXcds;
    const int x = bid % kXcds, i = bid / kXcds;
    exact_coords(x * per + min(x, rem) + i, a.exact_per_batch, a.Hq, a.Hkv,
                 (a.N + kRowsPerWave - 1) / kRowsPerWave, kWaves, bkv, w_in);
  } else if (!a.causal) {  // consecutive logical workgroups on one XCD (shared L2)
    const int bid = wid;
    const int per = nwg_map / kXcds, rem = nwg_map % kXcds;
    const int x = bid % kXcds, i = bid / kXcds;
    const int L = x * per + min(x, rem) + i;
    bkv = L / a.wg_per_bkv;
    w_in = L % a.wg_per_bkv;
  } else {  // longest (largest position block) first
    const int L = wid;
    const int wr = L / a.n_bkv;
    bkv = L % a.n_bkv;
    w_in = a.wg_per_bkv - 1 - wr;
  }
  const int b = bkv / a.Hkv, kvh = bkv % a.Hkv;
  const HeadGroup hg = head_group(kvh, a.Hq, a.Hkv);
  const SeqGeom sg = seq_geom(a.cu, a.T, a.N, b, a.Hq, a.Hkv);
  const int N = sg.n, g = hg.count;
  const int TB = (N + kRowsPerWave - 1) / kRowsPerWave;  // 64-row query blocks
  const int NT = (N + kTileKeys - 1) / kTileKeys;        // 32-key tiles
  // workgroups past this group's (or this sequence's) rows leave at once
  if (w_in * kWaves >= TB * g) return;
  const int slot = w_in * kWaves + wave;
  const int tb = slot / g, jh = slot % g;
  const bool wave_valid = tb < TB;
  const int h = hg.first + jh;
  // key tiles the workgroup streams, and the last one this wave computes
  // (-1: none). A causal wave's rows end at key tile 2*tb+1.
  const int maxtb = min((w_in * kWaves + kWaves - 1) / g, TB - 1);
  const int nt_all = a.causal ? min(2 * maxtb + 2, NT) : NT;
  const int last_all = !wave_valid ? -1 : (a.causal ? min(2 * tb + 1, NT - 1) : NT - 1);
  // Key-range split: this workgroup takes key tiles [kt0, kt0 + chunk) of
  // its rows. Below, tiles, keys, N and the causal positions are counted
  // from kt0, so the pipeline runs unchanged on the shifted range. With an
  // even chunk a causal wave either has a visible key for all its rows in
  // this range (kt0 <= 2*tb) or none (last = -1).
  const int chunk = split_chunk(NT, nsplit);
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
      ln.koff[ds] = (uint32_t)(ln.l32 * kRowBytes + (((ds * 2 + ln.lg) ^ swz_k(ln.l32)) * 16));
    const int j16 = lane & 15, g1 = (lane >> 4) & 1;
    const int row = ln.lg * 16 + (j16 >> 2);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int c16 = x * 4 + 2 * g1 + ((j16 & 3) >> 1);
      ln.voffr[x] = (uint32_t)(row * kRowBytes + ((c16 ^ swz_v(row)) * 16) + (j16 & 1) * 8);
    }
  }

  const int64_t kvrow0 = sg.kv_base + (int64_t)kvh * sg.stride;
  const int64_t qrow0 = sg.q_base + (int64_t)h * sg.stride;
  const uint16_t* kbase = a.k + (size_t)(kvrow0 + key_shift) * D;
  const uint16_t* vbase = a.v + (size_t)(kvrow0 + key_shift) * D;
  const int Nk = N - key_shift;  // keys of this sequence from the range start on
  const size_t qoff = (size_t)qrow0 * D;

  WaveState w;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int t = min(trow0 + qs * 32 + ln.l32, N - 1);
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (wave_valid) x = *reinterpret_cast<const u32x4_t*>(a.q + qoff + (size_t)t * D + (ds * 2 + ln.lg) * 8);
      x ^= a.qsign;
      w.qf[qs][ds] = x;
    }
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int i = 0; i < 16; ++i) w.acc_o[hh][x][i] = 0.f;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    w.pk1[x] = u32x4_t{0u, 0u, 0u, 0u};  // P(-1,h1) = 0: the first phase A's P.V is a no-op
    w.vf[x][0] = u32x4_t{0u, 0u, 0u, 0u};
    w.vf[x][1] = u32x4_t{0u, 0u, 0u, 0u};
  }
  w.m_run[0] = w.m_run[1] = -INFINITY;
  w.l_run[0] = w.l_run[1] = 0.f;

  // zero the ring once so that no LDS byte is ever uninitialised
#pragma unroll
  for (int sl = 0; sl < NBUF; ++sl)
    for (int e = tid; e < kSlotBytes / 16; e += kThreads)
      reinterpret_cast<u32x4_t*>(ring.p[sl])[e] = u32x4_t{0u, 0u, 0u, 0u};
  wait_vm_then_barrier(false);

  // prologue: tiles 0..2 landed, then tiles 3..5 in flight, S(0,h0)
  issue_tile<0>(ring, kbase, vbase, 0, Nk, wave, ln);
  issue_tile<1>(ring, kbase, vbase, 1, Nk, wave, ln);
  issue_tile<2>(ring, kbase, vbase, 2, Nk, wave, ln);
  wait_vm_then_barrier(false);
  issue_tile<3>(ring, kbase, vbase, 3, Nk, wave, ln);
  issue_tile<4>(ring, kbase, vbase, 4, Nk, wave, ln);
  issue_tile<5>(ring, kbase, vbase, 5, Nk, wave, ln);

  Ctx cx;
  cx.ring = ring;
  cx.kbase = kbase;
  cx.vbase = vbase;
  cx.N = Nk;
  cx.nt = nt;
  cx.last = last;
  cx.diag0 = 2 * tb - kt0;
  cx.causal = a.causal;
  cx.wave = wave;
  cx.t0 = trow0 + ln.l32 - key_shift;
  cx.t1 = trow0 + 32 + ln.l32 - key_shift;
  cx.c = a.c;

  read_k<0>(ring, ln, w.kf);
  mfma_s(w.kf, w.qf[0], w.sB);

  // Whole turns of the ring: steps past the last tile only barrier and issue
  // their DMAs (zero-filled, no memory access), so that every path issues the
  // same VMEM sequence and the compiler's own waits before LDS reads are exact
  // (with the DMAs of the last turn conditional it waited for every DMA before
  // the reads of one slot in six: 1033 -> 1045 TFLOP/s at 32k (8,4)).
  for (int j = 0; j < nt; j += NBUF) {
    step<0, false>(cx, ln, w, j);
    step<1, true>(cx, ln, w, j + 1);
    step<2, false>(cx, ln, w, j + 2);
    step<3, true>(cx, ln, w, j + 3);
    step<4, false>(cx, ln, w, j + 4);
    step<5, true>(cx, ln, w, j + 5);
  }
  if (last >= 0) mfma_pv(w.vf, w.pk1, w.acc_o[1]);  // drain P(last,h1) V(last)
  __builtin_amdgcn_s_waitcnt(0x0070);  // no DMA may outlive the workgroup

  if (!wave_valid) return;

  if (split_rows) {
    // ---- split epilogue: unnormalised O^T, m and l of this key range (fp32);
    // the merge kernel combines the ranges. A wave with no key in this range
    // writes nothing; the merge knows which ranges a row sees.
    if (last < 0) return;
    // partial rows: the global query rows, or (tail) the compact rows of
    // the tail units, 256 per unit: row trow0 + r of this wave is compact
    // row (unit * 4 + wave) * 64 + r
    const int64_t prows = tail ? (int64_t)(a.nwg - a.tail_start) * (kWaves * kRowsPerWave) : a.rows;
    const int64_t prow0 = tail ? ((int64_t)(wid - a.tail_start) * kWaves + wave) * kRowsPerWave : qrow0 + trow0;
    float* const part = tail ? a.tail_part : a.part;
    float* po = part + ((size_t)split * prows + prow0) * D;
    float* pml = part + (size_t)nsplit * prows * D + ((size_t)split * prows + prow0) * 2;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const float ltot = w.l_run[qs] + __shfl_xor(w.l_run[qs], 32);
      const int r = qs * 32 + ln.l32;
      if (trow0 + r < N) {
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int ab = 0; ab < 4; ++ab) {
            const f32x4_t v4 = {w.acc_o[qs][x][4 * ab], w.acc_o[qs][x][4 * ab + 1], w.acc_o[qs][x][4 * ab + 2],
                                w.acc_o[qs][x][4 * ab + 3]};
            *reinterpret_cast<f32x4_t*>(po + (size_t)r * D + x * 32 + 8 * ab + 4 * ln.lg) = v4;
          }
        if (ln.lg == 0) *reinterpret_cast<f32x2_t*>(pml + (size_t)r * 2) = f32x2_t{w.m_run[qs], ltot};
      }
    }
    return;
  }

  // ---- epilogue: O = O^T / l (bf16, nearest even); LSE = m ln2 + ln l
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const float ltot = w.l_run[qs] + __shfl_xor(w.l_run[qs], 32);
    const float inv = 1.0f / ltot;
    const int t = trow0 + qs * 32 + ln.l32;
    if (t < N) {
      uint16_t* orow = a.o + qoff + (size_t)t * D;
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int ab = 0; ab < 4; ++ab) {
          // accumulator entries 4ab..4ab+3 are head dims x*32 + 8ab + 4lg + 0..3
          u32x2_t wv;
          wv[0] = pack_bf16x2(w.acc_o[qs][x][4 * ab] * inv, w.acc_o[qs][x][4 * ab + 1] * inv);
          wv[1] = pack_bf16x2(w.acc_o[qs][x][4 * ab + 2] * inv, w.acc_o[qs][x][4 * ab + 3] * inv);
          *reinterpret_cast<u32x2_t*>(orow + x * 32 + 8 * ab + 4 * ln.lg) = wv;
        }
      if (a.lse != nullptr && ln.lg == 0)
        a.lse[(size_t)qrow0 + t] = (w.m_run[qs] + log2f(ltot)) * 0.69314718055994531f;
    }
  }
}

// Merge of the tail split: the key ranges of every compact row of the tail
// units (256 per unit, unit u = logical workgroup tail_start + u, row
// (u * 4 + wave) * 64 + r is query row trow0 + r of that wave's slot), with
// the streaming-softmax merge of split_merge.h. Dense encoder-style
// launches with equal head groups only, so every range holds keys of every
// row. 16 lanes per row, lane j holding head dims 4j..4j+3.
struct TailMergeArgs {
  const float* part;  // [S][rows][64] O, then [S][rows][2] (m, l)
  uint16_t* o;
  float* lse;
  int64_t rows;  // compact rows: (nwg - tail_start) * 256
  int tail_start, S, N, Hq, Hkv, wg_per_bkv;
};

__global__ __launch_bounds__(256) void attn_tail_merge_kernel(TailMergeArgs a) {
  typedef float f4_t __attribute__((ext_vector_type(4)));
  const int64_t cr = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;
  const int j = threadIdx.x % 16;
  if (cr >= a.rows) return;
  const int unit = (int)(cr / (kWaves * kRowsPerWave)), wave = (int)(cr / kRowsPerWave) % kWaves;
  const int r = (int)(cr % kRowsPerWave);
  const int L = a.tail_start + unit;
  const int bkv = L / a.wg_per_bkv, w_in = L % a.wg_per_bkv;
  const int b = bkv / a.Hkv, kvh = bkv % a.Hkv, g = a.Hq / a.Hkv;
  const int slot = w_in * kWaves + wave, tb = slot / g, jh = slot % g;
  const int t = tb * kRowsPerWave + r;
  if (t >= a.N) return;  // also every slot past the last position block
  const int64_t orow = ((int64_t)b * a.Hq + kvh * g + jh) * a.N + t;
  const int NT = (a.N + kTileKeys - 1) / kTileKeys;
  const int chunk = split_chunk(NT, a.S);
  const float* pml = a.part + (size_t)a.S * a.rows * D;
  float M = -INFINITY;
  for (int s = 0; s < a.S && s * chunk < NT; ++s) M = fmaxf(M, pml[((size_t)s * a.rows + cr) * 2]);
  float Lsum = 0.f;
  f4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.S && s * chunk < NT; ++s) {
    const f32x2_t ml = *reinterpret_cast<const f32x2_t*>(pml + ((size_t)s * a.rows + cr) * 2);
    const float wgt = __builtin_amdgcn_exp2f(ml[0] - M);
    Lsum += wgt * ml[1];
    acc += wgt * *reinterpret_cast<const f4_t*>(a.part + ((size_t)s * a.rows + cr) * D + 4 * j);
  }
  const float inv = 1.0f / Lsum;
  u32x2_t wv;
  wv[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  wv[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2_t*>(a.o + (size_t)orow * D + 4 * j) = wv;
  if (a.lse != nullptr && j == 0) a.lse[orow] = (M + log2f(Lsum)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_attn_fwd_bf16_d64(const AttnProblem& p, hipStream_t stream) {
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
  // packed encoder-style: pair-major order (seq_groups.h). Measured on the
  // packed 32k batch, unsplit: (8,4) 793 -> 862 TFLOP/s, (16,16) 746 -> 984
  // against the rotating spread order, whose workgroups on one XCD came from
  // many pairs (L2 hit rate 0.37).
  a.pair_major = (p.cu_seqlens != nullptr && !p.causal) ? 1 : 0;
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
  a.tail_start = 0;
  a.tail_split = 0;
  a.tail_part = nullptr;
  if (p.tail_split > 1) {
    // only where attn_fwd_tail_plan would plan one: dense, encoder-style,
    // equal head groups, unsplit
    if (p.cu_seqlens != nullptr || p.causal || uneven || a.nsplit != 1 || p.tail_ws == nullptr ||
        p.tail_units <= 0 || p.tail_units > a.nwg || p.tail_split > kMaxTailSplit)
      return hipErrorInvalidValue;
    a.tail_start = a.nwg - (int)p.tail_units;
    a.tail_split = p.tail_split;
    a.tail_part = p.tail_ws;
  }
  // with splits the grid covers whole runs of 8 (see the kernel's decode)
  const int64_t grid = a.tail_split > 1 ? (int64_t)a.tail_start + p.tail_units * p.tail_split
                       : a.nsplit == 1  ? a.nwg
                                        : ((int64_t)a.nwg + 7) / 8 * 8 * a.nsplit;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (!p.dry_run) {
    hipLaunchKernelGGL(attn_fwd_bf16_d64_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.tail_split > 1) {
    TailMergeArgs t;
    t.part = a.tail_part;
    t.o = a.o;
    t.lse = a.lse;
    t.rows = p.tail_units * (kWaves * kRowsPerWave);
    t.tail_start = a.tail_start;
    t.S = a.tail_split;
    t.N = a.N;
    t.Hq = a.Hq;
    t.Hkv = a.Hkv;
    t.wg_per_bkv = a.wg_per_bkv;
    const int64_t blocks = (t.rows + 15) / 16;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (p.dry_run) return hipSuccess;
    hipLaunchKernelGGL(attn_tail_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, t);
    return hipGetLastError();
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
  m.even = 1;
  return launch_split_merge<D>(m, stream, p.dry_run);
}

// Recommended key-range splits for this kernel, from measurements on MI355X
// (B=1, N=32768 and a packed 32k batch whose longest sequence has 18496
// tokens, d=64; TFLOP/s unsplit -> 2 / 3 / 4 splits):
//  * encoder-style packed (8,4) 766 -> 845 / 834 / 825, (16,16) 740 -> 874 /
//    803 / 830; dense (6,4) 1005 -> 1021;
//  * causal packed (8,4) 788 -> 650 / 755 / 580, dense (6,4) 939 -> 764: the
//    longest-first order already balances causal launches, and split
//    workgroups ran slower per tile, so causal launches are never split.
// Dense: the workgroups run in rounds of 2 * cus (two per CU), r =
// workgroups / slots. When the whole launch fits in one round, split as far
// as 4 ways while it still does; otherwise take two splits when they cut
// the whole-row rounds, ceil(r) -> ceil(2r)/2, by at least 10 %. Packed
// batch (T > 0 tokens, N the longest sequence), launched in pair-major
// order: two splits when packed_wants_split and the longest sequence's own
// workgroups fill between one and two rounds (r of B = 1), where its last
// round is left mostly empty; with more rounds the other sequences fill the
// tail (measured, pair-major, 2 ranges: (8,4) 845 -> 928 TFLOP/s at 1.13
// rounds, (16,16) 971 -> 904 at 2.28).
int attn_fwd_auto_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t T, bool causal, int cus,
                         int rows_per_wave) {
  if (causal) return 1;
  const int64_t NT = (N + kTileKeys - 1) / kTileKeys, TB = (N + rows_per_wave - 1) / rows_per_wave;
  int64_t wgs = 0;
  for (int j = 0; j < Hkv; ++j) wgs += group_wgs(j, (int)Hq, (int)Hkv, (int)TB, kWaves);
  const double slots = 2.0 * (cus > 0 ? cus : 256);
  if (T > 0) {
    const double r1 = (double)wgs / slots;
    return (packed_wants_split(N, T) && r1 > 1.0 && r1 < 2.0 && ceil(2.0 * r1) / 2.0 <= 0.9 * ceil(r1)) ? 2 : 1;
  }
  const double r = (double)(wgs * B) / slots;
  for (int S = 4; S >= 2; --S)
    if (S * r <= 1.0 && NT >= (int64_t)S * kMinSplitTiles) return S;
  if (NT >= 2 * kMinSplitTiles && ceil(2.0 * r) / 2.0 <= 0.9 * ceil(r)) return 2;
  return 1;
}

bool packed_wants_split(int64_t N, int64_t T) {
  return N >= 2 * kMinSplitTiles * kTileKeys && 4 * N >= T;
}

// Tail split of dense encoder-style launches (measured at N = 200000,
// (4,4): 3128 workgroups over 512 slots, a last round of 56). The
// workgroups fill rounds of 2 * cus slots; the R whole rounds run unsplit
// and the r workgroups past them, when they fill at most half a round,
// run as r * S workgroups of one key range each, S = floor(2 * cus / r)
// (at most kMaxTailSplit, each range at least kMinSplitTiles tiles):
// their last round then takes about 1/S of a whole workgroup's time.
// Equal head groups, bf16, d = 64 only. Returns S (0: no tail split) and
// the number of tail workgroups.
int attn_fwd_tail_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, bool causal, int cus, int64_t* units) {
  *units = 0;
  if (causal || B <= 0 || N <= 0 || Hkv <= 0 || Hq % Hkv != 0) return 0;
  const int64_t TB = (N + kRowsPerWave - 1) / kRowsPerWave, NT = (N + kTileKeys - 1) / kTileKeys;
  const int64_t nwg = (TB * (Hq / Hkv) + kWaves - 1) / kWaves * B * Hkv;
  const int64_t slots = 2 * (int64_t)(cus > 0 ? cus : 256);
  const int64_t r = nwg % slots;
  if (nwg < slots || r == 0 || 2 * r > slots) return 0;
  int64_t S = slots / r;
  if (S > kMaxTailSplit) S = kMaxTailSplit;
  while (S > 1 && NT < S * kMinSplitTiles) --S;
  if (S < 2) return 0;
  *units = r;
  return (int)S;
}

size_t attn_tail_workspace_bytes(int64_t units, int S) {
  if (units <= 0 || S <= 1) return 0;
  return (size_t)S * (size_t)units * (kWaves * kRowsPerWave) * (size_t)(D + 2) * sizeof(float);
}

size_t attn_split_workspace_bytes(int64_t rows, int64_t d, int nsplit) {
  if (rows <= 0 || nsplit <= 1) return 0;
  return (size_t)nsplit * (size_t)rows * (size_t)(d + 2) * sizeof(float);
}

}  // namespace sqa
