// SQA attention backward for head dims 64 and 128, bf16 in/out, gfx950.
//
// Operation: the exact derivative of the forward (query head i attends K/V
// head floor(i*H_kv/H_q), "GQA ..." page, "The idea"; fewer query heads than
// the baseline, SQA paper abstract, whose gains are quoted for training).
// With P = softmax(S), S = scale Q K^T (masked), upstream gradient dO:
//   D_t  = sum_c dO[t,c] O[t,c]          (equals rowsum(P * dP))
//   dP   = dO V^T,   dS = P * (dP - D)
//   dQ   = scale dS K,   dK_j = scale sum_{i in group j} dS_i^T Q_i,
//   dV_j = sum_{i in group j} P_i^T dO_i.
// P is recomputed from the forward's log-sum-exp: P = 2^(s*c - lse*log2 e)
// with c = scale*log2 e.
//
// Three kernels, all on the caller's stream:
//   1. bwd_rowterms_kernel: per query row, -lse*log2(e)/c and -D into two
//      planes of the workspace; the other kernels start their S and dP
//      MFMA chains from them (S' = S - lse log2(e)/c, dP' = dP - D), so that
//      P = 2^(c S') and dS = P dP' take one VALU operation per score fewer.
//   2. bwd_dkdv_kernel (K/V-stationary): a wave holds 32 keys of one K/V head
//      (K and V as MFMA B operands in registers) and streams every query tile
//      of every query head of the group through LDS: S = Q K^T and
//      dP = dO V^T (A = Q / dO rows), then dV^T += dO^T P and
//      dK^T += Q^T dS (A = transposed reads of Q / dO). Because the wave sees
//      the whole group, the group sum needs no atomics.
//   3. bwd_dq_kernel (Q-stationary, like the forward): a wave holds 32 query
//      rows (Q, dO in registers) and streams K/V tiles: S^T = K Q^T,
//      dP^T = V dO^T, dQ^T += K^T dS^T.
// Both streamed operands are DMA'd HBM -> LDS (buffer_load ... lds) into a
// ring of tiles in the layouts of bf16_tiles.h, with one barrier per tile.
// Every DMA is issued unconditionally -- tiles past the last one needed get
// an empty descriptor range and cost no memory traffic -- so the explicit
// vmcnt waits are exact. P and dS are rounded to bf16 (nearest even) for the
// MFMA products; everything else accumulates in fp32.
// Encoder-style launches may split (nsplit > 1): the dK/dV kernel over
// ranges of query tiles, the dQ kernel over ranges of key tiles; each range
// leaves a scaled fp32 partial and bwd_split_sum_kernel adds them.
//
// Head dim 128 (DH = 2 halves of 64): every 32-row tile is stored as two
// 64-wide half-tiles, products over the head dim add the two halves, and the
// dK/dV and dQ accumulators hold four 32-dim tiles. The same code then needs
// about twice the registers, so the d = 128 kernels run one wave per SIMD.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "bf16_tiles.h"
#include "kernels.h"
#include "seq_groups.h"

namespace sqa {
namespace {

using namespace tiles;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;

// s_waitcnt immediate (gfx9 encoding): vmcnt vm, expcnt 7, lgkmcnt lgkm.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// Wait until at most VM of this wave's DMAs are in flight and its LDS reads
// are done, then synchronise the workgroup.
template <int VM>
__device__ __forceinline__ void barrier_vm() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, 0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per head-dim width: DH halves of 64.
template <int DH>
struct Dims {
  static constexpr int D = kD * DH;           // elements per row
  static constexpr int RB = kRowBytes * DH;   // bytes per row in HBM
  static constexpr int MINB = DH == 1 ? 2 : 1;  // workgroups per CU the registers allow
};

// ------------------------------------------------------------------ row terms
struct RowArgs {
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  float* rt;    // plane 0 [B*H_q, Np]: -lse log2(e)/c; plane 1 (nrows floats later): -D.
                // Every head's rows are padded to Np, a multiple of 32
  int64_t nrows;  // B*H_q*Np
  int N, Np;
  float inv_c;    // 1/c
};

// Eight lanes per query row: each forms the products of 8*DH bf16 pairs
// exactly (v_dot2_f32_bf16) and the eight partial sums are added with lane
// shuffles. Padding rows (t >= N) get 0 in both planes, so row-term tiles
// are always whole.
template <int DH>
__global__ __launch_bounds__(256) void bwd_rowterms_kernel(RowArgs a) {
  constexpr int D = Dims<DH>::D;
  const int64_t prow = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  const int64_t bh = prow / a.Np;
  const int t = (int)(prow - bh * a.Np);
  const bool valid = prow < a.nrows && t < a.N;
  const int64_t row = bh * a.N + t;
  float acc = 0.f;
  if (valid) {
#pragma unroll
    for (int h = 0; h < DH; ++h) {
      const u32x4_t ov = *reinterpret_cast<const u32x4_t*>(a.o + row * D + h * kD + part * 8);
      const u32x4_t dv = *reinterpret_cast<const u32x4_t*>(a.dout + row * D + h * kD + part * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // copy the elements out first: a bit cast of a vector-element
        // expression reads element 0
        const uint32_t ow = ov[w], dw = dv[w];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ow), __builtin_bit_cast(bf16x2_t, dw),
                                              acc, false);
      }
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (prow < a.nrows && part == 0) {
    a.rt[prow] = valid ? -(a.lse[row] * kLog2e) * a.inv_c : 0.f;
    a.rt[a.nrows + prow] = valid ? -acc : 0.f;
  }
}

// Workgroup -> (b*H_kv + K/V head, index w_in within that head).
// Encoder-style: consecutive logical workgroups on one XCD (they share the
// streamed operand in L2). Causal: workgroups launch largest-work first,
// which is ascending w_in, or descending with `reverse`. Uneven head groups
// or packed sequences (`spread`): the spread_coords order, which deals every
// group and sequence over all XCDs; packed encoder-style (`pair_major`): the
// pair_major_coords order (consecutive workgroups of an XCD share one pair's
// streamed operand in L2). Returns false for a logical index past its pair's
// last workgroup.
__device__ __forceinline__ bool wg_coords(int bid, int pair_major, int spread, int block, int causal, bool reverse,
                                          int nwg, int wg_per_bkv, int n_bkv, int& bkv, int& w_in) {
  if (pair_major) return pair_major_coords(bid, n_bkv, wg_per_bkv, bkv, w_in);
  if (spread) {
    spread_coords(bid, n_bkv, wg_per_bkv, causal && reverse, block, bkv, w_in);
  } else if (!causal) {
    const int per = nwg / kXcds, rem = nwg % kXcds;
    const int x = bid % kXcds, i = bid / kXcds;
    const int L = x * per + min(x, rem) + i;
    bkv = L / wg_per_bkv;
    w_in = L % wg_per_bkv;
  } else {
    const int L = bid;
    const int wr = L / n_bkv;
    bkv = L % n_bkv;
    w_in = reverse ? wg_per_bkv - 1 - wr : wr;
  }
  return true;
}

// Range splits (encoder-style only): runs of 8 consecutive workgroups take
// one split index, cycling over the splits, so that the splits of logical
// workgroup wid run on its XCD (wid % 8); with one split wid = blockIdx.x.
__device__ __forceinline__ void split_decode(int nsplit, int& split, int& wid) {
  const int g8 = (int)(blockIdx.x >> 3), x8 = (int)(blockIdx.x & 7);
  split = g8 % nsplit;
  wid = (g8 / nsplit) * 8 + x8;
}

// fp32 partial of one row from a transposed accumulator pair (layout of
// store_tr_row), times mul.
__device__ __forceinline__ void store_tr_row_f32(float* row, const f32x16_t (&o)[2], float mul, int lg) {
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int ab = 0; ab < 4; ++ab) {
      const f32x4_t v = {o[x][4 * ab] * mul, o[x][4 * ab + 1] * mul, o[x][4 * ab + 2] * mul, o[x][4 * ab + 3] * mul};
      *reinterpret_cast<f32x4_t*>(row + x * 32 + 8 * ab + 4 * lg) = v;
    }
}

// init + sum over the DH halves of A_rows(h) . B(h).
template <int DH>
__device__ __forceinline__ f32x16_t mfma_rows(const uint8_t* tile0, const ReadOffsets& ro, const u32x4_t (&b)[DH][4],
                                              const f32x16_t& init) {
  f32x16_t acc = init;
#pragma unroll
  for (int h = 0; h < DH; ++h) {
    u32x4_t a[4];
    read_rows(tile0 + h * kTileBytes, ro, a);
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) acc = mfma(a[ds], b[h][ds], acc);
  }
  return acc;
}

// ------------------------------------------------------------------ dK, dV
// A step s is one 32-row query tile of one query head of the group (steps
// ordered by query tile, then head). Software-pipelined over steps:
//   phase s: MFMA  dV^T += dO(s-1)^T P(s-1), dK^T += Q(s-1)^T dS(s-1), from
//                  transposed fragments read into registers in phase s-1,
//                  interleaved with
//            VALU  P(s) = 2^(c S'), dS(s) = P dP' (S' and dP' started from
//                  the row terms);
//            LDS   the transposed Q and dO fragments of step s for phase s+1;
//            then MFMA S'(s+1), dP'(s+1) into the registers the softmax has
//            just consumed (one score buffer keeps the d = 64 wave at two
//            waves per SIMD: 249 VGPRs).
// Q and dO of a step sit in LDS once each, in the shared layout of
// bf16_tiles.h (row reads for S and dP, transposed reads for dK and dV); six
// ring slots give four steps of lookahead.
constexpr int kKvBuf = 6;  // ring slots

template <int DH>
struct KvCfg {
  static constexpr int kQ = 0;                            // Q half-tiles
  static constexpr int kDo = DH * kTileBytes;             // dO half-tiles
  static constexpr int kRt = 2 * DH * kTileBytes;         // row terms
  static constexpr int kSlot = 2 * DH * kTileBytes + 1024;
  static constexpr int kDma = 2 * DH + 1;                 // DMA instructions per wave per step
};

struct KvArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* rt;   // row terms, plane 0 [B*H_q, Np] (-lse log2(e)/c), plane 1 rt_plane floats later (-D)
  int64_t rt_plane;
  uint16_t* dk;
  uint16_t* dv;
  const int* cu;  // packed sequence offsets (nullptr: dense)
  int64_t T;      // packed: total tokens
  int N, Np, Hq, Hkv, wg_per_bkv, n_bkv, nwg;  // N: the (longest) sequence; Np: row-term rows per head
  int spread;  // uneven head groups or packed sequences: spread_coords order
  int spread_block;  // its rotation block
  int pair_major;    // packed encoder-style: pair_major_coords order
  float c, scale;
  int causal;
  int nsplit;        // query-range splits (encoder-style only; 1: none)
  float* part_k;     // nsplit > 1: [nsplit][kv rows][D] fp32 partial dK (scaled), then dV
  float* part_v;
  int64_t kv_rows;   // B*Hkv*N (packed: Hkv*T)
};

struct KvRing {
  uint8_t* p[kKvBuf];
};

struct KvCtx {
  KvRing ring;
  const uint16_t* q;     // Q of sequence b, head 0
  const uint16_t* dout;  // dO of sequence b, head 0
  const float* rt;       // row terms of sequence b, head 0 (plane 0)
  int64_t stride, rt_stride;  // rows between heads of Q/dO and of the row terms
  uint32_t rt_plane_bytes;    // from plane 0 to plane 1
  int N, g, h0, qt0, kb, causal, wave, first;  // N: this sequence; first: the first step this wave computes
  int diag0;                  // causal: the first step of query tile kb (its g steps hold the diagonal)
  int64_t d_head, d_wrap;     // cursor moves (elements) to the next head / to head 0 of the next tile
  int64_t rt_wrap;            // the same in the row terms (to the next head: rt_stride)
  float c;
  float masked;  // score whose exponent s*c is -inf: -inf * sign(c)
  uint32_t off;
  ReadOffsets ro;
};

template <int DH>
struct KvState {
  u32x4_t kb_f[DH][4], vb_f[DH][4];   // K and V rows of this wave's 32 keys as B operands
  f32x16_t acc_k[DH][2], acc_v[DH][2];  // dK^T, dV^T
  f32x16_t sc, dp;                      // S and dP of the current step
  u32x4_t pk[2][2], dsk[2][2];          // P and dS of steps s-1 and s, packed as B operands
  u32x4_t qt_f[DH][2][2], dt_f[DH][2][2];  // transposed Q and dO fragments of the step whose dK/dV come next
};

// The source of the next step's DMA: step s is query tile qt0 + s / g of
// query head h0 + s % g, so the cursor walks the group's heads and then the
// next tile, by fixed moves (no division by g and no 64-bit product per step).
struct KvCursor {
  int64_t off;     // elements into Q and dO: head h0 + i, row row0
  int64_t rt_off;  // floats into the row terms: the same head and row
  int row0, i;
};

__device__ __forceinline__ void kv_advance(const KvCtx& cx, KvCursor& u) {
  const bool wrap = u.i + 1 == cx.g;
  u.i = wrap ? 0 : u.i + 1;
  u.row0 += wrap ? kTileRows : 0;
  u.off += wrap ? cx.d_wrap : cx.d_head;
  u.rt_off += wrap ? cx.rt_wrap : cx.rt_stride;
}

// DMA the step at cursor u into ring slot SLOT, then move u to the next step.
template <int DH, int SLOT>
__device__ __forceinline__ void kv_issue(const KvCtx& cx, KvCursor& u) {
  using C = KvCfg<DH>;
  constexpr int RB = Dims<DH>::RB;
  const int row0 = u.row0;
  uint8_t* slot = cx.ring.p[SLOT];
  const float* rb = cx.rt + u.rt_off - row0;
  const int trem = max(cx.N - row0, 0) * RB;
#pragma unroll
  for (int h = 0; h < DH; ++h) {
    __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void*)(cx.q + u.off), (short)0, trem, kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void_t*)(slot + C::kQ + h * kTileBytes + cx.wave * 1024), 16,
                                             cx.off + h * kRowBytes, 0, 0, 0);
    __amdgpu_buffer_rsrc_t rd =
        __builtin_amdgcn_make_buffer_rsrc((void*)(cx.dout + u.off), (short)0, trem, kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void_t*)(slot + C::kDo + h * kTileBytes + cx.wave * 1024), 16,
                                             cx.off + h * kRowBytes, 0, 0, 0);
  }
  // row terms of the 32 rows (whole tiles stay inside the planes thanks to
  // their padding) land in the first 256 B of the area: lanes 0-7 bring
  // plane 0's 128 B, lanes 8-15 plane 1's; every wave writes the same bytes
  // (lanes past 16 are out of range and write zeros beyond them)
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t roff = lane < 8 ? lane * 16u : (lane < 16 ? cx.rt_plane_bytes + (lane - 8) * 16u : 0x80000000u);
  const int rem = row0 < cx.N ? (int)cx.rt_plane_bytes + kTileRows * 4 : 0;
  __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(rb + row0), (short)0, rem, kBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(slot + C::kRt), 16, roff, 0, 0, 0);
  kv_advance(cx, u);
}

// S' = S - lse log2(e)/c and dP' = dP - D of the step in slot SLOT: the
// chains start from the step's row terms (entry e <-> query row lg*16 + e).
template <int DH, int SLOT>
__device__ __forceinline__ void kv_scores(const KvCtx& cx, KvState<DH>& w) {
  using C = KvCfg<DH>;
  const int lg = (threadIdx.x & 63) >> 5;
  const f32x4_t* r0 = reinterpret_cast<const f32x4_t*>(cx.ring.p[SLOT] + C::kRt + lg * 64);
  const f32x4_t* r1 = reinterpret_cast<const f32x4_t*>(cx.ring.p[SLOT] + C::kRt + 128 + lg * 64);
  f32x16_t i0, i1;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4_t a = r0[q], b = r1[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      i0[4 * q + e] = a[e];
      i1[4 * q + e] = b[e];
    }
  }
  w.sc = mfma_rows<DH>(cx.ring.p[SLOT] + C::kQ, cx.ro, w.kb_f, i0);
  w.dp = mfma_rows<DH>(cx.ring.p[SLOT] + C::kDo, cx.ro, w.vb_f, i1);
}

// dV^T += dO^T P and dK^T += Q^T dS of the step whose transposed fragments
// sit in w.qt_f / w.dt_f.
template <int DH>
__device__ __forceinline__ void kv_grads(const u32x4_t (&pk)[2], const u32x4_t (&dsk)[2], KvState<DH>& w) {
#pragma unroll
  for (int h = 0; h < DH; ++h) {
    mfma_tr(w.dt_f[h], pk, w.acc_v[h]);
    mfma_tr(w.qt_f[h], dsk, w.acc_k[h]);
  }
}

// Transposed Q and dO fragments of the step in `slot`, for the next phase.
template <int DH>
__device__ __forceinline__ void kv_read_tr(const uint8_t* slot, const ReadOffsets& ro, KvState<DH>& w) {
  using C = KvCfg<DH>;
#pragma unroll
  for (int h = 0; h < DH; ++h) {
    read_tr_shared(slot + C::kQ + h * kTileBytes, ro, w.qt_f[h]);
    read_tr_shared(slot + C::kDo + h * kTileBytes, ro, w.dt_f[h]);
  }
}

// Scheduling hints: 8*DH MFMAs, each followed by 8/DH VALU instructions of
// the independent softmax work.
template <int DH>
__device__ __forceinline__ void kv_interleave() {
#pragma unroll
  for (int i = 0; i < 8 * DH; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 8 / DH, 0);  // VALU
  }
}

template <int DH, int SLOT, int P>
__device__ __forceinline__ void kv_phase(const KvCtx& cx, KvState<DH>& w, KvCursor& u, int s) {
  using C = KvCfg<DH>;
  constexpr int AHEAD = (SLOT + 4) % kKvBuf;
  constexpr int PREV = (SLOT + kKvBuf - 1) % kKvBuf;
  constexpr int NEXT = (SLOT + 1) % kKvBuf;
  // step s+1 has landed (steps s+2, s+3 may still be in flight); every wave
  // is done with step s-2, whose slot receives step s+4
  barrier_vm<2 * C::kDma>();
  kv_issue<DH, AHEAD>(cx, u);  // step s + 4
  const int lane = threadIdx.x & 63, lg = lane >> 5, l32 = lane & 31;
  // Masks of S(s). Steps before the wave's first (causal: query tiles that
  // see none of its keys) run the same code fully masked (P = dS = 0), so
  // every wave keeps one pipeline from step 0; on the causal diagonal step,
  // query rows before the key (entry e <-> query lg*16 + e).
  if (s < cx.first) {
#pragma unroll
    for (int e = 0; e < 16; ++e) w.sc[e] = cx.masked;
  } else if (cx.causal && (unsigned)(s - cx.diag0) < (unsigned)cx.g) {  // query tile kb
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (lg * 16 + e < l32) w.sc[e] = cx.masked;
  }
  kv_grads<DH>(w.pk[P ^ 1], w.dsk[P ^ 1], w);   // step s-1
  kv_read_tr<DH>(cx.ring.p[SLOT], cx.ro, w);     // step s, for the next phase

  f32x16_t p, ds;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    p[e] = __builtin_amdgcn_exp2f(w.sc[e] * cx.c);
    ds[e] = p[e] * w.dp[e];
  }
  pack_pairs(p, w.pk[P]);
  pack_pairs(ds, w.dsk[P]);
  kv_interleave<DH>();
  kv_scores<DH, NEXT>(cx, w);  // S(s+1), dP(s+1)
}

// dK/dV of the last step (its transposed fragments were read in its phase).
template <int DH>
__device__ __forceinline__ void kv_drain(KvState<DH>& w, int par) {
  if (par) kv_grads<DH>(w.pk[1], w.dsk[1], w);
  else kv_grads<DH>(w.pk[0], w.dsk[0], w);
}

template <int DH>
__global__ __launch_bounds__(kThreads, Dims<DH>::MINB) void bwd_dkdv_kernel(KvArgs a) {
  using C = KvCfg<DH>;
  constexpr int D = Dims<DH>::D;
  __shared__ __attribute__((aligned(16))) uint8_t ring0[C::kSlot];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[C::kSlot];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[C::kSlot];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[C::kSlot];
  __shared__ __attribute__((aligned(16))) uint8_t ring4[C::kSlot];
  __shared__ __attribute__((aligned(16))) uint8_t ring5[C::kSlot];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lg = lane >> 5, l32 = lane & 31;
  int split, wid, bkv, w_in;
  split_decode(a.nsplit, split, wid);
  if (wid >= a.nwg) return;
  if (!wg_coords(wid, a.pair_major, a.spread, a.spread_block, a.causal, false, a.nwg, a.wg_per_bkv, a.n_bkv, bkv,
                 w_in))
    return;
  const int b = bkv / a.Hkv, kvh = bkv % a.Hkv;
  const SeqGeom sg = seq_geom(a.cu, a.T, a.N, b, a.Hq, a.Hkv);
  const int N = sg.n;
  const int KB = (N + kTileRows - 1) / kTileRows;  // key (and query) tiles of this sequence
  if (w_in * kWaves >= KB) return;  // no keys for this workgroup (whole workgroup)
  // query-range split (encoder-style): this workgroup streams query tiles
  // [qa, qb) and leaves a partial dK/dV; one range (qa = 0, qb = KB) otherwise
  const int qchunk = split_chunk(KB, a.nsplit);
  const bool split_rows = KB > qchunk;
  const int qa = split * qchunk;
  if (qa >= KB) return;
  const int qb = min(KB, qa + qchunk);

  KvCtx cx;
  cx.ring.p[0] = ring0;
  cx.ring.p[1] = ring1;
  cx.ring.p[2] = ring2;
  cx.ring.p[3] = ring3;
  cx.ring.p[4] = ring4;
  cx.ring.p[5] = ring5;
  cx.q = a.q + (size_t)sg.q_base * D;
  cx.dout = a.dout + (size_t)sg.q_base * D;
  cx.rt = a.rt + (a.cu != nullptr ? (size_t)sg.q_base : (size_t)b * a.Hq * a.Np);
  cx.rt_plane_bytes = (uint32_t)(a.rt_plane * 4);
  cx.stride = sg.stride;
  cx.rt_stride = a.Np;
  cx.N = N;
  const HeadGroup hg = head_group(kvh, a.Hq, a.Hkv);
  cx.g = hg.count;
  cx.h0 = hg.first;
  cx.qt0 = a.causal ? w_in * kWaves : qa;  // the first query tile any key of this workgroup sees
  cx.kb = w_in * kWaves + wave;
  cx.causal = a.causal;
  cx.wave = wave;
  cx.c = a.c;
  cx.masked = a.c > 0.f ? -INFINITY : INFINITY;
  cx.off = dma_off_shared<Dims<DH>::RB>(wave, lane);
  cx.ro = read_offsets_shared(lane);
  const bool wave_valid = cx.kb < KB;
  const int nsteps = max(qb - cx.qt0, 0) * cx.g;
  // causal: this wave's keys are first seen by query tile kb, i.e. step (kb - qt0) * g
  cx.first = !wave_valid ? nsteps : (a.causal ? min((cx.kb - cx.qt0) * cx.g, nsteps) : 0);
  cx.diag0 = (cx.kb - cx.qt0) * cx.g;
  cx.d_head = cx.stride * D;
  cx.d_wrap = (int64_t)kTileRows * D - (int64_t)(cx.g - 1) * cx.stride * D;
  cx.rt_wrap = (int64_t)kTileRows - (int64_t)(cx.g - 1) * cx.rt_stride;
  const size_t kv_row0 = (size_t)(sg.kv_base + (int64_t)kvh * sg.stride);

  KvState<DH> w;
  {
    const int u = min(cx.kb * kTileRows + l32, N - 1);
#pragma unroll
    for (int h = 0; h < DH; ++h) {
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        w.kb_f[h][ds] = u32x4_t{0u, 0u, 0u, 0u};
        w.vb_f[h][ds] = u32x4_t{0u, 0u, 0u, 0u};
      }
      if (wave_valid) {
        load_row_frags(a.k + (kv_row0 + u) * D + h * kD, lg, w.kb_f[h]);
        load_row_frags(a.v + (kv_row0 + u) * D + h * kD, lg, w.vb_f[h]);
      }
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        w.acc_k[h][x] = zero16();
        w.acc_v[h][x] = zero16();
      }
    }
    // P and dS of the step before a wave's first are 0 (and its transposed
    // fragments finite zeros): its first dK/dV products add nothing
#pragma unroll
    for (int h = 0; h < DH; ++h)
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          w.qt_f[h][x][hh] = u32x4_t{0u, 0u, 0u, 0u};
          w.dt_f[h][x][hh] = u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        w.pk[par][x] = u32x4_t{0u, 0u, 0u, 0u};
        w.dsk[par][x] = u32x4_t{0u, 0u, 0u, 0u};
      }
  }

  // zero the ring once so that no LDS byte is ever uninitialised
  for (int e = tid; e < C::kSlot / 16; e += kThreads) {
    reinterpret_cast<u32x4_t*>(ring0)[e] = u32x4_t{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4_t*>(ring1)[e] = u32x4_t{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4_t*>(ring2)[e] = u32x4_t{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4_t*>(ring3)[e] = u32x4_t{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4_t*>(ring4)[e] = u32x4_t{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4_t*>(ring5)[e] = u32x4_t{0u, 0u, 0u, 0u};
  }
  barrier_vm<0>();

  // prologue: steps 0..3 in flight (empty ranges past the end), wait for
  // steps 0..2, then S(0) and dP(0)
  KvCursor cur;
  cur.i = 0;
  cur.row0 = cx.qt0 * kTileRows;
  cur.off = (int64_t)cx.h0 * cx.stride * D + (int64_t)cur.row0 * D;
  cur.rt_off = (int64_t)cx.h0 * cx.rt_stride + cur.row0;
  kv_issue<DH, 0>(cx, cur);
  kv_issue<DH, 1>(cx, cur);
  kv_issue<DH, 2>(cx, cur);
  kv_issue<DH, 3>(cx, cur);
  barrier_vm<C::kDma>();
  kv_scores<DH, 0>(cx, w);

  // whole six-phase rounds first (ring slot period 6, register parity 2)
  int s = 0;
  for (; s + kKvBuf <= nsteps; s += kKvBuf) {
    kv_phase<DH, 0, 0>(cx, w, cur, s);
    kv_phase<DH, 1, 1>(cx, w, cur, s + 1);
    kv_phase<DH, 2, 0>(cx, w, cur, s + 2);
    kv_phase<DH, 3, 1>(cx, w, cur, s + 3);
    kv_phase<DH, 4, 0>(cx, w, cur, s + 4);
    kv_phase<DH, 5, 1>(cx, w, cur, s + 5);
  }
  if (s < nsteps) kv_phase<DH, 0, 0>(cx, w, cur, s);
  if (s + 1 < nsteps) kv_phase<DH, 1, 1>(cx, w, cur, s + 1);
  if (s + 2 < nsteps) kv_phase<DH, 2, 0>(cx, w, cur, s + 2);
  if (s + 3 < nsteps) kv_phase<DH, 3, 1>(cx, w, cur, s + 3);
  if (s + 4 < nsteps) kv_phase<DH, 4, 0>(cx, w, cur, s + 4);
  // drain the DMAs still in flight before the wave ends
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

  const int u = cx.kb * kTileRows + l32;
  if (cx.first >= nsteps) return;  // no step for this wave (no barrier follows)
  // dK/dV of the last step (its slot is still intact: later DMAs went elsewhere)
  const int last = nsteps - 1;
  kv_drain<DH>(w, last & 1);
  if (u >= N) return;
  if (split_rows) {
    const size_t prow = ((size_t)split * a.kv_rows + kv_row0 + u) * D;
#pragma unroll
    for (int h = 0; h < DH; ++h) {
      store_tr_row_f32(a.part_k + prow + h * kD, w.acc_k[h], a.scale, lg);
      store_tr_row_f32(a.part_v + prow + h * kD, w.acc_v[h], 1.0f, lg);
    }
    return;
  }
#pragma unroll
  for (int h = 0; h < DH; ++h) {
    store_tr_row(a.dk + (kv_row0 + u) * D + h * kD, w.acc_k[h], a.scale, lg);
    store_tr_row(a.dv + (kv_row0 + u) * D + h * kD, w.acc_v[h], 1.0f, lg);
  }
}

// ------------------------------------------------------------------ dQ
// Software-pipelined over 32-key tiles j (one stage, as the forward):
//   phase j: MFMA  dQ^T += K(j-1)^T dS(j-1)^T  and  S^T(j+1), dP^T(j+1) - D
//            VALU  P(j) = 2^(s c - lse2), dS(j) = P (dP - D)
// (the dP^T accumulator starts from -D, the row's D in every entry, which
// saves the subtraction per score)
// The fragments the next phase multiplies (K and V rows of tile j+2, the
// transposed K of tile j) are read from LDS during this phase.
constexpr int kDqBuf = 5;  // ring slots

template <int DH>
struct DqCfg {
  static constexpr int kK = 0;                       // K half-tiles, row layout
  static constexpr int kV = DH * kTileBytes;         // V half-tiles, row layout
  static constexpr int kKt = 2 * DH * kTileBytes;    // K half-tiles, transposed layout
  static constexpr int kSlot = 3 * DH * kTileBytes;
  static constexpr int kDma = 3 * DH;                // DMA instructions per wave per tile
};

struct DqArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* rt;   // row terms, plane 0 [B*H_q, Np] (-lse log2(e)/c), plane 1 rt_plane floats later (-D)
  int64_t rt_plane;
  uint16_t* dq;
  const int* cu;  // packed sequence offsets (nullptr: dense)
  int64_t T;      // packed: total tokens
  int N, Np, Hq, Hkv, wg_per_bkv, n_bkv, nwg;  // sized for the longest sequence and the largest group
  int spread;  // uneven head groups or packed sequences: spread_coords order
  int spread_block;  // its rotation block
  int pair_major;   // packed encoder-style: pair_major_coords order
  float c, scale;
  int causal;
  int nsplit;       // key-range splits (encoder-style only; 1: none)
  float* part_q;    // nsplit > 1: [nsplit][q rows][D] fp32 partial dQ (scaled)
  int64_t q_rows;   // B*Hq*N (packed: Hq*T)
};

struct DqRing {
  uint8_t* p[kDqBuf];
};

struct DqCtx {
  DqRing ring;
  const uint16_t* kbase;
  const uint16_t* vbase;
  int N, nlim, last, tb, causal, wave, t;
  float c;
  float masked;  // score whose exponent s*c is -inf: -inf * sign(c)
  uint32_t off_rows, off_tr;
  ReadOffsets ro;
};

template <int DH>
struct DqState {
  u32x4_t qf[DH][4], df[DH][4];  // Q and dO of this wave's 32 rows as B operands
  f32x16_t acc[DH][2];           // dQ^T
  u32x4_t kr[DH][4], vr[DH][4];  // K and V row fragments of the next S^T, dP^T
  u32x4_t kt[DH][2][2];          // transposed K fragments of the next dQ product
  f32x16_t sc[2], dp[2];         // S^T and dP^T of tiles j (index j & 1) and j+1
  u32x4_t dsk[2][2];             // dS of tiles j-1 and j, packed as B operands
  float lse2, dd;
  f32x16_t ndd;                  // -D in every entry: dP^T starts from it, so dS = P dP^T
};

template <int DH, int SLOT>
__device__ __forceinline__ void dq_issue(const DqCtx& cx, int kt) {
  using C = DqCfg<DH>;
  constexpr int RB = Dims<DH>::RB;
  const int row0 = kt * kTileRows;
  uint8_t* slot = cx.ring.p[SLOT];
#pragma unroll
  for (int h = 0; h < DH; ++h) {
    const uint32_t hb = h * kRowBytes;
    dma_tile_part<RB>(cx.kbase, row0, cx.nlim, slot + C::kK + h * kTileBytes + cx.wave * 1024, cx.off_rows + hb);
    dma_tile_part<RB>(cx.vbase, row0, cx.nlim, slot + C::kV + h * kTileBytes + cx.wave * 1024, cx.off_rows + hb);
    dma_tile_part<RB>(cx.kbase, row0, cx.nlim, slot + C::kKt + h * kTileBytes + cx.wave * 1024, cx.off_tr + hb);
  }
}

template <int DH>
__device__ __forceinline__ void dq_read_rows(const uint8_t* slot, const ReadOffsets& ro, DqState<DH>& w) {
  using C = DqCfg<DH>;
#pragma unroll
  for (int h = 0; h < DH; ++h) {
    read_rows(slot + C::kK + h * kTileBytes, ro, w.kr[h]);
    read_rows(slot + C::kV + h * kTileBytes, ro, w.vr[h]);
  }
}

template <int DH>
__device__ __forceinline__ f32x16_t mfma_regs(const u32x4_t (&a)[DH][4], const u32x4_t (&b)[DH][4],
                                             const f32x16_t& init) {
  f32x16_t acc = init;
#pragma unroll
  for (int h = 0; h < DH; ++h)
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) acc = mfma(a[h][ds], b[h][ds], acc);
  return acc;
}

// Scheduling hints: 12*DH MFMAs, each followed by 5/DH (at least 2) VALU
// instructions of the independent softmax work.
template <int DH>
__device__ __forceinline__ void dq_interleave() {
#pragma unroll
  for (int i = 0; i < 12 * DH; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, DH == 1 ? 5 : 2, 0);  // VALU
  }
}

template <int DH, int SLOT, int P>
__device__ __forceinline__ void dq_phase(const DqCtx& cx, DqState<DH>& w, int j) {
  using C = DqCfg<DH>;
  constexpr int AHEAD = (SLOT + 4) % kDqBuf;
  constexpr int NEXT2 = (SLOT + 2) % kDqBuf;
  // tile j+2 has landed (tile j+3 may still be in flight); every wave is done
  // with tile j-1, whose slot receives tile j+4
  barrier_vm<C::kDma>();
  dq_issue<DH, AHEAD>(cx, j + 4);
  if (j > cx.last) return;
  const int lg = (threadIdx.x & 63) >> 5;
  // mask S^T(j) on diagonal and tail tiles only, before the phase's MFMAs so
  // that the MFMA/softmax block below stays one basic block
  if ((cx.causal && j == cx.tb) || (j * kTileRows + kTileRows > cx.N)) {
    const int key0 = j * kTileRows + lg * 16;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (!(key0 + e < cx.N && (!cx.causal || key0 + e <= cx.t))) w.sc[P][e] = cx.masked;
  }

#pragma unroll
  for (int h = 0; h < DH; ++h) mfma_tr(w.kt[h], w.dsk[P ^ 1], w.acc[h]);  // dQ^T += K(j-1)^T dS(j-1)^T
#pragma unroll
  for (int h = 0; h < DH; ++h) read_tr(cx.ring.p[SLOT] + C::kKt + h * kTileBytes, cx.ro, w.kt[h]);  // K(j)^T
  w.sc[P ^ 1] = mfma_regs<DH>(w.kr, w.qf, zero16());  // S^T(j+1)
  w.dp[P ^ 1] = mfma_regs<DH>(w.vr, w.df, w.ndd);  // dP^T(j+1) - D
  dq_read_rows<DH>(cx.ring.p[NEXT2], cx.ro, w);  // K(j+2), V(j+2)

  f32x16_t ds;
#pragma unroll
  for (int e = 0; e < 16; ++e)
    ds[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(w.sc[P][e], cx.c, -w.lse2)) * w.dp[P][e];
  pack_pairs(ds, w.dsk[P]);
  dq_interleave<DH>();
}

template <int DH>
__global__ __launch_bounds__(kThreads, Dims<DH>::MINB) void bwd_dq_kernel(DqArgs a) {
  using C = DqCfg<DH>;
  constexpr int D = Dims<DH>::D;
  __shared__ __attribute__((aligned(16))) uint8_t ring0[C::kSlot];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[C::kSlot];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[C::kSlot];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[C::kSlot];
  __shared__ __attribute__((aligned(16))) uint8_t ring4[C::kSlot];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lg = lane >> 5, l32 = lane & 31;
  int split, wid, bkv, w_in;
  split_decode(a.nsplit, split, wid);
  if (wid >= a.nwg) return;
  if (!wg_coords(wid, a.pair_major, a.spread, a.spread_block, a.causal, true, a.nwg, a.wg_per_bkv, a.n_bkv, bkv,
                 w_in))
    return;
  const int b = bkv / a.Hkv, kvh = bkv % a.Hkv;
  const int slot = w_in * kWaves + wave;
  const HeadGroup hg = head_group(kvh, a.Hq, a.Hkv);
  const SeqGeom sg = seq_geom(a.cu, a.T, a.N, b, a.Hq, a.Hkv);
  const int N = sg.n, g = hg.count;
  const int TB = (N + kTileRows - 1) / kTileRows;  // 32-row query (and key) tiles of this sequence
  if (w_in * kWaves >= TB * g) return;  // past this group's rows (whole workgroup)
  const int tb = slot / g, jh = slot % g;
  const bool wave_valid = tb < TB;
  const int h = hg.first + jh;
  // key tiles the workgroup streams, and the last one this wave uses
  const int maxtb = min((w_in * kWaves + kWaves - 1) / g, TB - 1);
  const int nt_all = a.causal ? maxtb + 1 : TB;
  // key-range split (encoder-style): key tiles [ka, ka + nt) with K/V
  // pointers, N and the tile index counted from ka; one range otherwise
  const int kchunk = split_chunk(TB, a.nsplit);
  const bool split_rows = TB > kchunk;
  const int ka = split * kchunk;
  if (ka >= nt_all) return;
  const int nt = min(nt_all - ka, kchunk);
  const int key_shift = ka * kTileRows;

  DqCtx cx;
  cx.ring.p[0] = ring0;
  cx.ring.p[1] = ring1;
  cx.ring.p[2] = ring2;
  cx.ring.p[3] = ring3;
  cx.ring.p[4] = ring4;
  const int64_t kvrow0 = sg.kv_base + (int64_t)kvh * sg.stride;
  const int64_t qrow0 = sg.q_base + (int64_t)h * sg.stride;
  const int64_t rtrow0 = a.cu != nullptr ? sg.q_base + (int64_t)h * a.Np : ((int64_t)b * a.Hq + h) * a.Np;
  cx.kbase = a.k + (size_t)(kvrow0 + key_shift) * D;
  cx.vbase = a.v + (size_t)(kvrow0 + key_shift) * D;
  cx.N = N - key_shift;
  cx.nlim = min(cx.N, nt * kTileRows);
  cx.last = !wave_valid ? -1 : (a.causal ? tb : nt - 1);
  cx.tb = tb;
  cx.causal = a.causal;
  cx.wave = wave;
  cx.t = tb * kTileRows + l32;
  cx.c = a.c;
  cx.masked = a.c > 0.f ? -INFINITY : INFINITY;
  cx.off_rows = dma_off_rows<Dims<DH>::RB>(wave, lane);
  cx.off_tr = dma_off_tr<Dims<DH>::RB>(wave, lane);
  cx.ro = read_offsets(lane);

  const size_t row_q = (size_t)qrow0 + min(cx.t, N - 1);
  DqState<DH> w;
#pragma unroll
  for (int hh = 0; hh < DH; ++hh) {
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      w.qf[hh][ds] = u32x4_t{0u, 0u, 0u, 0u};
      w.df[hh][ds] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  w.lse2 = 0.f;
  w.dd = 0.f;
  if (wave_valid) {
#pragma unroll
    for (int hh = 0; hh < DH; ++hh) {
      load_row_frags(a.q + row_q * D + hh * kD, lg, w.qf[hh]);
      load_row_frags(a.dout + row_q * D + hh * kD, lg, w.df[hh]);
    }
    const size_t rr = (size_t)rtrow0 + min(cx.t, N - 1);
    w.lse2 = -a.rt[rr] * a.c;  // lse log2(e)
    w.dd = -a.rt[a.rt_plane + rr];
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) w.ndd[e] = -w.dd;
#pragma unroll
  for (int hh = 0; hh < DH; ++hh) {
    w.acc[hh][0] = zero16();
    w.acc[hh][1] = zero16();
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      w.kt[hh][x][0] = u32x4_t{0u, 0u, 0u, 0u};  // K(-1) = 0 and dS(-1) = 0: the first dQ product is a no-op
      w.kt[hh][x][1] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  w.dsk[1][0] = u32x4_t{0u, 0u, 0u, 0u};
  w.dsk[1][1] = u32x4_t{0u, 0u, 0u, 0u};

  for (int e = tid; e < C::kSlot / 16; e += kThreads) {
    reinterpret_cast<u32x4_t*>(ring0)[e] = u32x4_t{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4_t*>(ring1)[e] = u32x4_t{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4_t*>(ring2)[e] = u32x4_t{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4_t*>(ring3)[e] = u32x4_t{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4_t*>(ring4)[e] = u32x4_t{0u, 0u, 0u, 0u};
  }
  barrier_vm<0>();

  // prologue: tiles 0..3 in flight, wait for tiles 0..2, S^T(0) and dP^T(0),
  // then the row fragments of tile 1
  dq_issue<DH, 0>(cx, 0);
  dq_issue<DH, 1>(cx, 1);
  dq_issue<DH, 2>(cx, 2);
  dq_issue<DH, 3>(cx, 3);
  barrier_vm<C::kDma>();
  dq_read_rows<DH>(ring0, cx.ro, w);
  w.sc[0] = mfma_regs<DH>(w.kr, w.qf, zero16());
  w.dp[0] = mfma_regs<DH>(w.vr, w.df, w.ndd);
  dq_read_rows<DH>(ring1, cx.ro, w);

  // whole ten-phase rounds first (ring slot period 5, register parity 2)
  int j = 0;
  for (; j + 2 * kDqBuf <= nt; j += 2 * kDqBuf) {
    dq_phase<DH, 0, 0>(cx, w, j);
    dq_phase<DH, 1, 1>(cx, w, j + 1);
    dq_phase<DH, 2, 0>(cx, w, j + 2);
    dq_phase<DH, 3, 1>(cx, w, j + 3);
    dq_phase<DH, 4, 0>(cx, w, j + 4);
    dq_phase<DH, 0, 1>(cx, w, j + 5);
    dq_phase<DH, 1, 0>(cx, w, j + 6);
    dq_phase<DH, 2, 1>(cx, w, j + 7);
    dq_phase<DH, 3, 0>(cx, w, j + 8);
    dq_phase<DH, 4, 1>(cx, w, j + 9);
  }
  if (j < nt) dq_phase<DH, 0, 0>(cx, w, j);
  if (j + 1 < nt) dq_phase<DH, 1, 1>(cx, w, j + 1);
  if (j + 2 < nt) dq_phase<DH, 2, 0>(cx, w, j + 2);
  if (j + 3 < nt) dq_phase<DH, 3, 1>(cx, w, j + 3);
  if (j + 4 < nt) dq_phase<DH, 4, 0>(cx, w, j + 4);
  if (j + 5 < nt) dq_phase<DH, 0, 1>(cx, w, j + 5);
  if (j + 6 < nt) dq_phase<DH, 1, 0>(cx, w, j + 6);
  if (j + 7 < nt) dq_phase<DH, 2, 1>(cx, w, j + 7);
  if (j + 8 < nt) dq_phase<DH, 3, 0>(cx, w, j + 8);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

  if (!wave_valid || cx.t >= N) return;
  // drain dQ^T += K(last)^T dS(last)^T
#pragma unroll
  for (int hh = 0; hh < DH; ++hh) {
    if (cx.last & 1) mfma_tr(w.kt[hh], w.dsk[1], w.acc[hh]);
    else mfma_tr(w.kt[hh], w.dsk[0], w.acc[hh]);
    if (split_rows)
      store_tr_row_f32(a.part_q + ((size_t)split * a.q_rows + qrow0 + cx.t) * D + hh * kD, w.acc[hh], a.scale, lg);
    else
      store_tr_row(a.dq + ((size_t)qrow0 + cx.t) * D + hh * kD, w.acc[hh], a.scale, lg);
  }
}

// out = sum of the range partials of each row (fp32, already scaled) as
// bf16, one thread per 4 values. A row's ranges are those holding a 32-row
// tile of its sequence; rows of sequences that were not split were written
// by the gradient kernels. Rows are [B, H, N] (dense) or [H, T] (packed).
struct SumArgs {
  const float* part;
  uint16_t* out;
  const int* cu;
  int64_t T, rows;
  int N, B, D, nsplit;
};

__global__ __launch_bounds__(256) void bwd_split_sum_kernel(SumArgs a) {
  const int per_row = a.D / 4;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= a.rows * per_row) return;
  const int64_t r = e / per_row;
  const int c4 = (int)(e % per_row);
  int t, n;
  if (a.cu == nullptr) {
    t = (int)(r % a.N);
    n = a.N;
  } else {
    const int64_t p = r % a.T;  // token; its sequence is the last b with start(b) <= p
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
  const int NT = (n + kTileRows - 1) / kTileRows;
  const int chunk = split_chunk(NT, a.nsplit);
  if (NT <= chunk) return;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.nsplit && s * chunk < NT; ++s)
    acc += *reinterpret_cast<const f32x4_t*>(a.part + ((size_t)s * a.rows + r) * a.D + 4 * c4);
  u32x2_t o;
  o[0] = pack_bf16x2(acc[0], acc[1]);
  o[1] = pack_bf16x2(acc[2], acc[3]);
  *reinterpret_cast<u32x2_t*>(a.out + (size_t)r * a.D + 4 * c4) = o;
}

hipError_t launch_split_sum(const float* part, void* out, const BwdProblem& p, int64_t rows, hipStream_t stream) {
  if (p.B > 0x7fffffff) return hipErrorInvalidValue;
  SumArgs a;
  a.part = part;
  a.out = static_cast<uint16_t*>(out);
  a.cu = p.cu_seqlens;
  a.T = p.T;
  a.rows = rows;
  a.N = (int)p.N;
  a.B = (int)p.B;
  a.D = (int)p.D;
  a.nsplit = p.nsplit;
  const int64_t blocks = (rows * (p.D / 4) + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (p.dry_run) return hipSuccess;
  hipLaunchKernelGGL(bwd_split_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int DH>
hipError_t launch_bwd(const BwdProblem& p, hipStream_t stream) {
  constexpr int RB = Dims<DH>::RB;
  if (p.N * RB > 0x7fffffffLL) return hipErrorInvalidValue;  // buffer descriptor range
  const bool packed = p.cu_seqlens != nullptr;
  const int N = (int)p.N;  // the (longest) sequence
  // row-term rows per head: dense, N padded to whole tiles; packed, T + 32
  const int64_t Np64 = packed ? p.T + kTileRows : (p.N + kTileRows - 1) / kTileRows * kTileRows;
  if (Np64 > 0x7fffffff) return hipErrorInvalidValue;
  const int Np = (int)Np64;
  // c = scale * log2(e), kept away from 0 so that a masked score (+-inf)
  // times c is -inf; at scale 0 the scores s*c stay below 1e-22 in
  // magnitude and round away exactly as 0 would
  float c = p.scale * kLog2e;
  if (fabsf(c) < 1e-30f) c = p.scale < 0.f ? -1e-30f : 1e-30f;
  float* rt = static_cast<float*>(p.rowterms);
  // two planes of row terms, 4 bytes per row each; a row-term DMA spans
  // from a row of plane 0 to 128 bytes into plane 1 (32-bit range)
  const int64_t rt_rows = (packed ? 1 : p.B) * p.Hq * Np64;
  if (rt_rows > (0x7fffffffLL - 256) / 4) return hipErrorInvalidValue;
  const int nsplit = p.nsplit < 1 ? 1 : p.nsplit;
  if (nsplit > 1 && (p.causal || p.split_ws == nullptr)) return hipErrorInvalidValue;
  const int64_t q_rows = packed ? p.Hq * p.T : p.B * p.Hq * p.N;
  const int64_t kv_rows = packed ? p.Hkv * p.T : p.B * p.Hkv * p.N;
  float* part_q = p.split_ws;
  float* part_k = part_q == nullptr ? nullptr : part_q + (size_t)nsplit * q_rows * p.D;
  float* part_v = part_k == nullptr ? nullptr : part_k + (size_t)nsplit * kv_rows * p.D;
  // with splits the grids cover whole runs of 8 (see split_decode)
  auto grid_of = [&](int64_t nwg) { return nsplit == 1 ? nwg : (nwg + 7) / 8 * 8 * nsplit; };
  const int spread = (packed || p.Hq % p.Hkv != 0) ? 1 : 0;
  const int pair_major = (packed && !p.causal) ? 1 : 0;  // as the d = 64 forward
  if (p.B * p.Hkv > 0x7fffffff || p.B * p.Hq > 0x7fffffff) return hipErrorInvalidValue;
  const int n_bkv = (int)(p.B * p.Hkv);
  const int block = spread_block(packed, n_bkv);

  {
    // a packed batch is, for the row terms, one sequence of T tokens
    RowArgs a;
    a.o = static_cast<const uint16_t*>(p.o);
    a.dout = static_cast<const uint16_t*>(p.dout);
    a.lse = p.lse;
    a.rt = rt;
    a.nrows = rt_rows;
    a.N = packed ? (int)p.T : N;
    a.Np = Np;
    a.inv_c = 1.0f / c;
    const int64_t nblk = (a.nrows + 31) / 32;
    if (nblk > 0x7fffffff) return hipErrorInvalidValue;
    if (!p.dry_run) {
      hipLaunchKernelGGL(bwd_rowterms_kernel<DH>, dim3((unsigned)nblk), dim3(256), 0, stream, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const int tiles = (N + kTileRows - 1) / kTileRows;  // of the longest sequence
  {
    KvArgs a;
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.dout = static_cast<const uint16_t*>(p.dout);
    a.rt = rt;
    a.rt_plane = rt_rows;
    a.dk = static_cast<uint16_t*>(p.dk);
    a.dv = static_cast<uint16_t*>(p.dv);
    a.cu = p.cu_seqlens;
    a.T = p.T;
    a.N = N;
    a.Np = Np;
    a.Hq = (int)p.Hq;
    a.Hkv = (int)p.Hkv;
    a.spread = spread;
    a.spread_block = block;
    a.wg_per_bkv = (tiles + kWaves - 1) / kWaves;
    a.n_bkv = n_bkv;
    a.pair_major = pair_major;
    const int64_t nwg = pair_major ? pair_major_nwg(a.n_bkv, a.wg_per_bkv) : (int64_t)a.wg_per_bkv * a.n_bkv;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    a.nwg = (int)nwg;
    a.c = c;
    a.scale = p.scale;
    a.causal = p.causal;
    a.nsplit = nsplit;
    a.part_k = part_k;
    a.part_v = part_v;
    a.kv_rows = kv_rows;
    const int64_t grid = grid_of(a.nwg);
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (!p.dry_run) {
      hipLaunchKernelGGL(bwd_dkdv_kernel<DH>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  {
    DqArgs a;
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.dout = static_cast<const uint16_t*>(p.dout);
    a.rt = rt;
    a.rt_plane = rt_rows;
    a.dq = static_cast<uint16_t*>(p.dq);
    a.cu = p.cu_seqlens;
    a.T = p.T;
    a.N = N;
    a.Np = Np;
    a.Hq = (int)p.Hq;
    a.Hkv = (int)p.Hkv;
    a.spread = spread;
    a.spread_block = block;
    const int64_t slots = (int64_t)tiles * max_group(a.Hq, a.Hkv);
    if ((slots + kWaves - 1) / kWaves > 0x7fffffff || (int64_t)tiles * p.Hq > 0x7fffffff) return hipErrorInvalidValue;
    a.wg_per_bkv = (int)((slots + kWaves - 1) / kWaves);
    a.n_bkv = n_bkv;
    a.pair_major = pair_major;
    const int64_t nwg = pair_major ? pair_major_nwg(a.n_bkv, a.wg_per_bkv) : (int64_t)a.wg_per_bkv * a.n_bkv;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    a.nwg = (int)nwg;
    a.c = c;
    a.scale = p.scale;
    a.causal = p.causal;
    a.nsplit = nsplit;
    a.part_q = part_q;
    a.q_rows = q_rows;
    const int64_t grid = grid_of(a.nwg);
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (!p.dry_run) {
      hipLaunchKernelGGL(bwd_dq_kernel<DH>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (nsplit == 1) return hipSuccess;
  }
  hipError_t e = launch_split_sum(part_k, p.dk, p, kv_rows, stream);
  if (e == hipSuccess) e = launch_split_sum(part_v, p.dv, p, kv_rows, stream);
  if (e == hipSuccess) e = launch_split_sum(part_q, p.dq, p, q_rows, stream);
  return e;
}

}  // namespace

size_t attn_bwd_split_bytes(int64_t q_rows, int64_t kv_rows, int64_t D, int nsplit) {
  if (nsplit <= 1 || q_rows <= 0 || kv_rows <= 0) return 0;
  return (size_t)nsplit * (size_t)(q_rows + 2 * kv_rows) * (size_t)D * sizeof(float);
}

// Recommended range splits for the backward (encoder-style only), by the
// round model of the d = 64 forward applied to both gradient kernels: the
// dK/dV kernel's workgroups hold 128 keys of one K/V head, the dQ kernel's
// four 32-row query slots; Dims<DH>::MINB workgroups fit per CU. Two splits
// when they cut the rounds of the busier kernel by at least 10 %, or fill a
// launch that is under half a round. Packed batches (T > 0 tokens, N the
// longest sequence, pair-major order) as the forward's: two splits when
// packed_wants_split and the longest sequence's own dK/dV workgroups fill
// between one and two rounds (measured at 32k, longest sequence 18496
// tokens, d = 64, counted TFLOP/s, unsplit -> 2 ranges: (8,4) 629 -> 688 at
// 1.13 rounds, (16,16) 738 -> 699 at 4.5). Causal launches are not split.
int attn_bwd_auto_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t T, int64_t D, bool causal,
                         int cus) {
  if (causal || (D != 64 && D != 128) || B <= 0 || N <= 0) return 1;
  const int64_t tiles = (N + kTileRows - 1) / kTileRows;
  if (T > 0) {
    const int minb1 = D == 64 ? Dims<1>::MINB : Dims<2>::MINB;
    const double r1 = (double)(Hkv * ((tiles + kWaves - 1) / kWaves)) / ((double)(cus > 0 ? cus : 256) * minb1);
    return (tiles >= 2 * kMinSplitTiles && packed_wants_split(N, T) && r1 > 1.0 && r1 < 2.0 &&
            ceil(2.0 * r1) / 2.0 <= 0.9 * ceil(r1))
               ? 2
               : 1;
  }
  if (tiles < 2 * kMinSplitTiles) return 1;
  const int minb = D == 64 ? Dims<1>::MINB : Dims<2>::MINB;
  const double slots = (double)(cus > 0 ? cus : 256) * minb;
  int64_t wq = 0;
  for (int j = 0; j < Hkv; ++j) wq += group_wgs(j, (int)Hq, (int)Hkv, (int)tiles, kWaves);
  const double r_kv = (double)(B * Hkv * ((tiles + kWaves - 1) / kWaves)) / slots;
  const double r_q = (double)(B * wq) / slots;
  for (const double r : {r_kv, r_q})
    if (2.0 * r <= 1.0 || ceil(2.0 * r) / 2.0 <= 0.9 * ceil(r)) return 2;
  return 1;
}

size_t attn_bwd_rowterm_bytes(int64_t B, int64_t Hq, int64_t N) {
  const int64_t Np = (N + kTileRows - 1) / kTileRows * kTileRows;
  return (size_t)(B * Hq * Np) * sizeof(float2);
}

// Packed sequences: row terms [H_q, T + 32]; a 32-row tile read from any
// row of any sequence then stays inside the buffer.
size_t attn_bwd_rowterm_bytes_packed(int64_t Hq, int64_t T) { return (size_t)(Hq * (T + kTileRows)) * sizeof(float2); }

hipError_t launch_attn_bwd_bf16(const BwdProblem& p, hipStream_t stream) {
  if (p.D == 64) return launch_bwd<1>(p, stream);
  if (p.D == 128) return launch_bwd<2>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace sqa

// Row-term buffer of the allocation-free backward (sqa_attn_bwd_noalloc):
// one copy per GPU, loaded with the code object and held until the process
// ends. Host code never passes this name to a kernel (on the host it is only
// a stand-in for the device symbol); it passes the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[sqa::kNoAllocScratchBytes];

namespace sqa {

// Device address of `scratch` on the current device, looked up once per
// device and cached (concurrent first calls on one device store the same
// address).
hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    cache[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace sqa
