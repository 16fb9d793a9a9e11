// SQA attention forward, bf16 in/out, fp32 softmax state, for gfx950: the
// kernel for head dims 16 and 32 (64 and 128 have their own pipelined
// kernels).
//
// What is computed: per query head i and position t, softmax attention over
// the keys of K/V head floor(i*H_kv/H_q) (contiguous query-head groups as in
// grouped-query attention, "GQA ..." page, "The idea"), with H_q below the
// baseline head count (SQA paper abstract). Encoder-style (all keys) or
// causal (keys u <= t).
//
// Work decomposition (MI355X-first design, not taken from the pages):
//   * A workgroup is 4 waves that share one (batch, K/V head). Each wave owns
//     a "slot": 32*QS consecutive query positions (QS = 1 or 2 MFMA row
//     tiles) of one query head of the group. Slots are ordered (position
//     block, head-in-group), so the 4
//     waves of a workgroup read the same K/V head -- for groups of g >= 2
//     heads they are different query heads at the same positions, which is
//     the reuse SQA/GQA grouping offers. Group sizes may differ by one head
//     and packed sequences by length; the grid covers the largest group and
//     the longest sequence, and workgroups with no rows leave at once.
//   * K/V are streamed in 64-key tiles, HBM -> registers -> LDS, double
//     buffered with one barrier per tile; each tile is read from HBM once per
//     workgroup and consumed by 4 x 32*QS query rows. On request
//     (nsplit > 1) each row block's key tiles are cut into ranges computed by
//     separate workgroups, whose fp32 partial softmax states are merged
//     afterwards (split_merge.h).
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = K tile from LDS, B = Q held in
//     registers). The accumulator layout then already is the B operand of
//     O^T = V^T P^T, so probabilities never leave registers. K rows are
//     stored in LDS under the permutation pi (below) so that each lane's 16
//     accumulator entries are 16 consecutive keys; V^T is stored transposed
//     (built in registers with a 4x4 transpose) so the A operand of the P.V
//     product is one 16-byte LDS read.
//   * Online softmax in fp32 with base-2 exponentials (v_exp_f32) of
//     s*c - m, c = |scale|*log2(e). The running maximum m is raised lazily:
//     probabilities are computed against m as it stands, and only when a
//     lane's sum of its 32 probabilities of a tile exceeds kSumLimit (or is
//     not finite) is the tile's exact row maximum taken, O and l rescaled
//     and the tile's probabilities recomputed; at d = 16 a wave's first
//     tile takes its exact maximum at once. Between refreshes every probability is <= kSumLimit, far
//     inside the bf16/fp32 range, and no tile pays for a row maximum.
//   * Probabilities are rounded to bf16 (round to nearest even) for the P.V
//     MFMA; the row sum l adds the same rounded values, so the weights that
//     multiply V sum exactly to l.
//   * Causal: tiles above a wave's diagonal are skipped; only the diagonal
//     tile and a ragged tail tile are masked. Workgroups are issued
//     longest-first. Encoder-style: blockIdx is remapped so consecutive
//     workgroups (same K/V head) land on the same XCD and share its L2.
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

constexpr int kThreads = 256;      // 4 waves of 64
constexpr int kWaves = 4;
constexpr int kMaxRowsPerWave = 64;  // query rows per wave: QS (1 or 2) 32-row MFMA tiles
constexpr int kTileKeys = 64;      // keys per K/V tile
constexpr float kSumLimit = 1048576.0f;  // 2^20
constexpr float kMaskedScore = -3.0e38f;
constexpr float kMinC = 1e-30f;          // |scale|*log2(e) is clamped up to this
constexpr int kXcds = 8;

template <int D>
struct Cfg {
  static_assert(D == 16 || D == 32, "head dim");
  static constexpr int DSTEPS = D / 16;            // MFMA k-steps over d for S^T
  static constexpr int DSUB = (D + 31) / 32;       // 32-row O^T tiles over d
  static constexpr int KROW = D + 8;               // LDS pitch of a K row (bf16)
  static constexpr int VROWS = DSUB * 32;          // rows of V^T in LDS
  static constexpr int VROW = kTileKeys + 8;       // LDS pitch of a V^T row (bf16)
  static constexpr int KBUF = kTileKeys * KROW;    // bf16 elements per K buffer
  static constexpr int VBUF = VROWS * VROW;        // bf16 elements per V^T buffer
  static constexpr int BUF = KBUF + VBUF;
  static constexpr int KCHUNKS = kTileKeys * D / 8;          // 16-byte chunks per K tile
  static constexpr int KLOADS = (KCHUNKS + kThreads - 1) / kThreads;
  static constexpr int VBLOCKS = (kTileKeys / 4) * (D / 4);  // 4x4 blocks per V tile
  static constexpr int VLOADS = (VBLOCKS + kThreads - 1) / kThreads;
};

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int* cu;   // packed sequence offsets (nullptr: dense)
  int64_t T;       // packed: total tokens
  int N, Hq, Hkv;  // N: the (longest) sequence length
  int wg_per_bkv;  // workgroups per (batch, K/V head), for the largest group
  int n_bkv;       // B * Hkv
  int nwg;
  int spread;      // 1: spread_coords order (packed sequences, causal uneven groups)
  int spread_block;   // rotation block of the spread order
  int exact_per_batch;  // > 0: exact_coords order with this many workgroups per batch
  int pair_major;  // packed encoder-style: pair_major_coords order
  int snake;       // dense causal: the CU count; dispatch order reversed in every other round of that many
  float c;         // |scale| * log2(e)
  uint32_t qsign;  // 0x80008000 flips both bf16 halves when scale < 0
  int causal;
  int nsplit;      // key-range splits (1: none)
  float* part;     // nsplit > 1: [nsplit][rows][D] unnormalised O, then [nsplit][rows][2] (m, l)
  int64_t rows;    // query rows: B*Hq*N (packed: Hq*T)
};

// MFMA row r of a 32-key sub-tile holds key pi(r); the accumulator entry i
// of lane-half lg then is key lg*16 + i. pi_inv places a key in LDS.
__device__ __forceinline__ int pi_inv(int p) {
  return ((p & 15) >> 2) * 8 + (p >> 4) * 4 + (p & 3);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  bf16x2_t h = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}


template <int D>
struct TileRegs {
  u32x4_t k[Cfg<D>::KLOADS];
  u32x2_t v[Cfg<D>::VLOADS][4];
};

// HBM -> registers for K/V tile kt (key rows clamped into [0, N)).
template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const uint16_t* kbase,
                                          const uint16_t* vbase, int kt, int N, int tid) {
  using C = Cfg<D>;
  const int key0 = kt * kTileKeys;
#pragma unroll
  for (int it = 0; it < C::KLOADS; ++it) {
    const int c = tid + it * kThreads;
    if (c < C::KCHUNKS) {
      const int key = c / (D / 8), dc = c % (D / 8);
      const int row = min(key0 + key, N - 1);
      r.k[it] = *reinterpret_cast<const u32x4_t*>(kbase + (size_t)row * D + dc * 8);
    }
  }
#pragma unroll
  for (int it = 0; it < C::VLOADS; ++it) {
    const int blk = tid + it * kThreads;
    if (blk < C::VBLOCKS) {
      const int kg = blk / (D / 4), dg = blk % (D / 4);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = min(key0 + kg * 4 + rr, N - 1);
        r.v[it][rr] = *reinterpret_cast<const u32x2_t*>(vbase + (size_t)row * D + dg * 4);
      }
    }
  }
}

// registers -> LDS: K rows under pi_inv, V transposed (4x4 blocks).
template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, uint16_t* buf, int tid) {
  using C = Cfg<D>;
  uint16_t* ks = buf;
  uint16_t* vs = buf + C::KBUF;
#pragma unroll
  for (int it = 0; it < C::KLOADS; ++it) {
    const int c = tid + it * kThreads;
    if (c < C::KCHUNKS) {
      const int key = c / (D / 8), dc = c % (D / 8);
      const int lrow = (key & ~31) + pi_inv(key & 31);
      *reinterpret_cast<u32x4_t*>(ks + lrow * C::KROW + dc * 8) = r.k[it];
    }
  }
#pragma unroll
  for (int it = 0; it < C::VLOADS; ++it) {
    const int blk = tid + it * kThreads;
    if (blk < C::VBLOCKS) {
      const int kg = blk / (D / 4), dg = blk % (D / 4);
      // r.v[it][rr] = {V[key rr][d0], V[rr][d0+1]} , {V[rr][d0+2], V[rr][d0+3]}
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int word = cc >> 1;
        const bool hi = cc & 1;
        uint32_t e[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const uint32_t x = r.v[it][rr][word];  // scalar copy of the vector element
          e[rr] = hi ? (x >> 16) : (x & 0xffffu);
        }
        u32x2_t out;
        out[0] = e[0] | (e[1] << 16);
        out[1] = e[2] | (e[3] << 16);
        const int d = dg * 4 + cc;
        const int lrow = (d & ~31) + pi_inv(d & 31);
        *reinterpret_cast<u32x2_t*>(vs + lrow * C::VROW + kg * 4) = out;
      }
    }
  }
}

// Probabilities of query tile qs (both 32-key halves of a 64-key tile)
// against the maximum m, rounded to bf16 and packed as the B operand of
// O^T += V^T P^T; returns the lane's sum of its 32 rounded probabilities,
// accumulated in two partial sums (two short dependency chains).
template <int QS>
__device__ __forceinline__ float exp_rows(const f32x16_t (&s)[2][QS], int qs, uint32_t (&pk)[2][QS][2][4],
                                          float c, float m) {
  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
  const float mneg = -m;
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int kx = 0; kx < 2; ++kx)
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kx][qs][2 * w], c, mneg));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kx][qs][2 * w + 1], c, mneg));
      const uint32_t pp = pack_bf16x2(p0, p1);
      pk[kx][qs][w >> 2][w & 3] = pp;
      if (w & 1) l1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp), ones, l1, false);
      else l0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp), ones, l0, false);
    }
  return l0 + l1;
}

// S^T = K Q^T of query tile qs against both 32-key halves of the tile.
template <int D, int QS>
__device__ __forceinline__ void tile_scores(const bf16x8_t (&kf)[2][Cfg<D>::DSTEPS],
                                            const u32x4_t (&qf)[QS][Cfg<D>::DSTEPS], int qs,
                                            f32x16_t (&s)[2][QS]) {
#pragma unroll
  for (int kx = 0; kx < 2; ++kx) {
    f32x16_t acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int ds = 0; ds < Cfg<D>::DSTEPS; ++ds)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kx][ds], as_bf16x8(qf[qs][ds]), acc, 0, 0, 0);
    s[kx][qs] = acc;
  }
}

// Invisible keys (causal: key > t; tail: key >= N) get kMaskedScore, whose
// probability underflows to exactly 0 for any c >= kMinC once m is finite;
// every row's first tile (tile 0) holds a visible key (key 0), so m is finite
// after it. Only a wave's diagonal tile and the ragged last tile need this.
template <int QS>
__device__ __forceinline__ void mask_tile(f32x16_t (&s)[2][QS], int qs, int key0, int N, int causal, int trow0,
                                          int l32, int lg) {
  const int t = trow0 + qs * 32 + l32;
#pragma unroll
  for (int kx = 0; kx < 2; ++kx)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + kx * 32 + lg * 16 + i;
      const bool ok = key < N && (!causal || key <= t);
      if (!ok) s[kx][qs][i] = kMaskedScore;
    }
}

// Online softmax (fp32) of query tile qs against the running maximum as it
// stands; if a lane's probabilities grew too large (or m was still -inf),
// take the exact row maximum, rescale O and l and recompute.
template <int D, int QS, bool FIRST>
__device__ __forceinline__ void tile_softmax(const f32x16_t (&s)[2][QS], int qs, uint32_t (&pk)[2][QS][2][4],
                                             f32x16_t (&acc_o)[Cfg<D>::DSUB][QS], float (&m_run)[QS],
                                             float (&l_run)[QS], float c) {
  if constexpr (FIRST) {
    // the wave's first tile: m is still -inf, so take the tile's maximum
    // at once (O and l are zero: nothing to rescale)
    float mx = s[0][qs][0];
#pragma unroll
    for (int kx = 0; kx < 2; ++kx)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kx][qs][i]);
    const float cand = mx * c;
    m_run[qs] = fmaxf(cand, __shfl_xor(cand, 32));
    l_run[qs] += exp_rows<QS>(s, qs, pk, c, m_run[qs]);
    return;
  }
  float lsum = exp_rows<QS>(s, qs, pk, c, m_run[qs]);
  if (__ballot(!(lsum <= kSumLimit))) {
    float mx = s[0][qs][0];
#pragma unroll
    for (int kx = 0; kx < 2; ++kx)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kx][qs][i]);
    const float cand = mx * c;
    const float other = __shfl_xor(cand, 32);
    const float mnew = fmaxf(m_run[qs], fmaxf(cand, other));
    const float alpha = (m_run[qs] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[qs] - mnew);
    m_run[qs] = mnew;
    l_run[qs] *= alpha;
#pragma unroll
    for (int x = 0; x < Cfg<D>::DSUB; ++x)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_o[x][qs][i] *= alpha;
    lsum = exp_rows<QS>(s, qs, pk, c, m_run[qs]);
  }
  l_run[qs] += lsum;
}

// O^T += V^T P^T for query tile qs.
template <int D, int QS>
__device__ __forceinline__ void tile_pv(const uint16_t* vs, const uint32_t (&pk)[2][QS][2][4], int qs,
                                        f32x16_t (&acc_o)[Cfg<D>::DSUB][QS], int l32, int lg) {
  using C = Cfg<D>;
#pragma unroll
  for (int x = 0; x < C::DSUB; ++x)
#pragma unroll
    for (int kx = 0; kx < 2; ++kx)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const bf16x8_t vf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
            vs + (x * 32 + l32) * C::VROW + kx * 32 + lg * 16 + hh * 8));
        const u32x4_t pw = {pk[kx][qs][hh][0], pk[kx][qs][hh][1], pk[kx][qs][hh][2], pk[kx][qs][hh][3]};
        acc_o[x][qs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, as_bf16x8(pw), acc_o[x][qs], 0, 0, 0);
      }
}

// One K/V tile for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
// With two query tiles the MFMAs of one overlap the softmax of the other:
// S(1) is issued next to the softmax of tile 0, P(0).V next to that of tile 1.
// MASKED adds the causal and tail masks.
template <int D, int QS, bool MASKED, bool FIRST>
__device__ __forceinline__ void process_tile(const uint16_t* ks, const u32x4_t (&qf)[QS][Cfg<D>::DSTEPS],
                                             f32x16_t (&acc_o)[Cfg<D>::DSUB][QS], float (&m_run)[QS],
                                             float (&l_run)[QS], float c, int key0, int N, int causal,
                                             int trow0, int l32, int lg) {
  using C = Cfg<D>;
  const uint16_t* vs = ks + C::KBUF;
  bf16x8_t kf[2][C::DSTEPS];
#pragma unroll
  for (int kx = 0; kx < 2; ++kx)
#pragma unroll
    for (int ds = 0; ds < C::DSTEPS; ++ds)
      kf[kx][ds] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(ks + (kx * 32 + l32) * C::KROW + (ds * 2 + lg) * 8));

  f32x16_t s[2][QS];
  uint32_t pk[2][QS][2][4];  // [kx][qs][half][word] bf16 pairs
  tile_scores<D, QS>(kf, qf, 0, s);
  if constexpr (MASKED) mask_tile<QS>(s, 0, key0, N, causal, trow0, l32, lg);
  if constexpr (QS == 2) tile_scores<D, QS>(kf, qf, 1, s);
  tile_softmax<D, QS, FIRST>(s, 0, pk, acc_o, m_run, l_run, c);
  tile_pv<D, QS>(vs, pk, 0, acc_o, l32, lg);
  if constexpr (QS == 2) {
    if constexpr (MASKED) mask_tile<QS>(s, 1, key0, N, causal, trow0, l32, lg);
    tile_softmax<D, QS, FIRST>(s, 1, pk, acc_o, m_run, l_run, c);
    tile_pv<D, QS>(vs, pk, 1, acc_o, l32, lg);
  }
}

template <int D, int QS>
__global__ __launch_bounds__(kThreads, QS == 1 ? 4 : 2) void attn_fwd_bf16_kernel(Args a) {
  using C = Cfg<D>;
  constexpr int kRowsPerWave = 32 * QS;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, lg = lane >> 5;

  // ---- workgroup -> (key-range split, batch*Hkv, slot range); runs of 8
  // consecutive workgroups take one split index, so that the splits of
  // logical workgroup wid run on XCD wid % 8 (one split: wid = blockIdx.x)
  const int g8 = (int)(blockIdx.x >> 3), x8 = (int)(blockIdx.x & 7);
  const int split = g8 % a.nsplit;
  const int wid = (g8 / a.nsplit) * 8 + x8;
  if (wid >= a.nwg) return;
  int bkv, w_in;
  if (a.pair_major) {
    if (!pair_major_coords(wid, a.n_bkv, a.wg_per_bkv, bkv, w_in)) return;
  } else if (a.spread) {  // packed sequences, or uneven groups under a causal mask
    spread_coords(wid, a.n_bkv, a.wg_per_bkv, a.causal != 0, a.spread_block, bkv, w_in);
  } else if (a.exact_per_batch > 0) {  // uneven groups, encoder-style: XCD-contiguous, exact counts
    const int bid = wid;
    const int per = a.nwg / kXcds, rem = a.nwg % kXcds;
    const int x = bid % kXcds, i = bid / kXcds;
    exact_coords(x * per + min(x, rem) + i, a.exact_per_batch, a.Hq, a.Hkv,
                 (a.N + kRowsPerWave - 1) / kRowsPerWave, kWaves, bkv, w_in);
  } else if (!a.causal) {
    // consecutive logical workgroups on one XCD (hardware deals blockIdx
    // round-robin over the XCDs)
    const int bid = wid;
    const int per = a.nwg / kXcds, rem = a.nwg % kXcds;
    const int x = bid % kXcds, i = bid / kXcds;
    const int L = x * per + min(x, rem) + i;
    bkv = L / a.wg_per_bkv;
    w_in = L % a.wg_per_bkv;
  } else {
    // longest (largest position block) first; within every other full
    // round of `snake` workgroups the order runs backwards, so that the
    // CUs that took the longest blocks of one round take the shortest of
    // the next (measured on the SQAT-m attention, B16 N1024 (8,4) d = 16
    // causal: 24.1 -> 22.7 us)
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
  // workgroups past this group's (or this sequence's) rows leave at once
  if (w_in * kWaves >= TB * g) return;
  const int slot = w_in * kWaves + wave;
  const int tb = slot / g, jh = slot % g;
  const bool wave_valid = tb < TB;
  const int h = hg.first + jh;

  // key tiles the workgroup streams and the wave's last one (causal: the
  // tile holding its last row, which is also its only masked diagonal tile)
  const int NT = (N + kTileKeys - 1) / kTileKeys;
  int nt;
  if (a.causal) {
    const int maxtb = min((w_in * kWaves + kWaves - 1) / g, TB - 1);
    nt = min((maxtb * kRowsPerWave + kRowsPerWave - 1) / kTileKeys + 1, NT);
  } else {
    nt = NT;
  }
  const int diag = min((tb * kRowsPerWave + kRowsPerWave - 1) / kTileKeys, NT - 1);
  // key-range split: this workgroup streams key tiles [kt0, kt_end) of its
  // rows. A causal wave holds at most 64 rows, one tile's worth, so it sees
  // a key of every row in a range that starts at or before its diagonal tile
  // (kt0 * 64 <= its first row) and none in a later one.
  const int chunk = split_chunk(NT, a.nsplit, kMinSplitTiles64, false);
  const bool split_rows = NT > chunk;
  const int kt0 = split * chunk;
  if (kt0 >= nt) return;
  const int kt_end = min(nt, kt0 + chunk);
  const int wave_last = min(a.causal ? diag : nt - 1, kt_end - 1);

  const int64_t kvrow0 = sg.kv_base + (int64_t)kvh * sg.stride;
  const int64_t qrow0 = sg.q_base + (int64_t)h * sg.stride;
  const uint16_t* kbase = a.k + (size_t)kvrow0 * D;
  const uint16_t* vbase = a.v + (size_t)kvrow0 * D;
  const size_t qoff = (size_t)qrow0 * D;

  // ---- Q fragments (B operand): query l32 of each 32-row tile, d chunk ds*2+lg
  u32x4_t qf[QS][C::DSTEPS];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const int t = min(tb * kRowsPerWave + qs * 32 + l32, N - 1);
#pragma unroll
    for (int ds = 0; ds < C::DSTEPS; ++ds) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (wave_valid) x = *reinterpret_cast<const u32x4_t*>(a.q + qoff + (size_t)t * D + (ds * 2 + lg) * 8);
      x ^= a.qsign;
      qf[qs][ds] = x;
    }
  }

  // V^T rows that hold no head dimension (D < 32) must read as finite zeros.
  // At d = 16 the rows pi_inv(d), d < 16, are those with bit 2 clear; the
  // other 16 rows of each buffer are zeroed here, 16 bytes per store.
  if constexpr (C::VROWS > D) {
    static_assert(D == 16, "only d = 16 pads V^T");
    constexpr int kRowChunks = C::VROW * 2 / 16;  // 16-byte chunks per V^T row
    static_assert(C::VROW * 2 % 16 == 0 && C::KBUF * 2 % 16 == 0 && C::BUF * 2 % 16 == 0, "16-byte rows");
    for (int e = tid; e < 2 * 16 * kRowChunks; e += kThreads) {
      const int bsel = e / (16 * kRowChunks), rem = e % (16 * kRowChunks);
      const int pr = rem / kRowChunks, ch = rem % kRowChunks;
      const int lr = ((pr >> 2) << 3) + 4 + (pr & 3);
      uint8_t* row = reinterpret_cast<uint8_t*>(smem + bsel * C::BUF + C::KBUF + lr * C::VROW);
      *reinterpret_cast<u32x4_t*>(row + ch * 16) = u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  f32x16_t acc_o[C::DSUB][QS];
#pragma unroll
  for (int x = 0; x < C::DSUB; ++x)
#pragma unroll
    for (int qs = 0; qs < QS; ++qs)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_o[x][qs][i] = 0.f;
  float m_run[QS], l_run[QS];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    m_run[qs] = -INFINITY;
    l_run[qs] = 0.f;
  }

  TileRegs<D> regs;
  load_tile<D>(regs, kbase, vbase, kt0, N, tid);
  __syncthreads();  // zero-fill above is complete before tile stores
  store_tile<D>(regs, smem, tid);
  __syncthreads();

  const float c = a.c;
  for (int kt = kt0; kt < kt_end; ++kt) {
    const int cur = (kt - kt0) & 1;
    if (kt + 1 < kt_end) load_tile<D>(regs, kbase, vbase, kt + 1, N, tid);

    if (wave_valid && kt <= wave_last) {
      const uint16_t* ks = smem + cur * C::BUF;
      const int key0 = kt * kTileKeys;
      const bool masked = (a.causal && kt == diag) || (key0 + kTileKeys > N);
      const int trow0 = tb * kRowsPerWave;
      // d = 16 takes the first tile's maximum at once (SQAT-m attention
      // 27.5 -> 25.9 us with the padded-row zero fill above); at d = 32 the
      // extra tile variant cost 3-4 % and the first tile stays on the lazy path
      if (D == 16 && kt == kt0) {
        if (masked)
          process_tile<D, QS, true, true>(ks, qf, acc_o, m_run, l_run, c, key0, N, a.causal, trow0, l32, lg);
        else
          process_tile<D, QS, false, true>(ks, qf, acc_o, m_run, l_run, c, key0, N, a.causal, trow0, l32, lg);
      } else if (masked) {
        process_tile<D, QS, true, false>(ks, qf, acc_o, m_run, l_run, c, key0, N, a.causal, trow0, l32, lg);
      } else {
        process_tile<D, QS, false, false>(ks, qf, acc_o, m_run, l_run, c, key0, N, a.causal, trow0, l32, lg);
      }
    }

    if (kt + 1 < kt_end) store_tile<D>(regs, smem + (cur ^ 1) * C::BUF, tid);
    __syncthreads();
  }

  if (!wave_valid) return;

  if (split_rows) {
    // ---- split epilogue: unnormalised O^T, m and l of this key range (fp32)
    if (wave_last < kt0) return;  // no key of this range for the wave's rows
    float* po = a.part + ((size_t)split * a.rows + qrow0) * D;
    float* pml = a.part + (size_t)a.nsplit * a.rows * D + ((size_t)split * a.rows + qrow0) * 2;
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      const float ltot = l_run[qs] + __shfl_xor(l_run[qs], 32);
      const int t = tb * kRowsPerWave + qs * 32 + l32;
      if (t < N) {
#pragma unroll
        for (int x = 0; x < C::DSUB; ++x) {
          const int d0 = x * 32 + lg * 16;
          if (d0 < D) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const f32x4_t v4 = {acc_o[x][qs][4 * e], acc_o[x][qs][4 * e + 1], acc_o[x][qs][4 * e + 2],
                                  acc_o[x][qs][4 * e + 3]};
              *reinterpret_cast<f32x4_t*>(po + (size_t)t * D + d0 + 4 * e) = v4;
            }
          }
        }
        if (lg == 0) *reinterpret_cast<f32x2_t*>(pml + (size_t)t * 2) = f32x2_t{m_run[qs], ltot};
      }
    }
    return;
  }

  // ---- epilogue: O = O^T / l (bf16, nearest even), LSE = m ln2 + ln l
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const float ltot = l_run[qs] + __shfl_xor(l_run[qs], 32);
    const float inv = 1.0f / ltot;
    const int t = tb * kRowsPerWave + qs * 32 + l32;
    if (t < N) {
#pragma unroll
      for (int x = 0; x < C::DSUB; ++x) {
        const int d0 = x * 32 + lg * 16;
        if (d0 < D) {
          u32x4_t w0, w1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w0[e] = pack_bf16x2(acc_o[x][qs][2 * e] * inv, acc_o[x][qs][2 * e + 1] * inv);
            w1[e] = pack_bf16x2(acc_o[x][qs][8 + 2 * e] * inv, acc_o[x][qs][8 + 2 * e + 1] * inv);
          }
          uint16_t* dst = a.o + qoff + (size_t)t * D + d0;
          // non-temporal: no dirty L2 line left to write back at the end
          // (SQAT-m attention: 22.8 -> 22.1 us)
          __builtin_nontemporal_store(w0, reinterpret_cast<u32x4_t*>(dst));
          __builtin_nontemporal_store(w1, reinterpret_cast<u32x4_t*>(dst + 8));
        }
      }
      if (a.lse != nullptr && lg == 0) {
        a.lse[(size_t)qrow0 + t] = (m_run[qs] + log2f(ltot)) * 0.69314718055994531f;
      }
    }
  }
}

template <int D, int QS>
hipError_t launch_d(const AttnProblem& p, hipStream_t stream) {
  constexpr int kRowsPerWave = 32 * QS;
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
  a.snake = (!p.dry_run && p.causal && !a.spread && a.exact_per_batch == 0 && !a.pair_major) ? device_cus() : 0;
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
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, QS>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
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
  m.min_tiles = kMinSplitTiles64;
  m.even = 0;
  return launch_split_merge<D>(m, stream, p.dry_run);
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnProblem& p, hipStream_t stream) {
  if (p.D == 64) return launch_attn_fwd_bf16_d64(p, stream);
  if (p.tail_split > 1) return hipErrorInvalidValue;  // the tail split is a d = 64 schedule
  // Unsplit d = 16 and d = 32: the kernels that fold the scale and the
  // running maximum into the score MFMAs (attn_fwd_bf16_d16.hip,
  // attn_fwd_bf16_d32.hip). This one serves their key-range splits (and the
  // longest N): under a causal mask with 32-row waves (112 VGPRs, four waves
  // per SIMD), whose extra waves hide the latency of the short causal tile
  // chains (B16 N1024 (8,4): 27.7 -> 23.1 us; N = 4096: +20 %; N = 32768:
  // +9 %); encoder-style d = 16 and d = 32 with 64-row waves.
  if (p.D == 16 && p.nsplit <= 1 && p.N * 32 < 0x7fffffffLL) return launch_attn_fwd_bf16_d16(p, stream);
  if (p.D == 16) return p.causal ? launch_d<16, 1>(p, stream) : launch_d<16, 2>(p, stream);
  if (p.D == 32 && p.nsplit <= 1 && p.N * 64 < 0x7fffffffLL) return launch_attn_fwd_bf16_d32(p, stream);
  if (p.D == 32) return launch_d<32, 2>(p, stream);
  if (p.D == 128) return launch_attn_fwd_bf16_d128(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace sqa
