// Head groups and sequence geometry shared by the attention kernels.
//
// Head groups: query head i reads K/V head floor(i*H_kv/H_q) (contiguous
// query-head groups, "GQA ..." page, "The idea"). The query heads of K/V head
// j are then i in [first, first + count) with first = ceil(j*H_q/H_kv); group
// sizes differ by at most one and are >= 1 when H_kv <= H_q, and equal
// H_q/H_kv when H_kv divides H_q.
//
// Sequences: dense tensors are [B, H, N, d]; packed variable-length tensors
// are [H, T, d] with sequence b owning tokens cu[b] .. cu[b+1]-1 of every
// head. In both, row t of sequence b, head h is row base + h*stride + t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sqa {

struct HeadGroup {
  int first, count;
};

__host__ __device__ __forceinline__ HeadGroup head_group(int j, int Hq, int Hkv) {
  const int first = (j * Hq + Hkv - 1) / Hkv;
  const int next = ((j + 1) * Hq + Hkv - 1) / Hkv;
  return HeadGroup{first, next - first};
}

// largest group: ceil(H_q / H_kv)
__host__ __device__ __forceinline__ int max_group(int Hq, int Hkv) { return (Hq + Hkv - 1) / Hkv; }

struct SeqGeom {
  int64_t q_base;   // row of (sequence b, query head 0, t = 0)
  int64_t kv_base;  // row of (sequence b, K/V head 0, t = 0)
  int64_t stride;   // rows between consecutive heads
  int n;            // rows of the sequence
};

// cu == nullptr: dense, every sequence has N rows. Otherwise packed with
// offsets cu[0..B] into T tokens; the offsets are clamped into [0, T] and the
// length to at most N (the longest sequence the launch was sized for), so a
// bad offset array cannot move any access outside the tensors.
__device__ __forceinline__ SeqGeom seq_geom(const int* cu, int64_t T, int N, int b, int Hq, int Hkv) {
  SeqGeom g;
  if (cu == nullptr) {
    g.q_base = (int64_t)b * Hq * N;
    g.kv_base = (int64_t)b * Hkv * N;
    g.stride = N;
    g.n = N;
  } else {
    int64_t s = cu[b], e = cu[b + 1];
    s = s < 0 ? 0 : (s > T ? T : s);
    e = e < s ? s : (e > T ? T : e);
    g.q_base = s;
    g.kv_base = s;
    g.stride = T;
    g.n = (int)(e - s < (int64_t)N ? e - s : (int64_t)N);
  }
  return g;
}

// Workgroup -> (b*H_kv + K/V head, workgroup index within it) for launches
// whose workgroups differ in work beyond the causal triangle: uneven head
// groups or packed sequences of different lengths. Workgroup indices are
// outermost (descending if `descending`, so that under a causal mask the
// longest rows start first) and the (batch, K/V head) pairs are rotated by
// one every `block` indices. block = 1 deals the workgroups of any one pair
// -- one long sequence, one large group -- over all XCDs instead of landing
// on one. A larger block keeps runs of consecutive workgroups of one XCD
// (bid, bid + 8, ...) on the same pair, so that they stream the same K/V
// tiles close together in time and share that XCD's L2, while the rotation
// still evens out the work of groups of different sizes.
__device__ __forceinline__ void spread_coords(int bid, int n_bkv, int wg_per_bkv, bool descending, int block,
                                              int& bkv, int& w_in) {
  const int wr = bid / n_bkv, r = bid % n_bkv;
  bkv = (r + wr / block) % n_bkv;
  w_in = descending ? wg_per_bkv - 1 - wr : wr;
}

// Pair-major order for packed encoder-style launches: XCD x (= wid % 8)
// walks the (sequence, K/V head) pairs in turn and takes, of each, the
// workgroup indices w_in = x, x + 8, x + 16, ...; every pair is dealt evenly
// over the XCDs, and consecutive workgroups of an XCD share one pair's K/V
// in its L2. The grid covers n_bkv * ceil(wg_per_bkv / 8) * 8 logical
// workgroups (pair_major_nwg); indices past a pair's last workgroup exit.
__device__ __forceinline__ bool pair_major_coords(int wid, int n_bkv, int wg_per_bkv, int& bkv, int& w_in) {
  const int J = (wg_per_bkv + 7) / 8;
  const int x = wid & 7, k = wid >> 3;
  bkv = k / J;
  w_in = (k % J) * 8 + x;
  return bkv < n_bkv && w_in < wg_per_bkv;
}
__host__ __forceinline__ int64_t pair_major_nwg(int64_t n_bkv, int64_t wg_per_bkv) {
  return n_bkv * ((wg_per_bkv + 7) / 8) * 8;
}

// Rotation block for spread_coords. Packed sequences: 1 (a block would put
// the workgroups of the longest sequence on one XCD: 2-4x slower). Dense
// batches with uneven head groups: 16 once there are at least four
// (batch, K/V head) pairs. Measured at N = 32768, d = 64 on MI355X, this took
// the causal forward of (12,8) from 766 to 1030 TFLOP/s, (20,8) from 856 to
// 1078 and (6,4) from 818 to 979, and the backward of (12,8) from 599 to 665
// (causal 571 to 692); with two or three pairs the one-step rotation already
// keeps each XCD on one pair and stayed about 3 % ahead.
__host__ __forceinline__ int spread_block(bool packed, int64_t n_bkv) { return (!packed && n_bkv >= 4) ? 16 : 1; }

// Workgroups of K/V head j when each takes W slots of (position block,
// query head) and a head has TB position blocks.
__host__ __device__ __forceinline__ int group_wgs(int j, int Hq, int Hkv, int TB, int W) {
  return (TB * head_group(j, Hq, Hkv).count + W - 1) / W;
}

// Logical workgroup L -> (b*H_kv + K/V head, index within it) for a grid of
// exactly B * per_batch workgroups, per_batch = sum_j group_wgs(j): groups
// of different sizes get their own counts, so consecutive L stay on one
// K/V head (shared L2 under an XCD-contiguous order) with no idle
// workgroups. A scalar walk over the H_kv groups.
__device__ __forceinline__ void exact_coords(int L, int per_batch, int Hq, int Hkv, int TB, int W, int& bkv,
                                             int& w_in) {
  const int b = L / per_batch;
  int r = L % per_batch, j = 0;
  for (; j < Hkv - 1; ++j) {
    const int n = group_wgs(j, Hq, Hkv, TB, W);
    if (r < n) break;
    r -= n;
  }
  bkv = b * Hkv + j;
  w_in = r;
}

// Range splits: with S splits the NT tiles of a sequence are cut into
// chunks of split_chunk(NT, S, ...) tiles (split s takes tiles
// [s*chunk, (s+1)*chunk)); a sequence with NT <= chunk is not split. A
// chunk holds at least min_tiles tiles; `even` rounds it up to an even
// count, which the 32-key-tile kernels need so that a causal wave of 64
// rows either sees a key of every row in a range or none (the 64-key-tile
// kernel needs no rounding: its waves hold at most 64 rows).
constexpr int kMinSplitTiles = 32;   // 32-key (or 32-row) tiles: ranges of >= 1024
constexpr int kMinSplitTiles64 = 4;  // 64-key tiles: ranges of >= 256 keys
__host__ __device__ __forceinline__ int split_chunk(int NT, int nsplit, int min_tiles, bool even) {
  int c = (NT + nsplit - 1) / nsplit;
  if (even) c = (c + 1) & ~1;
  return c < min_tiles ? min_tiles : c;
}
__host__ __device__ __forceinline__ int split_chunk(int NT, int nsplit) {
  return split_chunk(NT, nsplit, kMinSplitTiles, true);
}

}  // namespace sqa
