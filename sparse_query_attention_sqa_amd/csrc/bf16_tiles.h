// Shared gfx950 building blocks for the head-dim-64 bf16 attention kernels:
// operand types, the LDS tile layouts, HBM->LDS DMA of 32-row tiles and the
// MFMA operand reads.
//
// Tiles are 32 rows x 64 bf16 (128 B per row, 4 KB), row-major in LDS with
// the row's eight 16-byte chunks XOR-swizzled. Two layouts serve the two ways
// a tile feeds v_mfma_f32_32x32x16_bf16:
//   * "row layout": LDS row r holds tile row pi(r) (swizzle swz_k). Read with
//     read_rows, it is the A operand with M = tile rows and K = head dims;
//     the permutation pi makes entry i of accumulator lane-half lg belong to
//     tile row lg*16 + i.
//   * "transposed layout": LDS row r holds tile row r (swizzle swz_v). Read
//     with read_tr (ds_read_b64_tr_b16), it is the A operand with M = head
//     dims and K = tile rows, with k position (hh, lg, s) <-> tile row
//     lg*16 + hh*8 + s -- the order in which pack_pairs lays a row-layout
//     accumulator out as a B operand.
// MFMA lane layout (v_mfma_f32_32x32x16_bf16): A lane l -> row l%32,
// k = (l/32)*8 + s; B lane l -> column l%32, same k; accumulator entry i of
// lane l -> row 8*(i/4) + (l/32)*4 + i%4, column l%32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sqa {
namespace tiles {

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

constexpr int kD = 64;                         // head dim
constexpr int kTileRows = 32;
constexpr int kRowBytes = kD * 2;              // 128 B
constexpr int kTileBytes = kTileRows * kRowBytes;  // 4 KB
constexpr int kBufferWord3 = 0x00020000;       // raw buffer descriptor flags (gfx9)

__device__ __forceinline__ int pi_row(int r) { return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3); }
__device__ __forceinline__ int swz_k(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_v(int r) { return 2 * (r & 3); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ f32x16_t mfma(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Per-lane byte offsets. A wave DMAs 8 tile rows (rows 8*part .. 8*part+7)
// of one tile, one 16-byte chunk per lane; these are the lane's source
// offsets within the tile for the two layouts. RB is the row pitch of the
// array in HBM: 128 B for head dim 64; for head dim 128 a tile is two 64-wide
// halves, and half h adds h*128 to the offset.
template <int RB = kRowBytes>
__device__ __forceinline__ uint32_t dma_off_rows(int part, int lane) {
  const int r = part * 8 + (lane >> 3), s = lane & 7;
  return (uint32_t)(pi_row(r) * RB + ((s ^ swz_k(r)) * 16));
}
template <int RB = kRowBytes>
__device__ __forceinline__ uint32_t dma_off_tr(int part, int lane) {
  const int r = part * 8 + (lane >> 3), s = lane & 7;
  return (uint32_t)(r * RB + ((s ^ swz_v(r)) * 16));
}

// Read offsets within a tile: row-layout A fragments (k steps ds = 0..3) and
// transposed-layout fragments (x = head-dim half 0/1).
struct ReadOffsets {
  uint32_t rows[4];
  uint32_t tr[2];
  uint32_t tr_hi[2];  // shared layout only: the same reads 8 LDS rows further on
};
__device__ __forceinline__ ReadOffsets read_offsets(int lane) {
  ReadOffsets o;
  const int l32 = lane & 31, lg = lane >> 5;
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) o.rows[ds] = (uint32_t)(l32 * kRowBytes + (((ds * 2 + lg) ^ swz_k(l32)) * 16));
  const int j16 = lane & 15, g1 = (lane >> 4) & 1;
  const int row = lg * 16 + (j16 >> 2);
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int c16 = x * 4 + 2 * g1 + ((j16 & 3) >> 1);
    o.tr[x] = (uint32_t)(row * kRowBytes + ((c16 ^ swz_v(row)) * 16) + (j16 & 1) * 8);
  }
  return o;
}

// "Shared layout": LDS row r holds tile row pi(r), as in the row layout, but
// with the swizzle swz_s(r) = f((r>>1)&7), f(k) = 4*(k&1) + (k>>1). The LDS
// has 64 four-byte banks (256 B); a 16-byte read serves 16 lanes per cycle
// and a ds_read_b64_tr_b16 32 lanes. Rows of one parity in an aligned block
// of 16 then take eight different chunk positions (row reads: 16 rows, one
// logical chunk, conflict-free), and rows R and R+2 of an aligned block of 4
// differ in bit 2 of the swizzle, so their 64-byte halves land in opposite
// bank halves (transposed reads: 4 rows x 4 chunks, conflict-free). One copy
// of a tile thus serves both operand forms: read_rows with
// read_offsets_shared().rows, and read_tr_shared, whose k position
// (hh, lg, s) <-> tile row lg*16 + hh*8 + s sits at LDS row hh*16 + lg*4 + s
// (s < 4) or hh*16 + 8 + lg*4 + s - 4 (s >= 4).
__device__ __forceinline__ int swz_s(int r) {
  const int k = (r >> 1) & 7;
  return ((k & 1) << 2) | (k >> 1);
}
template <int RB = kRowBytes>
__device__ __forceinline__ uint32_t dma_off_shared(int part, int lane) {
  const int r = part * 8 + (lane >> 3), s = lane & 7;
  return (uint32_t)(pi_row(r) * RB + ((s ^ swz_s(r)) * 16));
}
__device__ __forceinline__ ReadOffsets read_offsets_shared(int lane) {
  ReadOffsets o;
  const int l32 = lane & 31, lg = lane >> 5;
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) o.rows[ds] = (uint32_t)(l32 * kRowBytes + (((ds * 2 + lg) ^ swz_s(l32)) * 16));
  const int j16 = lane & 15, g1 = (lane >> 4) & 1;
  const int row = lg * 4 + (j16 >> 2);
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int c16 = x * 4 + 2 * g1 + ((j16 & 3) >> 1);
    // swz_s ignores bit 4 of the row (the hh * 16 rows read_tr_shared adds)
    // but not bit 3, so the reads 8 rows on get their own offsets
    o.tr[x] = (uint32_t)(row * kRowBytes + ((c16 ^ swz_s(row)) * 16) + (j16 & 1) * 8);
    o.tr_hi[x] = (uint32_t)((row + 8) * kRowBytes + ((c16 ^ swz_s(row + 8)) * 16) + (j16 & 1) * 8);
  }
  return o;
}

// DMA one wave's 8 rows of a tile that starts at row `row0` of a bf16
// array with RB-byte rows whose valid rows end at `nlim`; rows at or past
// nlim are zero-filled by the descriptor range check without any memory
// access.
template <int RB = kRowBytes>
__device__ __forceinline__ void dma_tile_part(const uint16_t* base, int row0, int nlim, uint8_t* lds_part,
                                              uint32_t voff) {
  const int rem = max(nlim - row0, 0) * RB;
  __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)row0 * (RB / 2)), (short)0, rem, kBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_part, 16, voff, 0, 0, 0);
}

// Row-layout A fragments of the tile at `tile` (k steps 0..3).
__device__ __forceinline__ void read_rows(const uint8_t* tile, const ReadOffsets& ro, u32x4_t (&f)[4]) {
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) f[ds] = *reinterpret_cast<const u32x4_t*>(tile + ro.rows[ds]);
}

// Transposed-layout A fragments [x][hh] of the tile at `tile`: head-dim row
// x*32 + l%32 against tile rows lg*16 + hh*8 + 0..7.
__device__ __forceinline__ void read_tr(const uint8_t* tile, const ReadOffsets& ro, u32x4_t (&f)[2][2]) {
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint8_t* p = tile + ro.tr[x] + hh * 8 * kRowBytes;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * kRowBytes));
      const u32x2_t a = __builtin_bit_cast(u32x2_t, lo);
      const u32x2_t b = __builtin_bit_cast(u32x2_t, hi);
      f[x][hh] = u32x4_t{a[0], a[1], b[0], b[1]};
    }
}

// Transposed A fragments [x][hh] of a shared-layout tile (see read_tr for
// the operand; the k positions map to LDS rows as stated at swz_s).
__device__ __forceinline__ void read_tr_shared(const uint8_t* tile, const ReadOffsets& ro, u32x4_t (&f)[2][2]) {
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const s16x4_t lo =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + ro.tr[x] + hh * 16 * kRowBytes));
      const s16x4_t hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + ro.tr_hi[x] + hh * 16 * kRowBytes));
      const u32x2_t a = __builtin_bit_cast(u32x2_t, lo);
      const u32x2_t b = __builtin_bit_cast(u32x2_t, hi);
      f[x][hh] = u32x4_t{a[0], a[1], b[0], b[1]};
    }
}

// B-operand fragments (k = head dims) of one 64-wide row taken straight from
// global memory: lane l holds dims (ds*2 + l/32)*8 .. +8 of `row`.
__device__ __forceinline__ void load_row_frags(const uint16_t* row, int lg, u32x4_t (&f)[4]) {
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) f[ds] = *reinterpret_cast<const u32x4_t*>(row + (ds * 2 + lg) * 8);
}

// acc (+)= A_rows . B over the 4 head-dim k steps.
__device__ __forceinline__ f32x16_t mfma_k64(const u32x4_t (&a)[4], const u32x4_t (&b)[4]) {
  f32x16_t acc = zero16();
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) acc = mfma(a[ds], b[ds], acc);
  return acc;
}

// o[x] += A_tr[x] . P over the 32 tile rows (two k steps of 16).
__device__ __forceinline__ void mfma_tr(const u32x4_t (&a)[2][2], const u32x4_t (&p)[2], f32x16_t (&o)[2]) {
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int x = 0; x < 2; ++x) o[x] = mfma(a[x][hh], p[hh], o[x]);
}

// Round a row-layout accumulator's 16 entries to bf16 pairs laid out as the
// B operand (k = tile rows) for mfma_tr.
__device__ __forceinline__ void pack_pairs(const f32x16_t& v, u32x4_t (&p)[2]) {
#pragma unroll
  for (int w = 0; w < 8; ++w) p[w >> 2][w & 3] = pack_bf16x2(v[2 * w], v[2 * w + 1]);
}

// Write a transposed accumulator pair o[x] (entry i of lane l: head dim
// x*32 + 8*(i/4) + 4*(l/32) + i%4 of output row l%32) times `mul` as bf16.
__device__ __forceinline__ void store_tr_row(uint16_t* row, const f32x16_t (&o)[2], float mul, int lg) {
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int ab = 0; ab < 4; ++ab) {
      u32x2_t wv;
      wv[0] = pack_bf16x2(o[x][4 * ab] * mul, o[x][4 * ab + 1] * mul);
      wv[1] = pack_bf16x2(o[x][4 * ab + 2] * mul, o[x][4 * ab + 3] * mul);
      *reinterpret_cast<u32x2_t*>(row + x * 32 + 8 * ab + 4 * lg) = wv;
    }
}

}  // namespace tiles
}  // namespace sqa
