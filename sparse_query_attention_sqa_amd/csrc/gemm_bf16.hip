// bf16 GEMMs of the SQA layer and the SQAT-m block on gfx950, with fused
// epilogues (SQAT-m model card, "Architecture details": RoPE, RMS Norm,
// SwiGLU feed forward; "Model size difference": H_q*d-wide query and output
// projections, H_kv*d-wide key and value projections).
//
//   C [M, n-range] = A [M, K] . W [K, n-range],  A row-major (or the
//   attention output O [B, Hq, N, d] read as O_flat [B*N, Hq*d]), W [K, Ncols]
//   row-major, fp32 accumulation (v_mfma_f32_32x32x16_bf16).
//
// Formulation: C^T = W^T A^T, so that W^T is the MFMA A operand read with
// ds_read_b64_tr_b16 from W stored row-major in LDS, and A^T the B operand
// read as 16-byte row chunks -- the layouts of bf16_tiles.h. Each lane then
// owns one output row and runs of 4 consecutive columns, so RoPE partners
// (c and c +- d/2), SwiGLU's gate and up, and the residual all meet in
// registers.
//
// Tiling: the output columns are cut into 64-wide segments of the weight
// parts (W_q | W_k | W_v for the QKV projection, one matrix otherwise); a
// 4-wave workgroup computes 64*MB rows x two segments (SwiGLU: one segment of
// both gate and up), and wave (wm, wn) owns 32*MB rows of segment wn as 2*MB
// 32x32 accumulators (MB = 2, or 1 for small grids, which then get twice the
// workgroups). The reduction runs in 64-wide chunks, DMA'd HBM -> LDS with
// buffer_load ... lds into a ring of S stages with S-1 chunks in flight
// (S = 3 with MB = 1 for small grids, S = 2 otherwise); rows past M,
// columns past the part's width and reduction indices past K -- including
// whole chunks past the end, so every step issues the same DMAs and the
// waits are exact -- are zero-filled by the descriptor's range check (their
// lanes get an out-of-range offset).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bf16_tiles.h"
#include "kernels.h"

namespace sqa {
namespace {

using namespace tiles;

constexpr int kThreads = 256;
constexpr int TK = 64;                       // reduction chunk
constexpr uint32_t kOOB = 0x80000000u;       // an offset past every descriptor range

// MB = 32-row blocks per wave: a workgroup (two waves along the rows) takes
// TM = 64*MB rows; a stage holds the A tiles ([32 m][64 k], 2*MB of them)
// and the 4 W tiles ([32 k][64 n]).
template <int MB>
struct Tiling {
  static_assert(MB == 1 || MB == 2, "32 or 64 rows per wave");
  static constexpr int TM = 64 * MB;
  static constexpr int kATiles = 2 * MB;
  static constexpr int kStageBytes = (kATiles + 4) * kTileBytes;
  static constexpr int kAParts = 2 * MB;      // A DMAs (8 rows each) per wave per chunk
  static constexpr int kDma = kAParts + 4;    // DMAs per wave per chunk
};

// s_waitcnt immediate (gfx9 encoding): vmcnt vm, expcnt 7, lgkmcnt 0.
constexpr int waitcnt_vm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_QKV = 2 };

// Where the reduction operand rows come from.
struct ARows {
  const uint16_t* p;
  int64_t M, K;
  int gather;      // 1: O [B, Hq, N, d] read as O_flat
  int64_t N, Hq, d;
};

// One weight part: a [K, ncols] row-major matrix.
struct WPart {
  const uint16_t* w;
  int64_t ncols;
};

struct GemmArgs {
  ARows A;
  WPart part[3];      // QKV: W_q, W_k, W_v; SwiGLU: gate, up; store: one
  int nparts;
  int segs[3];        // 64-column segments of each part
  int segs_total;     // sum of segs
  int tiles_total;    // column tiles: ceil(segs_total / 2) (SwiGLU: segs[0])
  int epi;
  // store epilogue
  const uint16_t* resid;  // [M, ncols] or nullptr
  uint16_t* y;            // [M, ncols] (SwiGLU: h [M, F])
  // QKV epilogue
  uint16_t* qkv[3];       // Q [B,Hq,N,d], K/V [B,Hkv,N,d]
  double rope_theta[32];  // rope_base^(-2c/d) / (2 pi): revolutions per position, pair c < d/2
  int64_t Nseq, Hq, Hkv, d;
};

// Row part of the byte offset of A[m][k] for a DMA lane, fixed across the
// reduction (element units): row-major m*K, gathered ((b*Hq)*N + t)*d. All
// offsets fit in 32 bits (checked at launch); d is a power of two.
template <bool GATHER>
__device__ __forceinline__ uint32_t a_row_base(const ARows& A, uint32_t m) {
  if (!GATHER) return m * (uint32_t)A.K;
  const uint32_t n = (uint32_t)A.N;
  const uint32_t b = m / n, t = m - b * n;
  return ((b * (uint32_t)A.Hq) * n + t) * (uint32_t)A.d;
}

// Byte offset of A[m][k .. k+8) given the row base (kOOB when outside);
// branch-free so that the per-lane conditions become selects.
template <bool GATHER>
__device__ __forceinline__ uint32_t a_offset(const ARows& A, uint32_t base, bool row_ok, uint32_t k,
                                             uint32_t dshift) {
  uint32_t e;
  if constexpr (GATHER) {
    const uint32_t h = k >> dshift, c = k & ((1u << dshift) - 1u);
    e = base + ((h * (uint32_t)A.N) << dshift) + c;
  } else {
    e = base + k;
  }
  return (row_ok && k < (uint32_t)A.K) ? e * 2u : kOOB;
}

// silu(g) * u with the hardware exp2 and reciprocal (about 1 ulp each):
// g / (1 + e^-g) = g * rcp(1 + 2^(-g log2 e)); saturates to 0 and to g.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * g);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int nrec = (int)min(bytes, (int64_t)0x7fffffff);
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nrec, kBufferWord3);
}

// QKV epilogue values of one 32-row block mb of a wave's accumulators
// (lane row at position t of its sequence, part `part`): wv[x][ab] holds
// the bf16 pairs of columns x*32 + 8*ab + 4*lg + 0..3 of the segment, with
// RoPE (rotate-half pairs (c, c + d/2)) applied to Q and K.
template <int MB>
__device__ __forceinline__ void qkv_rows(const GemmArgs& a, const f32x16_t (&acc)[2][MB], int mb, uint32_t t,
                                         int part, int lg, u32x2_t (&wv)[2][4]) {
  const int64_t d = a.d, half = d / 2;
  const bool rope = part < 2;
  // (cos, sin) of the angle t * theta_kp for pair indices
  // kp = 8*ab + 4*lg + e (mod half) of row t; for d = 16 one group of
  // four serves all. The angle is formed in revolutions and reduced to
  // [0, 1) in fp64, so that its rounding error does not grow with t, and
  // v_cos_f32 / v_sin_f32 take it in revolutions (measured on gfx950:
  // at most 1.3e-7 absolute error over [0, 1)).
  float2 cs[4][4];
  if (rope) {
#pragma unroll
    for (int ab = 0; ab < 4; ++ab) {
      if (d == 16 && ab > 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) cs[ab][e] = cs[0][e];
        continue;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // both candidates are lane-uniform (scalar loads from the kernel
      // arguments); a lane-indexed read became a global load whose
      // latency the epilogue waited out
      const double th0 = a.rope_theta[8 * ab + e], th1 = a.rope_theta[8 * ab + 4 + e];
      const double th = lg ? th1 : th0;
        const double rev = (double)t * th;
        const float f = (float)(rev - floor(rev));
        cs[ab][e] = make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
      }
    }
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int ab = 0; ab < 4; ++ab) {
      // column within the head: segments start on a head boundary
      const int64_t c0 = (x * 32 + 8 * ab + 4 * lg) & (d - 1);
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xv = acc[x][mb][4 * ab + e];
        if (!rope) {
          v[e] = xv;
          continue;
        }
        // the partner column c0 + e -+ d/2 of the same head sits in this
        // lane: d = 16 -> entry 4*(ab^1) + e of the same slot; d = 64 ->
        // the same entry of the other slot
        const float xp = (d == 16) ? acc[x][mb][4 * (ab ^ 1) + e] : acc[x ^ 1][mb][4 * ab + e];
        const float2 c2 = cs[ab][e];
        v[e] = (c0 + e < half) ? xv * c2.x - xp * c2.y : xp * c2.y + xv * c2.x;
      }
      wv[x][ab][0] = pack_bf16x2(v[0], v[1]);
      wv[x][ab][1] = pack_bf16x2(v[2], v[3]);
    }
}

// Epilogue of one 32-row block mb of a wave's accumulators: lane row m,
// columns nb + x*32 + 8*(i/4) + 4*lg + i%4 of weight part `part`. EPI_STORE:
// y [M, ncols] (+ the residual); EPI_QKV: RoPE on Q and K, scatter to
// [B, H, N, d].
template <int EPI, int MB>
__device__ __forceinline__ void store_rows(const GemmArgs& a, const f32x16_t (&acc)[2][MB], int mb, int64_t m, int part,
                                          int64_t nb, int lg) {
  if (EPI == EPI_STORE) {
    const int64_t ncols = a.part[0].ncols;
    // every residual load first: y may alias the residual, so a load placed
    // after a store of the row cannot move above it, and interleaved they
    // would pay one memory latency each
    u32x2_t rv[2][4];
    if (a.resid != nullptr) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int ab = 0; ab < 4; ++ab) {
          const int64_t n = nb + x * 32 + 8 * ab + 4 * lg;
          rv[x][ab] = (n < ncols) ? *reinterpret_cast<const u32x2_t*>(a.resid + m * ncols + n) : u32x2_t{0u, 0u};
        }
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int ab = 0; ab < 4; ++ab) {
        const int64_t n = nb + x * 32 + 8 * ab + 4 * lg;
        if (n >= ncols) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[x][mb][4 * ab + e];
        if (a.resid != nullptr) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t pr = rv[x][ab][e];
            v[2 * e] += __builtin_bit_cast(float, pr << 16);
            v[2 * e + 1] += __builtin_bit_cast(float, pr & 0xffff0000u);
          }
        }
        u32x2_t wv;
        wv[0] = pack_bf16x2(v[0], v[1]);
        wv[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2_t*>(a.y + m * ncols + n) = wv;
      }
  } else {  // EPI_QKV: scatter to [B, H, N, d]
    const int64_t ncols = a.part[part].ncols;
    const int64_t d = a.d;
    const uint32_t dsh = (d == 16) ? 4u : 6u;
    const uint32_t ns = (uint32_t)a.Nseq;
    const uint32_t b = (uint32_t)m / ns, t = (uint32_t)m - b * ns;
    const int64_t nheads = (part == 0) ? a.Hq : a.Hkv;
    // element offset of (b, head 0, t, 0); a head adds N*d
    uint16_t* dst_bt = a.qkv[part] + ((int64_t)b * nheads * ns + t) * d;
    const uint32_t head_stride = ns * (uint32_t)d;
    u32x2_t wv[2][4];
    qkv_rows<MB>(a, acc, mb, t, part, lg, wv);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int ab = 0; ab < 4; ++ab) {
        const int64_t n = nb + x * 32 + 8 * ab + 4 * lg;
        if (n >= ncols) continue;
        const int64_t head = n >> dsh, c0 = n & (d - 1);
        // non-temporal: the projections end by writing back every dirty L2
        // line, which this skips (SQAT-m layer QKV projection: 11.0 -> 9.4
        // us; staging through LDS for whole-line stores measured 10.8)
        __builtin_nontemporal_store(wv[x][ab], reinterpret_cast<u32x2_t*>(dst_bt + (uint32_t)head * head_stride + (uint32_t)c0));
      }
  }
}

// KFULL (K a multiple of the 64-wide chunk): every lane's DMA offset is fixed
// for the whole reduction and each chunk moves the descriptors' base instead.
// With per-chunk offsets in VGPRs that the register allocator then reuses for
// LDS read results, the compiler waits for the DMA just issued before those
// reads (it treats the DMA's offset operand like a load destination), and no
// chunk overlaps the next one's DMA.
template <int EPI, int S, bool GATHER, int MB, bool KFULL>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmArgs a) {
  static_assert(S >= 2 && S <= 4, "2 to 4 stages");
  using T = Tiling<MB>;
  constexpr int TM = T::TM;
  constexpr int kATiles = T::kATiles;
  constexpr int kStageBytes = T::kStageBytes;
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st2[S > 2 ? kStageBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st3[S > 3 ? kStageBytes : 16];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lg = lane >> 5, l32 = lane & 31;
  const int wm = wave & 1, wn = wave >> 1;

  // workgroup -> (row tile, column tile); W tile c (c = 0, 1) holds segment
  // 2*ct + c: (part, first column). SwiGLU: gate and up at column ct*64.
  const int mt = blockIdx.x / a.tiles_total;
  const int ct = blockIdx.x % a.tiles_total;
  const int64_t m0 = (int64_t)mt * TM;
  const ARows& A = a.A;
  const int64_t K = A.K;
  int sp0, sp1;          // part of W tile 0 / 1
  int64_t wc0, wc1;      // first column of W tile 0 / 1 within its part
  if (EPI == EPI_SWIGLU) {
    sp0 = 0;
    sp1 = 1;
    wc0 = wc1 = (int64_t)ct * 64;
  } else {
    auto seg = [&](int g, int& pt, int64_t& col) {
      pt = 0;
      while (pt < a.nparts - 1 && g >= a.segs[pt]) g -= a.segs[pt++];
      col = (int64_t)g * 64;  // past the part's width when g >= segs[pt]: all masked
    };
    seg(2 * ct, sp0, wc0);
    seg(2 * ct + 1, sp1, wc1);
  }

  // descriptors: A (whole operand; gathered offsets may go anywhere in O) and
  // the parts that feed the two W tiles
  const __amdgpu_buffer_rsrc_t ra = rsrc(A.p, A.M * A.K * 2);  // O has the size of O_flat
  const WPart wp0 = a.part[sp0];
  const WPart wp1 = a.part[sp1];
  const __amdgpu_buffer_rsrc_t rw0 = rsrc(wp0.w, K * wp0.ncols * 2);
  const __amdgpu_buffer_rsrc_t rw1 = rsrc(wp1.w, K * wp1.ncols * 2);

  // This wave DMAs parts (8 rows each) of A tile atile -- all four of tile
  // `wave` for MB = 2, parts 2*(wave/2) + 0, 1 of tile wave % 2 for MB = 1 --
  // and W tile `wave` (kh = wave / 2, c = wave % 2; 4 parts of 8 k-rows).
  // Per-lane row terms are fixed across the reduction and computed once here.
  const int r8 = lane >> 3, s = lane & 7;
  const uint32_t dshift = GATHER ? (uint32_t)__builtin_ctzll((unsigned long long)A.d) : 0u;
  constexpr int NQA = T::kAParts;
  const int atile = (MB == 2) ? wave : (wave & 1);
  const int aq0 = (MB == 2) ? 0 : 2 * (wave >> 1);
  uint32_t a_base[NQA], a_k[NQA];
  bool a_ok[NQA];
#pragma unroll
  for (int j = 0; j < NQA; ++j) {
    const int r = (aq0 + j) * 8 + r8;                 // row within the 32-row tile
    const int64_t m = m0 + atile * kTileRows + r;
    a_ok[j] = m < A.M;
    a_base[j] = a_ok[j] ? a_row_base<GATHER>(A, (uint32_t)m) : 0u;
    a_k[j] = 8u * (uint32_t)(s ^ swz_k(r));
  }
  const int wkh = wave >> 1, wc = wave & 1;
  const WPart wq = wc ? wp1 : wp0;
  const uint32_t wncols = (uint32_t)wq.ncols;
  uint32_t w_col[4], w_r[4];
  bool w_ok[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = q * 8 + r8;                         // k row within the 32-row tile
    const int64_t col = (wc ? wc1 : wc0) + 8 * (s ^ swz_v(r));
    w_ok[q] = col < wq.ncols;
    w_col[q] = (uint32_t)col;
    w_r[q] = (uint32_t)(wkh * kTileRows + r);
  }

  // KFULL: the lanes' offsets at k = 0 (rows past M, columns past the part's
  // width: kOOB)
  // (a_off0 has the largest NQA as its size: sized NQA, clang left the host
  // stub of the KFULL kernels undefined)
  uint32_t a_off0[4], w_off0[4];
#pragma unroll
  for (int j = 0; j < NQA; ++j) a_off0[j] = a_offset<GATHER>(A, a_base[j], a_ok[j], a_k[j], dshift);
#pragma unroll
  for (int q = 0; q < 4; ++q) w_off0[q] = w_ok[q] ? (w_r[q] * wncols + w_col[q]) * 2u : kOOB;
  const int64_t a_bytes = A.M * A.K * 2;
  const int64_t w_bytes = K * (int64_t)wncols * 2;
  const uint16_t* wbase = wc ? wp1.w : wp0.w;

  auto issue = [&](uint8_t* stage, int64_t k0) {
    if constexpr (KFULL) {
      // chunk k0: A from element adv on (row-major: k0; gathered: head
      // k0 / d, column k0 % d), W from row k0 on; the range checks count
      // from the moved bases, so chunks past K read nothing
      const int64_t adv = GATHER ? (((k0 >> dshift) * A.N) << dshift) + (k0 & ((1 << dshift) - 1)) : k0;
      const int64_t arem = a_bytes - adv * 2;
      const __amdgpu_buffer_rsrc_t rak = rsrc(A.p + adv, (k0 < K && arem > 0) ? arem : (int64_t)0);
      const int64_t wadv = k0 * (int64_t)wncols;
      const int64_t wrem = w_bytes - wadv * 2;
      const __amdgpu_buffer_rsrc_t rwk = rsrc(wbase + wadv, wrem > 0 ? wrem : (int64_t)0);
#pragma unroll
      for (int j = 0; j < NQA; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rak, (lds_void_t*)(stage + atile * kTileBytes + (aq0 + j) * 1024), 16,
                                                 a_off0[j], 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rwk, (lds_void_t*)(stage + (kATiles + wave) * kTileBytes + q * 1024),
                                                 16, w_off0[q], 0, 0, 0);
    } else {
      const uint32_t k32 = (uint32_t)k0;
#pragma unroll
      for (int j = 0; j < NQA; ++j) {
        const uint32_t off = a_offset<GATHER>(A, a_base[j], a_ok[j], k32 + a_k[j], dshift);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(stage + atile * kTileBytes + (aq0 + j) * 1024), 16,
                                                 off, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t k = k32 + w_r[q];
        const uint32_t off = (w_ok[q] && k < (uint32_t)K) ? (k * wncols + w_col[q]) * 2u : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wc ? rw1 : rw0,
                                                 (lds_void_t*)(stage + (kATiles + wave) * kTileBytes + q * 1024), 16,
                                                 off, 0, 0, 0);
      }
    }
  };

  // read offsets: A^T fragments (B operand) for k step (kh, hh): row l32,
  // logical chunk kh*4 + lg*2 + hh
  uint32_t boff[2][2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      boff[kh][hh] = (uint32_t)(l32 * kRowBytes + (((kh * 4 + lg * 2 + hh) ^ swz_k(l32)) * 16));
  const ReadOffsets ro = read_offsets(lane);
  // W tile and transposed-read offset feeding accumulator slot x of this
  // wave: SwiGLU -- gate (tile 0) and up (tile 1) at columns ct*64 + wn*32;
  // otherwise both 32-column halves of W tile wn
  const int wtile0 = (EPI == EPI_SWIGLU) ? 0 : wn;
  const int wtile1 = (EPI == EPI_SWIGLU) ? 1 : wn;
  const uint32_t toff0 = (EPI == EPI_SWIGLU) ? (wn ? ro.tr[1] : ro.tr[0]) : ro.tr[0];
  const uint32_t toff1 = (EPI == EPI_SWIGLU) ? (wn ? ro.tr[1] : ro.tr[0]) : ro.tr[1];

  f32x16_t acc[2][MB];  // [slot x][row block mb]
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[x][mb] = zero16();

  // One reduction chunk from stage CUR while chunk kc+S-1 streams into the
  // stage freed by chunk kc-1. The stages are separate LDS objects and the
  // loop is unrolled by S, so the compiler can tell the reads of one stage
  // from the DMA into another.
  auto chunk = [&](const uint8_t* cur, uint8_t* ahead, int kc) {
    // chunk kc landed (later ones may not have); every wave is done with
    // chunk kc-1, whose stage receives chunk kc+S-1
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((S - 2) * T::kDma));  // S-2 chunks may stay in flight
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(ahead, (int64_t)(kc + S - 1) * TK);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      u32x4_t wf[2][2];  // [slot][hh]
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const uint8_t* tile = cur + (kATiles + kh * 2 + (x ? wtile1 : wtile0)) * kTileBytes;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint8_t* p = tile + (x ? toff1 : toff0) + hh * 8 * kRowBytes;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * kRowBytes));
          const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
          wf[x][hh] = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
        }
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const uint8_t* at = cur + (wm * MB + mb) * kTileBytes;
          const u32x4_t af = *reinterpret_cast<const u32x4_t*>(at + boff[kh][hh]);
#pragma unroll
          for (int x = 0; x < 2; ++x) acc[x][mb] = mfma(wf[x][hh], af, acc[x][mb]);
        }
      }
    }
  };

  uint8_t* stg[4] = {st0, st1, st2, st3};
  const int nk = (int)((K + TK - 1) / TK);
#pragma unroll
  for (int j = 0; j < S - 1; ++j) issue(stg[j], (int64_t)j * TK);
  int kc = 0;
  for (; kc + S <= nk; kc += S) {
#pragma unroll
    for (int j = 0; j < S; ++j) chunk(stg[j], stg[(j + S - 1) % S], kc + j);
  }
#pragma unroll
  for (int j = 0; j < S - 1; ++j)
    if (kc + j < nk) chunk(stg[j], stg[(j + S - 1) % S], kc + j);
  // drain the zero-filling DMAs still in flight before the workgroup ends
  __builtin_amdgcn_s_waitcnt(0x0070);

  // ---------------- epilogues. Entry i of acc[x][mb] (lane l): row
  // m0 + wm*32*MB + mb*32 + l32; column (within the slot's 32) 8*(i/4) + 4*lg + i%4.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t m = m0 + wm * 32 * MB + mb * 32 + l32;
    if (m >= A.M) continue;
    if (EPI == EPI_SWIGLU) {
      const int64_t F = a.part[0].ncols;
#pragma unroll
      for (int ab = 0; ab < 4; ++ab) {
        const int64_t n = wc0 + wn * 32 + 8 * ab + 4 * lg;
        if (n >= F) continue;
        float h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = silu_mul(acc[0][mb][4 * ab + e], acc[1][mb][4 * ab + e]);
        u32x2_t wv;
        wv[0] = pack_bf16x2(h[0], h[1]);
        wv[1] = pack_bf16x2(h[2], h[3]);
        *reinterpret_cast<u32x2_t*>(a.y + m * F + n) = wv;
      }
    } else {
      const int part = (EPI == EPI_QKV) ? (wn ? sp1 : sp0) : 0;
      store_rows<EPI, MB>(a, acc, mb, m, part, wn ? wc1 : wc0, lg);
    }
  }
}

// Short reductions (K <= 256) over at most four 64-column segments with the
// store epilogue -- the SQAT-m output projection: a workgroup takes 64 rows
// and every segment, so A is read once, and holds the whole reduction in LDS
// (up to four 40 KB chunks), so every DMA is issued at the start and waited
// for once instead of chunk after chunk; one workgroup per CU. Wave w owns
// segment w: 64 rows (two 32-row blocks) x 64 columns (two 32-column slots).
// (The QKV projection ran slower this way, 11.2 against 10.2 us, and keeps
// the staged kernel.)
constexpr int kWideChunkBytes = 10 * kTileBytes;  // A [2][32 m][64 k], W [kh 2][seg 4][32 k][64 n]
constexpr int kWideMaxChunks = 4;

template <int EPI, bool GATHER>
__global__ __launch_bounds__(kThreads, 1) void gemm_wide_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWideMaxChunks * kWideChunkBytes];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lg = lane >> 5, l32 = lane & 31;
  const int64_t m0 = (int64_t)blockIdx.x * 64;
  const ARows& A = a.A;
  const int64_t K = A.K;
  const int nk = (int)((K + TK - 1) / TK);

  // segment `wave`: weight part and first column (past the part's width
  // when the parts have fewer than four segments: all masked)
  int part = 0;
  int64_t col0;
  {
    int g = wave;
    while (part < a.nparts - 1 && g >= a.segs[part]) g -= a.segs[part++];
    col0 = (int64_t)g * 64;
  }
  const WPart wp = a.part[part];
  const __amdgpu_buffer_rsrc_t ra = rsrc(A.p, A.M * A.K * 2);
  const __amdgpu_buffer_rsrc_t rw = rsrc(wp.w, K * wp.ncols * 2);

  // DMA lanes: A parts 2*(wave&1)+j (8 rows each) of A tile wave>>1, and the
  // four 8-row parts of W tiles (kh, segment wave), kh = 0, 1
  const int r8 = lane >> 3, s = lane & 7;
  const uint32_t dshift = GATHER ? (uint32_t)__builtin_ctzll((unsigned long long)A.d) : 0u;
  const int atile = wave >> 1;
  uint32_t a_base[2], a_k[2];
  bool a_ok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = (2 * (wave & 1) + j) * 8 + r8;
    const int64_t m = m0 + atile * kTileRows + r;
    a_ok[j] = m < A.M;
    a_base[j] = a_ok[j] ? a_row_base<GATHER>(A, (uint32_t)m) : 0u;
    a_k[j] = 8u * (uint32_t)(s ^ swz_k(r));
  }
  const uint32_t wncols = (uint32_t)wp.ncols;
  uint32_t w_col[4];
  bool w_ok[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = q * 8 + r8;
    const int64_t col = col0 + 8 * (s ^ swz_v(r));
    w_ok[q] = col < wp.ncols;
    w_col[q] = (uint32_t)col;
  }
  for (int kc = 0; kc < nk; ++kc) {
    uint8_t* stage = lds + kc * kWideChunkBytes;
    const uint32_t k32 = (uint32_t)(kc * TK);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t off = a_offset<GATHER>(A, a_base[j], a_ok[j], k32 + a_k[j], dshift);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(stage + atile * kTileBytes + (2 * (wave & 1) + j) * 1024),
                                               16, off, 0, 0, 0);
    }
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t k = k32 + (uint32_t)(kh * kTileRows + q * 8 + r8);
        const uint32_t off = (w_ok[q] && k < (uint32_t)K) ? (k * wncols + w_col[q]) * 2u : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rw, (lds_void_t*)(stage + (2 + kh * 4 + wave) * kTileBytes + q * 1024), 16, off, 0, 0, 0);
      }
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): every chunk landed
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  uint32_t boff[2][2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      boff[kh][hh] = (uint32_t)(l32 * kRowBytes + (((kh * 4 + lg * 2 + hh) ^ swz_k(l32)) * 16));
  const ReadOffsets ro = read_offsets(lane);
  f32x16_t acc[2][2];  // [slot x][row block mb]
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) acc[x][mb] = zero16();
  for (int kc = 0; kc < nk; ++kc) {
    const uint8_t* stage = lds + kc * kWideChunkBytes;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const uint8_t* wt = stage + (2 + kh * 4 + wave) * kTileBytes;
      u32x4_t wf[2][2];  // [slot][hh]
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint8_t* q = wt + ro.tr[x] + hh * 8 * kRowBytes;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)q);
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(q + 4 * kRowBytes));
          const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
          wf[x][hh] = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
        }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const u32x4_t af = *reinterpret_cast<const u32x4_t*>(stage + mb * kTileBytes + boff[kh][hh]);
#pragma unroll
          for (int x = 0; x < 2; ++x) acc[x][mb] = mfma(wf[x][hh], af, acc[x][mb]);
        }
    }
  }
  if constexpr (EPI == EPI_STORE) {
    // Coalesced store: every wave writes its 64 x 64 block to LDS as bf16
    // (rows of 128 B, 16-byte chunks XOR-swizzled by the row), then the
    // workgroup writes whole 512-byte rows of y, 16 bytes per lane, adding
    // the residual there, with non-temporal stores. SQAT-m output
    // projection: 7.3 us with 8-byte stores, one row per lane; 6.2 staged;
    // 5.7 staged and non-temporal (8-byte non-temporal stores: 14.4).
    const int64_t ncols = a.part[0].ncols;
    // the residual chunks of this thread's 8 row passes, loaded before the
    // staging so that their latency overlaps it (y may alias the residual:
    // each element is read before it is written)
    u32x4_t rvs[8];
    if (a.resid != nullptr) {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = it * 8 + (tid >> 5), cg = tid & 31;
        const int64_t m = m0 + r, n = (int64_t)cg * 8;
        rvs[it] = (m < A.M && n < ncols) ? *reinterpret_cast<const u32x4_t*>(a.resid + m * ncols + n)
                                         : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    __syncthreads();  // every wave is done reading the reduction chunks
    uint8_t* blk = lds + wave * 8192;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int ab = 0; ab < 4; ++ab) {
          const int r = mb * 32 + l32, c = x * 32 + 8 * ab + 4 * lg;  // 4 columns c..c+3
          u32x2_t wv;
          wv[0] = pack_bf16x2(acc[x][mb][4 * ab], acc[x][mb][4 * ab + 1]);
          wv[1] = pack_bf16x2(acc[x][mb][4 * ab + 2], acc[x][mb][4 * ab + 3]);
          *reinterpret_cast<u32x2_t*>(blk + r * 128 + (((c >> 3) ^ (r & 7)) << 4) + (c & 7) * 2) = wv;
        }
    __syncthreads();
    // 64 rows x (4 waves x 8 chunks): thread -> (row, chunk), 8 rows per
    // pass. All eight chunks are read and finished before the first store:
    // a register that still feeds a store in flight is rewritten only after
    // that store completes, so reads into one register per pass would
    // serialise the stores.
    u32x4_t vals[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = it * 8 + (tid >> 5), cg = tid & 31;  // cg: 16-byte chunk of the 256-column row
      const int w = cg >> 3, ch = cg & 7;
      vals[it] = *reinterpret_cast<const u32x4_t*>(lds + w * 8192 + r * 128 + ((ch ^ (r & 7)) << 4));
      if (a.resid != nullptr) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t v = vals[it][e], rv = rvs[it][e];
          const float lo = __builtin_bit_cast(float, v << 16) + __builtin_bit_cast(float, rv << 16);
          const float hi = __builtin_bit_cast(float, v & 0xffff0000u) + __builtin_bit_cast(float, rv & 0xffff0000u);
          vals[it][e] = pack_bf16x2(lo, hi);
        }
      }
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = it * 8 + (tid >> 5), cg = tid & 31;
      const int64_t m = m0 + r, n = (int64_t)cg * 8;
      if (m < A.M && n < ncols)
        __builtin_nontemporal_store(vals[it], reinterpret_cast<u32x4_t*>(a.y + m * ncols + n));
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int64_t m = m0 + mb * 32 + l32;
      if (m < A.M) store_rows<EPI, 2>(a, acc, mb, m, part, col0, lg);
    }
  }
}

template <int EPI, int S, bool GATHER, int MB, bool KFULL>
hipError_t launch_kernel(const GemmArgs& a, int64_t nblk, hipStream_t stream) {
  gemm_kernel<EPI, S, GATHER, MB, KFULL><<<dim3((unsigned)nblk), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

template <int EPI, int S, bool GATHER, int MB>
hipError_t launch_grid(const GemmArgs& a, hipStream_t stream, bool dry_run) {
  const int64_t mtiles = (a.A.M + Tiling<MB>::TM - 1) / Tiling<MB>::TM;
  const int64_t nblk = mtiles * a.tiles_total;
  if (nblk > 0x7fffffff || nblk <= 0) return hipErrorInvalidValue;
  if (dry_run) return hipSuccess;
  return a.A.K % TK == 0 ? launch_kernel<EPI, S, GATHER, MB, true>(a, nblk, stream)
                         : launch_kernel<EPI, S, GATHER, MB, false>(a, nblk, stream);
}

// Grids of at most 384 workgroups of 128 rows (about one per CU; the SQAT-m
// QKV, output and down projections) run 64-row workgroups with three stages
// instead: twice the workgroups, two per CU (72 KB of LDS each), two chunks
// in flight. Measured on the SQAT-m block (B16 N1024): QKV 11.3 -> 8.9 us,
// output projection 11.2 -> 10.0, down 17.2 -> 15.7 (128-row workgroups with
// four stages before; 64-row with two or four stages were slower). Larger
// grids (the gate/up projection) keep 128 rows and two stages.
template <int EPI, bool GATHER>
hipError_t launch_stages(const GemmArgs& a, hipStream_t stream, bool dry_run) {
  const int64_t nblk128 = ((a.A.M + 127) / 128) * a.tiles_total;
  if (nblk128 <= 384) return launch_grid<EPI, 3, GATHER, 1>(a, stream, dry_run);
  return launch_grid<EPI, 2, GATHER, 2>(a, stream, dry_run);
}

template <int EPI, bool GATHER>
hipError_t launch_wide(const GemmArgs& a, hipStream_t stream, bool dry_run) {
  const int64_t nblk = (a.A.M + 63) / 64;
  if (nblk > 0x7fffffff || nblk <= 0) return hipErrorInvalidValue;
  if (dry_run) return hipSuccess;
  hipLaunchKernelGGL((gemm_wide_kernel<EPI, GATHER>), dim3((unsigned)nblk), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch(const GemmArgs& a, int epi, hipStream_t stream, bool dry_run) {
  if (a.tiles_total <= 0 || a.A.M <= 0) return hipErrorInvalidValue;
  // short reductions over at most four segments, store epilogue: the wide
  // kernel (SQAT-m output projection, B16 N1024 D256: 7.3 -> 5.7 us)
  if (epi == EPI_STORE && a.A.K <= (int64_t)kWideMaxChunks * TK && a.segs_total <= 4)
    return a.A.gather ? launch_wide<EPI_STORE, true>(a, stream, dry_run) : launch_wide<EPI_STORE, false>(a, stream, dry_run);
  if (epi == EPI_STORE)
    return a.A.gather ? launch_stages<EPI_STORE, true>(a, stream, dry_run)
                      : launch_stages<EPI_STORE, false>(a, stream, dry_run);
  if (epi == EPI_SWIGLU) return launch_stages<EPI_SWIGLU, false>(a, stream, dry_run);
  return launch_stages<EPI_QKV, false>(a, stream, dry_run);
}

GemmArgs base_args() {
  GemmArgs a{};
  a.A.gather = 0;
  a.A.N = 1;
  a.A.Hq = 1;
  a.A.d = 1;
  return a;
}

// 32-bit DMA offsets: every byte a lane may address must fit in 2^31.
bool fits(int64_t bytes) { return bytes > 0 && bytes < 0x7fffffffLL; }

}  // namespace

hipError_t launch_qkv_rope(const QkvProblem& p, hipStream_t stream) {
  if (p.d != 16 && p.d != 64) return hipErrorInvalidValue;
  if (p.Dm % 8 != 0) return hipErrorInvalidValue;
  GemmArgs a = base_args();
  a.A.p = static_cast<const uint16_t*>(p.x);
  a.A.M = p.B * p.N;
  a.A.K = p.Dm;
  if (!fits(a.A.M * a.A.K * 2)) return hipErrorInvalidValue;
  const void* w[3] = {p.wq, p.wk, p.wv};
  const int64_t nc[3] = {p.Hq * p.d, p.Hkv * p.d, p.Hkv * p.d};
  // 32-bit offsets: weights, and the heads of one sequence in the scatter
  if (!fits(p.Dm * nc[0] * 2) || !fits(p.Dm * nc[1] * 2) || !fits(p.Hq * p.N * p.d * 2)) return hipErrorInvalidValue;
  a.nparts = 3;
  a.segs_total = 0;
  for (int i = 0; i < 3; ++i) {
    a.part[i].w = static_cast<const uint16_t*>(w[i]);
    a.part[i].ncols = nc[i];
    a.segs[i] = (int)((nc[i] + 63) / 64);
    a.segs_total += a.segs[i];
  }
  a.tiles_total = (a.segs_total + 1) / 2;
  a.epi = EPI_QKV;
  a.qkv[0] = static_cast<uint16_t*>(p.q);
  a.qkv[1] = static_cast<uint16_t*>(p.k);
  a.qkv[2] = static_cast<uint16_t*>(p.v);
  for (int c = 0; c < 32; ++c)
    a.rope_theta[c] =
        (c < p.d / 2) ? pow((double)p.rope_base, -2.0 * c / (double)p.d) / 6.283185307179586476925286766559 : 0.0;
  a.Nseq = p.N;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.d = p.d;
  return launch(a, EPI_QKV, stream, p.dry_run);
}

hipError_t launch_out_proj(const OprojProblem& p, hipStream_t stream) {
  if (p.d < 8 || (p.d & (p.d - 1)) != 0 || p.Dm % 8 != 0) return hipErrorInvalidValue;  // d a power of two
  GemmArgs a = base_args();
  a.A.p = static_cast<const uint16_t*>(p.o);
  a.A.M = p.B * p.N;
  a.A.K = p.Hq * p.d;
  a.A.gather = 1;
  a.A.N = p.N;
  a.A.Hq = p.Hq;
  a.A.d = p.d;
  if (!fits(a.A.M * a.A.K * 2) || !fits(a.A.K * p.Dm * 2) || !fits(a.A.M * p.Dm * 2)) return hipErrorInvalidValue;
  a.nparts = 1;
  a.part[0].w = static_cast<const uint16_t*>(p.wo);
  a.part[0].ncols = p.Dm;
  a.segs[0] = (int)((p.Dm + 63) / 64);
  a.segs_total = a.segs[0];
  a.tiles_total = (a.segs_total + 1) / 2;
  a.epi = EPI_STORE;
  a.resid = static_cast<const uint16_t*>(p.resid);
  a.y = static_cast<uint16_t*>(p.y);
  return launch(a, EPI_STORE, stream, p.dry_run);
}

hipError_t launch_dense_residual(const DenseProblem& p, hipStream_t stream) {
  if (p.K % 8 != 0 || p.Ncols % 8 != 0) return hipErrorInvalidValue;
  GemmArgs a = base_args();
  a.A.p = static_cast<const uint16_t*>(p.a);
  a.A.M = p.M;
  a.A.K = p.K;
  if (!fits(a.A.M * a.A.K * 2) || !fits(p.K * p.Ncols * 2) || !fits(p.M * p.Ncols * 2)) return hipErrorInvalidValue;
  a.nparts = 1;
  a.part[0].w = static_cast<const uint16_t*>(p.w);
  a.part[0].ncols = p.Ncols;
  a.segs[0] = (int)((p.Ncols + 63) / 64);
  a.segs_total = a.segs[0];
  a.tiles_total = (a.segs_total + 1) / 2;
  a.epi = EPI_STORE;
  a.resid = static_cast<const uint16_t*>(p.resid);
  a.y = static_cast<uint16_t*>(p.y);
  return launch(a, EPI_STORE, stream, p.dry_run);
}

hipError_t launch_gate_up(const GateUpProblem& p, hipStream_t stream) {
  if (p.K % 8 != 0 || p.F % 8 != 0) return hipErrorInvalidValue;
  GemmArgs a = base_args();
  a.A.p = static_cast<const uint16_t*>(p.z);
  a.A.M = p.M;
  a.A.K = p.K;
  if (!fits(a.A.M * a.A.K * 2) || !fits(p.K * p.F * 2) || !fits(p.M * p.F * 2)) return hipErrorInvalidValue;
  a.nparts = 2;
  a.part[0].w = static_cast<const uint16_t*>(p.w_gate);
  a.part[0].ncols = p.F;
  a.part[1].w = static_cast<const uint16_t*>(p.w_up);
  a.part[1].ncols = p.F;
  a.segs[0] = a.segs[1] = (int)((p.F + 63) / 64);
  a.segs_total = a.segs[0];
  a.tiles_total = a.segs[0];
  a.epi = EPI_SWIGLU;
  a.y = static_cast<uint16_t*>(p.h);
  return launch(a, EPI_SWIGLU, stream, p.dry_run);
}

}  // namespace sqa
