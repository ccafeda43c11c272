// Device-side building blocks for the gfx950 attention kernels: vector types,
// MFMA wrappers with their lane layouts, the LDS swizzle, the LDS transpose
// read, cross-half reductions and the two exp2 variants.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "exp2_poly_coeffs.h"

namespace fattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

#define FATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// MFMA 32x32x16 bf16 (gfx950).  With h = lane/32 and c = lane%32:
//   A (32×16): lane holds A[c][8h + e], e = 0..7
//   B (16×32): lane holds B[8h + e][c]
//   C (32×32): lane holds C[8(r/4) + 4h + r%4][c], r = 0..15
// Any simultaneous relabelling of the k index in A and B leaves the product
// unchanged; the kernels use that freedom to keep P in registers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp8 (e4m3fn for both operands) 32x32x64: A lane holds 32 k values of row c,
// B lane holds 32 k values of column c; the k split between the lane halves
// is the same for A and B, C as for mfma32.
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // format 0 = e4m3 for A (cbsz) and B (blgp); block scales 127 = 2^0.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Same product with the B operand scaled by 2^-4 (E8M0 block scale 123).
__device__ __forceinline__ f32x16 mfma32_fp8_bscale(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 123);
}

// Row index of accumulator register r in lane-half h (column = lane%32).
__device__ __forceinline__ constexpr int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// ---------------------------------------------------------------------------
// LDS tile layout for [rows][D] bf16 tiles: 16-byte chunks are XOR-swizzled
// per row so that the 32-row × 16-byte MFMA operand reads and the 8-row
// transpose reads spread over all banks.
// ---------------------------------------------------------------------------
// Rows of RB bytes (RB = 64, 128 or 256); the LDS has 64 four-byte banks, so a
// 256-byte window holds one row of 256 B, two of 128 B or four of 64 B. The
// 16-byte chunk index is XORed with a bijection of the row so that
//  * 16 consecutive rows read at the same chunk (the 16 lanes of a 16-byte
//    MFMA operand read) land on 16 different 16-byte bank groups, and
//  * 4 consecutive rows read over 4 consecutive chunks (a 16-lane group of the
//    8-byte transpose read) cover 4 disjoint bank groups.
template <int RB>
__device__ __forceinline__ int swz_chunk_rb(int row, int chunk) {
  if constexpr (RB == 256) {
    return chunk ^ (((row & 3) << 2) | ((row >> 2) & 3));
  } else if constexpr (RB == 128) {
    return chunk ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  } else {
    return chunk ^ ((row >> 2) & 3);
  }
}
// Byte offset of (row, 16-byte chunk) in a tile with RB-byte rows.
template <int RB>
__device__ __forceinline__ int tile_off_rb(int row, int chunk) {
  return row * RB + swz_chunk_rb<RB>(row, chunk) * 16;
}
// Byte offset of (row, 16-byte chunk) in a [rows][D] bf16 tile.
template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return tile_off_rb<D * 2>(row, chunk);
}

// ds_read_b64_tr_b16 on gfx950: within each 16-lane group g, output lane i
// receives, for e = 0..3, element i%4 of the 8-byte row addressed by lane
// 16g + 4e + i/4.
__device__ __forceinline__ bf16x4 lds_read_tr16(const char* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 FATTN_LDS*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// Buffer descriptor in scalar registers for the inline-assembly loads below:
// base address, stride 0, `bytes` records (loads at byte offsets ≥ bytes
// return zero), raw 32-bit data format.
__device__ __forceinline__ i32x4 make_rsrc_sgpr(const void* base, int bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000;
  return r;
}

// LDS byte address of a generic pointer into LDS. A generic address in the
// shared aperture carries the LDS address in its low 32 bits, so truncation
// is the cast (without the null test of an address-space cast, which would
// keep the 64-bit pointer alive in vector registers).
__device__ __forceinline__ int lds_addr(const char* p) { return (int)(uint32_t)(uintptr_t)p; }

// Moves LOADS × 1 KB of a tile into LDS with buffer loads: wave load i takes
// 16 bytes per lane from byte offset off[i] of the buffer [base, base + bytes)
// (zero past the end) to LDS at dst + (first + i)·1 KB + lane·16.
// The loads are issued by inline assembly, so the compiler does not track
// them: it would otherwise make every later LDS read wait for all of them
// (it cannot tell which LDS bytes they write). The caller orders them with
// wait_vmem() and a workgroup barrier before the data is read, and before
// the LDS range is written again.
// Each load sets m0 (the LDS destination) itself. The compiler treats m0 as
// a reserved register and does not honour it as a clobber; this is sound
// because none of the kernels' compiled code reads or writes m0 outside
// these asm statements (checked on the gfx950 assembly of every kernel), so
// no compiler value lives in m0 across them.
template <int LOADS>
__device__ __forceinline__ void buffer_to_lds(const void* base, int bytes, char* dst,
                                              const int (&off)[LOADS], int first) {
#if defined(__HIP_DEVICE_COMPILE__)
  const i32x4 rsrc = make_rsrc_sgpr(base, bytes);
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int m0v = __builtin_amdgcn_readfirstlane(lds_addr(dst + (first + i) * 1024));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0v), "v"(off[i]), "s"(rsrc)
                 : "memory", "m0");
  }
#endif
}

// 64 floats from `src` into LDS at `dst` (one 4-byte element per lane), by
// the same untracked load as buffer_to_lds.
__device__ __forceinline__ void stats_to_lds(const float* src, char* dst, int lane,
                                             int bytes = 256) {
#if defined(__HIP_DEVICE_COMPILE__)
  const i32x4 rsrc = make_rsrc_sgpr(src, bytes);
  const int m0v = __builtin_amdgcn_readfirstlane(lds_addr(dst));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(m0v), "v"(lane * 4), "s"(rsrc)
               : "memory", "m0");
#endif
}

// Block masks (block-sparse attention): one bit per 128-row mask block,
// kMaskWords 64-bit ballots per row or column of the mask (N <= 32768).
constexpr int kMaskBlockRows = 128;
constexpr int kMaskWords = 4;

// Bits of the mask blocks base[b * stride] for b < nb (a mask row: stride
// 1; a mask column: stride nb), identical in every lane.
__device__ __forceinline__ void load_mask_bits(const uint8_t* base, long stride, int nb, int lane,
                                               uint64_t (&mb)[kMaskWords]) {
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) {
    const int b = w * 64 + lane;
    mb[w] = __ballot(b < nb && base[b * stride] != 0);
  }
}

// First 64-row tile index >= j whose mask block (tile / 2) is set, or n if
// there is none below n.
__device__ __forceinline__ int next_mask_tile(const uint64_t (&mb)[kMaskWords], int j, int n) {
  if (j >= n) return n;
  const int b = j >> 1;
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) {
    if (w < (b >> 6)) continue;
    uint64_t bits = mb[w];
    if (w == (b >> 6)) bits &= ~0ull << (b & 63);
    if (bits != 0) {
      const int nbk = w * 64 + __builtin_ctzll(bits);
      return min(nbk == b ? j : 2 * nbk, n);
    }
  }
  return n;
}

// Number of tiles in [j0, n) whose mask block is set.
__device__ __forceinline__ int count_mask_tiles(const uint64_t (&mb)[kMaskWords], int j0, int n) {
  int cnt = 0;
  for (int j = next_mask_tile(mb, j0, n); j < n; j = next_mask_tile(mb, j + 1, n)) ++cnt;
  return cnt;
}

// Packed segments (rows [cu[s], cu[s+1]) clamped to [0, N]) ranked by
// decreasing length, ties by index: the segment of rank r (r < nseq), the
// same in every lane. Lane i ranks segment i by counting the longer ones;
// with more than 64 segments the order is left as it is (segment r).
__device__ __forceinline__ int segment_of_rank(const int* cu, int nseq, int N, int r, int lane) {
  if (nseq > 64) return r;
  int len = -1;
  if (lane < nseq) {
    const int a = min(max(cu[lane], 0), N);
    len = min(max(cu[lane + 1], a), N) - a;
  }
  int rank = 0;
  for (int j = 0; j < nseq; ++j) {
    const int lj = __builtin_amdgcn_readlane(len, j);
    rank += (lj > len || (lj == len && j < lane)) ? 1 : 0;
  }
  const uint64_t hit = __ballot(lane < nseq && rank == r);
  return hit ? (int)__builtin_ctzll(hit) : r;
}

// Wait until this wave's outstanding global loads (including those that
// write straight into LDS) have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ bf16x8 concat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Value of lane l combined with lane l^32 (both halves get the result).
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// exp2 variants (FlashAttention-4 gist, technical summary 2.B: 2^x computed
// either by the special-function unit or by a polynomial on FMA units).
// ---------------------------------------------------------------------------
enum { EXP_HW = 1, EXP_POLY = 2, EXP_SPLIT = 3 };

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^x = 2^n · 2^f with n = floor(x), f = x − n ∈ [0, 1); 2^f by a degree-3
// polynomial (own minimax fit, coefficients in exp2_poly_coeffs.h), 2^n
// applied with ldexp. x is clamped at −200 so that −∞ gives exactly 0.
__device__ __forceinline__ float exp2_poly(float x) {
  x = fmaxf(x, -200.0f);
  float n = __builtin_floorf(x);
  float f = x - n;
  float p = fmaf(fmaf(fmaf(kExp2PolyC3, f, kExp2PolyC2), f, kExp2PolyC1), f, kExp2PolyC0);
  return __builtin_amdgcn_ldexpf(p, (int)n);
}

template <int MODE>
__device__ __forceinline__ float exp2_sel(float x) {
  if constexpr (MODE == EXP_POLY) return exp2_poly(x);
  else return exp2_hw(x);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace fattn
