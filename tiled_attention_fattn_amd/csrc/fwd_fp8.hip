// fp8 (OCP e4m3fn) attention forward with incoherent processing, for gfx950.
//
// FlashAttention-3 page, innovation 3: Q and K are multiplied by a random
// orthogonal (Hadamard) matrix before fp8 quantisation, which spreads outlier
// coordinates and cannot change Q·Kᵀ. Here R = diag(s)·H_d/√d with s from
// SplitMix64 (Steele, Lea & Flood 2014) and H_d the Sylvester Hadamard matrix,
// applied row by row with a fast Walsh–Hadamard transform in registers.
//
// Scales: K' and V one per chunk of 128 keys of each (b,h) (K' the exact
// ratio x·448/amax of its chunk, V a power of two that the fp8 MFMA's block
// scale operand applies); Q' one per row (the row's own amax), which lets
// the attention kernel quantise the query rows it owns itself, so Q never
// makes a round trip through memory in e4m3.
//
// Launches (one stream):
//   1. fp8_prep   — one pass over K and V: each block holds one 128-key chunk
//                   of K·R (rotated in registers) or of V, takes its amax and
//                   quantises it: K8 = e4m3(x·448/amax) (one correctly
//                   rounded division, round to nearest even), V8 = e4m3(v·2^−e)
//                   written transposed ([d][keys]) in the key order the
//                   attention kernel's P operand uses; one (K, V) scale pair
//                   per chunk.
//   2. fwd_fp8    — attention. Prologue: each lane rotates its half of one
//                   bf16 Q row (the Walsh–Hadamard stages across the two
//                   lanes of the row by a lane-half swap), takes the row's
//                   amax and quantises it to Q8 and the residual term
//                   Q8lo = e4m3(16·(t − decode(Q8))). Loop: Sᵀ =
//                   K8·(Q8 + Q8lo/16)ᵀ (two MFMAs, the second with the
//                   block scale 2^-4) and Oᵀ += V8ᵀ·P8ᵀ on the
//                   32x32x64 f8f6f4 MFMA; P̃ = 2^(s·c − m) quantised to
//                   e4m3 as P̃·2^(8−τ−k) with τ = 1 and k ≥ 0 a per-row
//                   integer that rises when a tile max exceeds m + k + τ,
//                   so every stored value is at most 256 < 448; the PV and
//                   row-sum MFMAs take 2^k back as the P operand's block
//                   scale, so the offset m of O and l stays put and O needs
//                   no rescale (FlashAttention-4 gist, technical summary
//                   2.B: rescale only past a threshold; here the threshold
//                   is k = 32, past which m moves to the row max and O is
//                   rescaled); a tile's K scale joins the score factor, its
//                   V scale the PV MFMA's A block scale; O = Oᵀ/l with l the
//                   sum of the quantised P̃ (formed by one more MFMA); the
//                   optional LSE uses the fp32 sum before quantisation.
//
// Variants of the same launches: a block mask over 128×128 blocks (the
// attention kernel walks only the visible key tiles; the quantisation is
// unchanged), and packed variable-length sequences (each segment a sequence
// of its own: the preparation runs over (segment, chunk), chunks counted
// from the segment's first row; the attention kernel over (head, segment,
// query tile)).
#include <algorithm>
#include <type_traits>

#include "fattn_device.hpp"
#include "fattn_launch.h"

namespace fattn {

constexpr float kE4m3Max = 448.0f;
// Threshold of the fp8 softmax (log2 units) and the matching exponent of the
// fixed P scale: P̃·2^−k ≤ 2^τ, stored as P̃·2^(8−τ−k).
constexpr float kF8Tau = 1.0f;
constexpr float kF8PExp = 8.0f - kF8Tau;
// Largest per-row exponent k of the P operand's block scale before the
// accumulators are rescaled instead: O and l then hold at most 2^(8+k)·N
// times the largest |V| (V below 2^72 stays finite up to N = 2^15).
constexpr float kF8KMax = 32.0f;

// SplitMix64: state advanced by the golden-ratio increment, then mixed.
__device__ __forceinline__ float rotation_sign(uint64_t seed, int i) {
  uint64_t z = seed + (uint64_t)(i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z = z ^ (z >> 31);
  return (z >> 63) ? -1.0f : 1.0f;
}

// Packed variable-length sequences: rows [cu[s], cu[s+1]) of every head
// form segment s, a sequence of its own with its own K'/V scales. Without
// segments (cu = nullptr) the whole head is segment 0 (nseq = 1). Offsets are
// clamped to [0, N] and lengths to max_len, so no contents of cu address
// outside the tensors. A segment's V8ᵀ columns start at the 64-aligned
// column roundup64(row0) + 64·s, which leaves every segment its own whole
// 64-key blocks inside [0, roundup64(N) + 64·nseq).
struct Fp8Segs {
  const int* cu = nullptr;
  int nseq = 1;
  int max_len = 0;  // N without segments
};
__device__ __forceinline__ void seg_rows(const Fp8Segs& sg, int N, int s, int& row0, int& L) {
  if (sg.cu == nullptr) {
    row0 = 0;
    L = N;
    return;
  }
  row0 = min(max(sg.cu[s], 0), N);
  L = min(min(max(sg.cu[s + 1], row0), N) - row0, sg.max_len);
}
__device__ __forceinline__ int seg_vcol(const Fp8Segs& sg, int s, int row0) {
  return sg.cu == nullptr ? 0 : ((row0 + 63) & ~63) + 64 * s;
}

// Row-wise work of the prep kernels: a row of D elements is held by
// kLpr = D/32 consecutive lanes (a quad for D = 128), kEpl = 32 consecutive
// elements each (element index = lane_in_row·32 + e).
constexpr int kEpl = 32;

// x ↦ the value of the lane whose index differs in bit 0 (dpp = 0xB1) or
// bit 1 (dpp = 0x4E) within each quad (DPP quad_perm; no LDS traffic).
template <int DPP>
__device__ __forceinline__ float quad_xor(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), DPP, 0xF, 0xF, false));
}

// Unnormalised Walsh–Hadamard transform (Sylvester order) of one row: five
// butterfly stages inside each lane's 32 elements, then one stage per lane
// bit across the quad. In every butterfly the lower index takes a + b and
// the upper a − b.
template <int LPR>
__device__ __forceinline__ void fwht_row(float (&x)[kEpl], int lane_in_row) {
#pragma unroll
  for (int w = 1; w < kEpl; w <<= 1)
#pragma unroll
    for (int e = 0; e < kEpl; ++e)
      if (!(e & w)) {
        const float a = x[e], b = x[e + w];
        x[e] = a + b;
        x[e + w] = a - b;
      }
  if constexpr (LPR >= 2) {
    const bool upper = lane_in_row & 1;
#pragma unroll
    for (int e = 0; e < kEpl; ++e) {
      const float y = quad_xor<0xB1>(x[e]);
      x[e] = upper ? (y - x[e]) : (x[e] + y);
    }
  }
  if constexpr (LPR >= 4) {
    const bool upper = lane_in_row & 2;
#pragma unroll
    for (int e = 0; e < kEpl; ++e) {
      const float y = quad_xor<0x4E>(x[e]);
      x[e] = upper ? (y - x[e]) : (x[e] + y);
    }
  }
}

// Loads the 32 values of (row, part), rotated when `rot` (signs and the
// Walsh–Hadamard butterflies, without the 1/√d: the quantisation below is
// scale-invariant, so the factor joins the row's or chunk's scale instead);
// false if row >= N.
// Every lane of a row must call it (the rotation exchanges values).
template <int D>
__device__ __forceinline__ bool load_row_part(const bf16* src, int row, int N, int part, bool rot,
                                              const float* sgn, float (&x)[kEpl]) {
  constexpr int LPR = D / kEpl;
  const bool ok = row < N;
#pragma unroll
  for (int c = 0; c < kEpl / 8; ++c) {
    bf16x8 v = {};
    if (ok) v = *(const bf16x8*)(src + (size_t)row * D + part * kEpl + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[c * 8 + e] = (float)v[e];
  }
  if (rot) {
#pragma unroll
    for (int e = 0; e < kEpl; ++e) x[e] *= sgn[part * kEpl + e];
    fwht_row<LPR>(x, part);
  }
  return ok;
}

__device__ __forceinline__ float scale_from_amax(float a) { return a > 0.0f ? a / kE4m3Max : 1.0f; }

// E8M0 code of a positive normal power of two: its biased exponent.
__device__ __forceinline__ int e8m0_of(float pow2) { return (int)(__float_as_uint(pow2) >> 23); }

// The fp8 product with the A operand scaled by 2^(ea − 127) and the B operand
// by 2^(eb − 127) (E8M0 block scales; each lane's scale covers the 32 k
// values it holds).
__device__ __forceinline__ f32x16 mfma32_fp8_scaled(i32x8 a, i32x8 b, f32x16 c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

// Four e4m3 codes (round to nearest even), a in the lowest byte.
__device__ __forceinline__ int cvt_fp8x4(float a, float b, float c, float d) {
  // The first conversion writes the low half of a word whose high half the
  // second overwrites: starting from a's own bits lets the result take a's
  // register instead of a zeroed copy (one move fewer per four codes).
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}
// 1/√d of the rotation R = diag(s)·H_d/√d, applied to the scales.
template <int D>
constexpr float kInvSqrtD = D == 128 ? 0.08838834764831845f : 0.125f;

// Decode the four e4m3 codes of a packed word (lowest byte first).
__device__ __forceinline__ void dec_fp8x4(int w, float* out) {
  out[0] = __builtin_amdgcn_cvt_f32_fp8(w, 0);
  out[1] = __builtin_amdgcn_cvt_f32_fp8(w, 1);
  out[2] = __builtin_amdgcn_cvt_f32_fp8(w, 2);
  out[3] = __builtin_amdgcn_cvt_f32_fp8(w, 3);
}

// x·448/amax with one correctly rounded division (x·448 is exact for x of at
// most 21 significant bits, bf16 values among them), so exact e4m3
// midpoints stay exact.
//
// The quotient is formed by multiplying with the correctly rounded reciprocal
// of amax and one FMA correction from the exact remainder (Markstein's
// division step), which yields the correctly rounded fp32 quotient for
// normal operands at a quarter of the cost of a general division. An amax
// below 2^-100 (whose reciprocal could overflow) is scaled by 2^64 first,
// with x·448 alike, which is exact. Since |x| ≤ amax, the quotient never
// exceeds 448, so no e4m3 code saturates; amax = 0 (all x zero) gives 0.
struct Ratio448 {
  float am, inv, mul;
  __device__ explicit Ratio448(float a) {
    const bool tiny = a < 0x1p-100f;
    am = tiny ? a * 0x1p64f : a;
    mul = tiny ? kE4m3Max * 0x1p64f : kE4m3Max;
    inv = am > 0.0f ? __frcp_rn(am) : 0.0f;
  }
};
__device__ __forceinline__ float ratio448(float x, const Ratio448& r) {
  const float a = x * r.mul;
  const float q0 = a * r.inv;
  const float e = fmaf(-q0, r.am, a);    // exact remainder a − q0·amax
  return fmaf(e, r.inv, q0);
}

// Position of key r (0..63) inside its 64-key block of V8ᵀ.
__device__ __forceinline__ int v8_pos(int r) {
  const int s = 16 * (r >> 5) + 4 * ((r & 31) >> 3) + (r & 3);
  return 32 * ((r >> 2) & 1) + s;
}

// One pass of the preparation: grid (segments × 128-key chunks, BH, 2).
// blockIdx.z = 0: the chunk's K rows, rotated (Walsh–Hadamard in registers),
// take the chunk's amax and are quantised with the exact ratio
// x·448/amax; = 1: the chunk's V rows take a power-of-two scale 2^e (e the
// least with amax ≤ 448·2^e) and are quantised as e4m3(v·2^−e), an exact
// scaling, into V8ᵀ ([d][keys], the P-operand key order of v8_pos). Each
// thread holds its share of the chunk in registers between the two steps,
// so K and V are read once. scales: [BH·nseq][nchunks][2] (K, V) fp32.
// Keys past the segment's end give code 0; 64-key blocks past it are not
// written.
template <int D>
__global__ __launch_bounds__(256) void fp8_prep_kernel(const bf16* __restrict__ K,
                                                      const bf16* __restrict__ V,
                                                      uint8_t* __restrict__ k8,
                                                      uint8_t* __restrict__ v8t,
                                                      float* __restrict__ scales, int N,
                                                      int Npad, int rotate, uint64_t seed,
                                                      Fp8Segs sg, int nchunks) {
  constexpr int LPR = D / kEpl, RPB = 256 / LPR;   // K: lanes per row, rows per pass
  constexpr int KPASS = kFp8AmaxRows / RPB;        // K: passes over the chunk's rows
  constexpr int CHUNKS = D / 8;                    // V: 16-byte d-chunks per key row
  constexpr int VITEMS = 2 * 16 * CHUNKS;          // V: (sub-block, key quad, d-chunk) items
  constexpr int VPT = (VITEMS + 255) / 256;        // V: items per thread
  static_assert(kFp8AmaxRows == 128, "two 64-key V blocks per chunk");
  __shared__ float sgn[D];
  __shared__ float wmax[4];
  const int bh = blockIdx.y;
  const int seg = (int)blockIdx.x / nchunks, chunk = (int)blockIdx.x - seg * nchunks;
  int row0, L;
  seg_rows(sg, N, seg, row0, L);
  const int c0 = chunk * kFp8AmaxRows;  // first key of the chunk within the segment
  if (c0 >= L) return;                  // whole block
  const int unit = bh * sg.nseq + seg;
  float* sc = scales + ((size_t)unit * nchunks + chunk) * 2;
  const int c_end = min(L, c0 + kFp8AmaxRows);
  auto block_max = [&](float m) __device__ {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    return fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  };

  if (blockIdx.z == 0) {
    if (threadIdx.x < D) sgn[threadIdx.x] = rotation_sign(seed, threadIdx.x);
    __syncthreads();
    const size_t head = ((size_t)bh * N + row0) * D;
    const int part = threadIdx.x % LPR;
    float xs[KPASS][kEpl];
    bool ok[KPASS];
    float m = 0.0f;
#pragma unroll
    for (int u = 0; u < KPASS; ++u) {
      ok[u] = load_row_part<D>(K + head, c0 + u * RPB + threadIdx.x / LPR, c_end, part,
                               rotate != 0, sgn, xs[u]);
#pragma unroll
      for (int e = 0; e < kEpl; ++e) m = fmaxf(m, fabsf(xs[u][e]));
    }
    const float am = block_max(m);
    const Ratio448 rk(am);
    if (threadIdx.x == 0) sc[0] = scale_from_amax(rotate ? am * kInvSqrtD<D> : am);
#pragma unroll
    for (int u = 0; u < KPASS; ++u) {
      if (!ok[u]) continue;
      const size_t off = head + (size_t)(c0 + u * RPB + threadIdx.x / LPR) * D + part * kEpl;
#pragma unroll
      for (int c = 0; c < kEpl / 16; ++c) {  // 16 elements → one 16-byte store of codes
        float tt[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float x = xs[u][16 * c + e];
          tt[e] = ratio448(x, rk);
        }
        i32x4 w;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          w[g] = cvt_fp8x4(tt[4 * g], tt[4 * g + 1], tt[4 * g + 2], tt[4 * g + 3]);
        *(i32x4*)(k8 + off + 16 * c) = w;
      }
    }
  } else {
    // Item (sb, m, cc): sub-block sb (keys c0 + 64sb ..), keys 4m .. 4m+3,
    // d-chunk cc; its 8 values of each of the 4 keys.
    const bf16* src = V + ((size_t)bh * N + row0) * D;
    float x[VPT][4][8];
    float m = 0.0f;
#pragma unroll
    for (int it = 0; it < VPT; ++it) {
      const int item = threadIdx.x + 256 * it;
      const int sb = item / (16 * CHUNKS), rem = item % (16 * CHUNKS);
      const int mq = rem % 16, cc = rem / 16;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int key = c0 + 64 * sb + 4 * mq + u;
        bf16x8 v = {};
        if (item < VITEMS && key < c_end) v = *(const bf16x8*)(src + (size_t)key * D + cc * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[it][u][e] = (float)v[e];
          m = fmaxf(m, fabsf(x[it][u][e]));
        }
      }
    }
    const float am = block_max(m);
    // Least e with am ≤ 448·2^e: am/448 = f·2^k, f ∈ [0.5, 1); e = k − 1 when
    // f = 0.5 exactly (the quotient is exact there, a power of two). e stays
    // at least −126 so that 2^e is a normal float, whose exponent field is
    // the E8M0 code the attention kernel passes to the MFMA.
    int ex = 0;
    if (am > 0.0f) {
      int k;
      const float f = frexpf(am / kE4m3Max, &k);
      ex = max(f == 0.5f ? k - 1 : k, -126);
    }
    if (threadIdx.x == 0) sc[1] = ldexpf(1.0f, ex);
    uint8_t* dst = v8t + (size_t)bh * D * Npad + seg_vcol(sg, seg, row0) + c0;
#pragma unroll
    for (int it = 0; it < VPT; ++it) {
      const int item = threadIdx.x + 256 * it;
      const int sb = item / (16 * CHUNKS), rem = item % (16 * CHUNKS);
      const int mq = rem % 16, cc = rem / 16;
      if (item >= VITEMS || c0 + 64 * sb >= c_end) continue;  // a block past the end
      const int p = 64 * sb + v8_pos(4 * mq);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *(int*)(dst + (size_t)(cc * 8 + e) * Npad + p) =
            cvt_fp8x4(ldexpf(x[it][0][e], -ex), ldexpf(x[it][1][e], -ex),
                      ldexpf(x[it][2][e], -ex), ldexpf(x[it][3][e], -ex));
    }
  }
}

// ---------------------------------------------------------------------------
// fp8 attention kernel: 4 waves × 32 queries, 64-key tiles, two workgroups per
// compute unit. K8 and V8ᵀ tiles stream into LDS by buffer loads that write
// LDS directly (row-major, 64-bank swizzle), double-buffered and issued an
// iteration ahead. Software pipeline as in the bf16 forward: the softmax of
// tile j runs beside the MFMAs of S(j+1), the row max of tile j+1 beside
// PV(j).
// ---------------------------------------------------------------------------
constexpr int kF8Waves = 4;
constexpr int kF8BM = 32 * kF8Waves;
constexpr int kF8BN = 64;
// Causal issue groups (see the workgroup mapping): used for d = 128 when a
// unit has between these many query tiles (measured: +5% at 8 tiles, +8% at
// 4, but −8% at 16, where the fp8 tiles, half the bytes of bf16 ones, fit
// the L2 without grouping).
constexpr int kF8GroupMinTiles = 4, kF8GroupMaxTiles = 8;

// SPARSE: a block mask over 128-query × 128-key blocks (one per head, or
// shared): the workgroup (one 128-query block) reads its mask row once and
// walks only the visible 64-key tiles with the same schedule; a row that
// sees no key writes O = 0 (and LSE = −∞).
// VARLEN: packed segments (sg); the grid runs over (head, segment, query
// tile) and each workgroup treats its segment as a sequence of its own
// (rows offset to the segment start, its own K'/V scales and V8ᵀ columns).
template <int D, bool CAUSAL, bool WANT_LSE, int EXPM, bool SPARSE, bool VARLEN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_fp8_kernel(const bf16* __restrict__ Q, const uint8_t* __restrict__ k8,
                    const uint8_t* __restrict__ v8t, const float* __restrict__ scales,
                    bf16* __restrict__ O, float* __restrict__ LSE, int N, int Npad, int BH,
                    int n_qtiles, float scale_log2, int rotate, uint64_t seed,
                    const uint8_t* __restrict__ bmask, long mask_stride, Fp8Segs sg,
                    int group_units) {
  static_assert(!SPARSE || kF8BM == kMaskBlockRows, "one query tile per mask block row");
  static_assert(!(SPARSE && VARLEN), "block masks apply to whole sequences");
  constexpr int KD = D / 64;           // fp8 MFMA k-steps over d
  constexpr int KTILE = kF8BN * D;     // K8 tile [64 keys][D bytes]
  constexpr int VTILE = D * kF8BN;     // V8ᵀ tile [D][64 keys]
  constexpr int DT = D / 32;
  constexpr int KLOADS = KTILE / 1024 / kF8Waves;  // 1 KB wave loads per tile and wave
  constexpr int VLOADS = VTILE / 1024 / kF8Waves;
  // LDS: K slots 0, 1 then V slots 0, 1; the rotation's signs.
  __shared__ __attribute__((aligned(16))) char lds[2 * KTILE + 2 * VTILE];
  __shared__ __attribute__((aligned(16))) float sgn[D];
  // (K, V) scale pair of the 128-key chunk of the tile in each K slot,
  // loaded with the tile (one 4-byte element per lane, lanes 0 and 1).
  __shared__ __attribute__((aligned(16))) float scl[2][64];
  char* const k_lds = lds;
  char* const v_lds = lds + 2 * KTILE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, c = lane & 31;

  // Workgroup → (unit, query tile), a unit being a head or (head, segment).
  // Causal: tile-major from the last query tile down, heaviest first (ids
  // round-robin over the XCDs), within groups of group_units units (chosen
  // by the launch: for short sequences one group fills the resident
  // workgroups once, so the few units on each XCD keep their K8 and V8ᵀ in
  // its L2 while all their tiles run). Packed segments without the mask:
  // longest segment first (rank r takes the r-th longest), heads
  // interleaved within a rank. Otherwise each XCD gets a contiguous run of
  // tiles (one head's tiles share its L2).
  int unit, qt;
  if constexpr (CAUSAL) {
    const int units = BH * sg.nseq;
    const int gh = min(units, group_units);
    const int g0 = (int)(blockIdx.x / (gh * n_qtiles)) * gh;
    const int gsize = min(gh, units - g0);
    const int rem = (int)blockIdx.x - g0 * n_qtiles;
    const int step = rem / gsize;
    unit = g0 + (rem - step * gsize);
    qt = n_qtiles - 1 - step;
  } else if constexpr (VARLEN) {
    const int per_rank = BH * n_qtiles;
    const int r = (int)(blockIdx.x / per_rank);
    const int rem = blockIdx.x - r * per_rank;
    qt = rem / BH;
    const int b = rem - qt * BH;
    unit = b * sg.nseq + segment_of_rank(sg.cu, sg.nseq, N, r, lane);
  } else {
    const int total = n_qtiles * BH;
    int logical = blockIdx.x;
    if ((total & 7) == 0) logical = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    unit = logical / n_qtiles;
    qt = logical - unit * n_qtiles;
  }
  const int bh = VARLEN ? unit / sg.nseq : unit;
  const int seg = unit - bh * sg.nseq;
  // Rows [row0, row0 + L) of the head: the whole head, or one segment.
  int row0 = 0, L = N;
  if constexpr (VARLEN) seg_rows(sg, N, seg, row0, L);
  const int q_start = qt * kF8BM;
  if (q_start >= L) return;  // whole workgroup: a segment shorter than the grid's longest

  // Scale pairs (K, V) of this unit's 128-key chunks.
  const int nchunks = ((VARLEN ? sg.max_len : N) + kFp8AmaxRows - 1) / kFp8AmaxRows;
  const float* scl_g = scales + (size_t)unit * nchunks * 2;

  const size_t head = ((size_t)bh * N + row0) * D;
  const uint8_t* Kh = k8 + head;
  const int vcol = VARLEN ? seg_vcol(sg, seg, row0) : 0;
  const uint8_t* Vt = v8t + (size_t)bh * D * Npad + vcol;
  const int q0 = q_start + wave * 32;
  const int qi = q0 + c;
  // Q' operands (two e4m3 terms) and the exp2-domain score factor of this
  // lane's query row without the K scale, formed in the prologue below.
  i32x8 qreg[KD], qlo[KD];
  float c_log2;

  // Per-lane LDS offsets of the MFMA A operands: K8 row c (key), bytes
  // kk·64 + 32h .. +32 (two 16-byte chunks); V8ᵀ row c (d within a 32-row
  // tile), key bytes 32h .. +32.
  int koff[KD][2], voff[2];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk)
#pragma unroll
    for (int u = 0; u < 2; ++u) koff[kk][u] = tile_off_rb<D>(c, 4 * kk + 2 * h + u);
#pragma unroll
  for (int u = 0; u < 2; ++u) voff[u] = tile_off_rb<64>(c, 2 * h + u);

  const int kv_end = CAUSAL ? min(L, q_start + kF8BM) : L;
  const int n_kv = (kv_end + kF8BN - 1) / kF8BN;
  const int first_masked = CAUSAL ? min(q_start / kF8BN, L / kF8BN) : L / kF8BN;

  // Wave loads of the tiles (swizzle applied on the source side). K8 rows
  // past N read as zero (buffer range check); V8ᵀ is zero-padded to Npad.
  int ldk[KLOADS], ldv[VLOADS];
#pragma unroll
  for (int i = 0; i < KLOADS; ++i) {
    const int r = (wave * KLOADS + i) * (1024 / D) + lane / (D / 16);
    ldk[i] = r * D + swz_chunk_rb<D>(r, lane % (D / 16)) * 16;
  }
#pragma unroll
  for (int i = 0; i < VLOADS; ++i) {
    const int r = (wave * VLOADS + i) * 16 + lane / 4;
    ldv[i] = r * Npad + swz_chunk_rb<64>(r, lane % 4) * 16;
  }
  auto gload_k = [&](int slot, int j) __device__ {
    const int key0 = j * kF8BN;
    buffer_to_lds<KLOADS>(Kh + (size_t)key0 * D, (L - key0) * D, k_lds + slot * KTILE, ldk,
                          wave * KLOADS);
    if (wave == 0)
      stats_to_lds(scl_g + (j / 2) * 2, (char*)scl[slot], lane, 2 * (int)sizeof(float));
  };
  auto gload_v = [&](char* tile, int j) __device__ {
    const int key0 = j * kF8BN;
    buffer_to_lds<VLOADS>(Vt + key0, D * Npad - vcol - key0, tile, ldv, wave * VLOADS);
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  // Row sums: the normalisation of O uses the sum of the quantised P̃·2^(8−τ−k)
  // that enter the PV product, formed by the MFMA itself with an A operand of
  // e4m3 ones (every accumulator register of lane c then holds the sum for
  // query c), so numerator and denominator see the same probabilities. The
  // LSE, when requested, uses the fp32 sum of P̃ before quantisation.
  f32x16 lacc = {};
  i32x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = 0x38383838;  // e4m3 1.0 in every byte
  float l_part = 0.0f;

  auto scores = [&](const char* kt, f32x16 (&s)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
        const i32x4 a0 = *(const i32x4*)(kt + t * 32 * D + koff[kk][0]);
        const i32x4 a1 = *(const i32x4*)(kt + t * 32 * D + koff[kk][1]);
        const i32x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        s[t] = mfma32_fp8(a, qreg[kk], s[t]);
        s[t] = mfma32_fp8_bscale(a, qlo[kk], s[t]);
      }
    }
  };
  auto mask = [&](f32x16 (&s)[2], int key0) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 32 * t + acc_row(r, h);
        if (key >= L || (CAUSAL && key > qi)) s[t][r] = -INFINITY;
      }
  };
  auto tile_max = [&](const f32x16 (&s)[2], float c) {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    return half_max(mx) * c;
  };

  // Key tiles in processing order: all of [0, n_kv), or under a block mask
  // only those whose 128-key block this 128-query block sees (its mask row,
  // read once into 64-bit ballots).
  uint64_t mb[kMaskWords] = {};
  if constexpr (SPARSE) {
    const int nb = (N + kMaskBlockRows - 1) / kMaskBlockRows;
    load_mask_bits(bmask + bh * mask_stride + (long)qt * nb, 1, nb, lane, mb);
  }
  auto next_tile = [&](int j) __device__ {
    if constexpr (SPARSE) return next_mask_tile(mb, j, n_kv);
    return j;
  };
  const int c0 = next_tile(0), c1 = next_tile(c0 + 1);
  if (c0 >= n_kv) {  // no visible key for any row of the block: O = 0, LSE = −∞
    if (qi < L) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(i32x2*)(O + head + (size_t)qi * D + 32 * dt + 8 * g + 4 * h) = i32x2{};
      if constexpr (WANT_LSE) {
        if (h == 0) LSE[(size_t)bh * N + row0 + qi] = -INFINITY;
      }
    }
    return;
  }

  gload_k(0, c0);
  if (c1 < n_kv) gload_k(1, c1);
  gload_v(v_lds, c0);
  if (rotate && tid < D) sgn[tid] = rotation_sign(seed, tid);
  __syncthreads();

  // Q' operands while the first tiles load. Lane (c, h) holds elements
  // d = 64kk + 32h + e (e < 32) of query row qi: the B operand layout of the
  // score MFMA. Rotation: signs, then the unnormalised Walsh–Hadamard
  // butterflies over d bits 0–4 (in lane), bit 5 (the two lane halves, by a
  // half swap) and bit 6 (in lane, kk), in the same order and form as the
  // K preparation (lower index a + b, upper a − b); the 1/√d joins the
  // row's scale. The row's amax over both halves sets that scale; codes and
  // the residual term as in the K quantisation.
  {
    float x[KD][32];
    const bf16* Qrow = Q + head + (size_t)qi * D + 32 * h;
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 v = qi < L ? *(const bf16x8*)(Qrow + 64 * kk + 8 * u) : bf16x8{};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[kk][8 * u + e] = (float)v[e];
      }
    if (rotate) {
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
#pragma unroll
        for (int e = 0; e < 32; ++e) x[kk][e] *= sgn[64 * kk + 32 * h + e];
#pragma unroll
        for (int w = 1; w < 32; w <<= 1)
#pragma unroll
          for (int e = 0; e < 32; ++e)
            if (!(e & w)) {
              const float a = x[kk][e], b = x[kk][e + w];
              x[kk][e] = a + b;
              x[kk][e + w] = a - b;
            }
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[kk][e]),
                                                          __float_as_uint(x[kk][e]), false, false);
          const float lo = __uint_as_float(r[0]), hi = __uint_as_float(r[1]);
          x[kk][e] = fmaf(hi, h ? -1.0f : 1.0f, lo);  // lo + hi, or lo − hi
        }
      }
      if constexpr (KD == 2) {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const float a = x[0][e], b = x[1][e];
          x[0][e] = a + b;
          x[1][e] = a - b;
        }
      }
    }
    float am = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int e = 0; e < 32; ++e) am = fmaxf(am, fabsf(x[kk][e]));
    am = half_max(am);
    const Ratio448 rq(am);
    // Scores in the exp2 domain: s·c with c = scale·log2(e)·s_q(row)·s_k.
    c_log2 = scale_from_amax(rotate ? am * kInvSqrtD<D> : am) * scale_log2;
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        float tt[4], dec[4], r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = x[kk][4 * g + e];
          tt[e] = ratio448(v, rq);
        }
        const int w = cvt_fp8x4(tt[0], tt[1], tt[2], tt[3]);
        dec_fp8x4(w, dec);
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = 16.0f * (tt[e] - dec[e]);
        qreg[kk][g] = w;
        qlo[kk][g] = cvt_fp8x4(r[0], r[1], r[2], r[3]);
      }
  }
  wait_vmem();
  __syncthreads();
  // Score factor (with the K scale) and V scale of the tile being softmaxed.
  float c_cur = c_log2 * scl[0][0], sv_cur = scl[0][1];
  f32x16 s[2];
  scores(k_lds, s);
  if (c0 >= first_masked) mask(s, c0 * kF8BN);
  // The exponent offset m_c of O and l starts at tile 0's row max and stays
  // there: when a later tile's row max exceeds m_c + τ, the row's P̃ are
  // stored as P̃·2^−k instead (k the least integer that keeps them ≤ 2^τ)
  // and the PV and row-sum MFMAs take 2^k back as the P operand's block
  // scale, so O and l need no rescale. Only when k would pass kF8KMax does
  // the wave move m_c to the row max and rescale O and l.
  float m_c = tile_max(s, c_cur);
  float kr = 0.0f;          // the row's k
  float off = kF8PExp - m_c;
  int e8p = 127;            // E8M0 code of 2^k
  float pkr = 1.0f;         // 2^k, for the fp32 sum of the LSE
  // The first iteration refills K slot 0: every wave must have read K(0).
  __syncthreads();

  // Tile j (this iteration), jn and jn2 (the next two in processing order;
  // j + 1 and j + 2 without a block mask).
  auto iteration = [&](int j, int jn, int jn2, auto parity_tag, auto has_next_tag) __device__ {
    constexpr int PAR = decltype(parity_tag)::value;
    constexpr bool HAS_NEXT = decltype(has_next_tag)::value;
    (void)j;
    if constexpr (HAS_NEXT) {
      if (jn2 < n_kv) gload_k(PAR, jn2);
      gload_v(v_lds + (PAR ^ 1) * VTILE, jn);
    }
    // P̃·2^(8−τ−k) in e4m3; byte s of the operand: tile s/16, accumulator row s%16.
    i32x8 p8;
    float t_sum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        float pv4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // SPLIT: element e = 3 of every group of four on the polynomial.
          const float x = fmaf(s[t][4 * wd + e], c_cur, off);
          pv4[e] = (EXPM == EXP_POLY || (EXPM == EXP_SPLIT && e == 3)) ? exp2_poly(x) : exp2_hw(x);
          if constexpr (WANT_LSE) t_sum += pv4[e];
        }
        p8[4 * t + wd] = cvt_fp8x4(pv4[0], pv4[1], pv4[2], pv4[3]);
      }
    f32x16 ns[2];
    float c_next = 0.0f, sv_next = 0.0f;
    if constexpr (HAS_NEXT) {
      // Tile jn's scales sit with its K tile in slot PAR ^ 1 until the next
      // iteration refills that slot.
      c_next = c_log2 * scl[PAR ^ 1][0];
      sv_next = scl[PAR ^ 1][1];
      scores(k_lds + (PAR ^ 1) * KTILE, ns);
      // Keep the softmax of tile j beside these MFMAs.
      asm volatile("" ::"v"(p8));
      if (jn >= first_masked) mask(ns, jn * kF8BN);
    }
    const char* vt = v_lds + PAR * VTILE;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const i32x4 a0 = *(const i32x4*)(vt + dt * 32 * 64 + voff[0]);
      const i32x4 a1 = *(const i32x4*)(vt + dt * 32 * 64 + voff[1]);
      oacc[dt] = mfma32_fp8_scaled(__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7), p8,
                                   oacc[dt], e8m0_of(sv_cur), e8p);
    }
    lacc = mfma32_fp8_scaled(ones, p8, lacc, 127, e8p);
    if constexpr (WANT_LSE) l_part = fmaf(t_sum, pkr, l_part);
    if constexpr (HAS_NEXT) {
      const float mx = tile_max(ns, c_next);
      // NaN (a row with no key yet and none in this tile) leaves k as is.
      float k_new = fmaxf(kr, __builtin_ceilf(mx - m_c - kF8Tau));
      if (__ballot(k_new > kF8KMax)) {
        const bool resc = k_new > kF8KMax;
        const float m_new = resc ? mx : m_c;
        const float alpha = resc ? exp2_hw(m_c - m_new) : 1.0f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        lacc[0] *= alpha;  // only register 0 of the row-sum accumulator is read
        l_part *= alpha;
        m_c = m_new;
        k_new = resc ? 0.0f : k_new;
      }
      kr = k_new;
      off = kF8PExp - m_c - kr;
      pkr = __builtin_amdgcn_ldexpf(1.0f, (int)kr);
      e8p = e8m0_of(pkr);
      s[0] = ns[0];
      s[1] = ns[1];
      c_cur = c_next;
      sv_cur = sv_next;
      wait_vmem();
      __syncthreads();
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if constexpr (!SPARSE) {
    int j = 0;
    for (; j + 2 < n_kv; j += 2) {
      iteration(j, j + 1, j + 2, I0{}, std::true_type{});
      iteration(j + 1, j + 2, j + 3, I1{}, std::true_type{});
    }
    if (j + 1 < n_kv) {
      iteration(j, j + 1, j + 2, I0{}, std::true_type{});
      iteration(j + 1, n_kv, n_kv, I1{}, std::false_type{});
    } else {
      iteration(j, n_kv, n_kv, I0{}, std::false_type{});
    }
  } else {
    // The same schedule over the visible tiles only (n_act of them; slots
    // alternate by position): a, b, cc are the tiles at positions p, p+1, p+2.
    const int n_act = count_mask_tiles(mb, 0, n_kv);
    int a = c0, b = c1, cc = next_tile(c1 + 1);
    int p = 0;
    for (; p + 2 < n_act; p += 2) {
      iteration(a, b, cc, I0{}, std::true_type{});
      a = b;
      b = cc;
      cc = next_tile(cc + 1);
      iteration(a, b, cc, I1{}, std::true_type{});
      a = b;
      b = cc;
      cc = next_tile(cc + 1);
    }
    if (p + 1 < n_act) {
      iteration(a, b, cc, I0{}, std::true_type{});
      iteration(b, n_kv, n_kv, I1{}, std::false_type{});
    } else {
      iteration(a, n_kv, n_kv, I0{}, std::false_type{});
    }
  }

  const float inv = 1.0f / lacc[0];
  if (qi < L) {
    bf16* Orow = O + head + (size_t)qi * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        i32x2 w;
        w[0] = (int)pack_bf16x2(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv);
        w[1] = (int)pack_bf16x2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
        *(i32x2*)(Orow + 32 * dt + 8 * g + 4 * h) = w;
      }
    if constexpr (WANT_LSE) {
      const float l = half_sum(l_part);
      if (h == 0) LSE[(size_t)bh * N + row0 + qi] = (m_c + __builtin_log2f(l) - kF8PExp) * kLn2;
    }
  }
}

// The attention launch; `a` carries the operands shared by every variant.
struct Fp8Attend {
  const bf16* q;
  const uint8_t* k8;
  const uint8_t* v8t;
  const float* scales;
  bf16* o;
  float* lse;
  int BH, N;
  float scale;
  int rotate;
  uint64_t seed;
  const uint8_t* bmask = nullptr;  // block mask (SPARSE launches)
  long mask_stride = 0;            // elements between the masks of consecutive heads (0: shared)
  Fp8Segs sg{};                    // packed segments (VARLEN launches: sg.cu set)
};

// Columns of one head's V8ᵀ: N rounded up to 64, plus 64 per segment with
// packed segments (each starts on its own 64-key block).
static int fp8_vcols(int N, const Fp8Segs& sg) {
  const int npad = (N + kFp8Npad - 1) / kFp8Npad * kFp8Npad;
  return sg.cu != nullptr ? npad + kFp8Npad * sg.nseq : npad;
}

template <int D, bool CAUSAL, int EXPM, bool SPARSE, bool VARLEN>
static hipError_t launch_attend_s(const Fp8Attend& a, hipStream_t stream) {
  const int Npad = fp8_vcols(a.N, a.sg);
  const int rows = VARLEN ? a.sg.max_len : a.N;
  const int n_qtiles = (rows + kF8BM - 1) / kF8BM;
  const int units = a.BH * a.sg.nseq;
  const dim3 grid((unsigned)n_qtiles * units);
  int group_units = units;
  if constexpr (CAUSAL && D == 128) {
    // One group = the workgroups the device keeps resident (queried once),
    // rounded down to whole units, a multiple of 8 (the XCD count) so that
    // each XCD holds the same units from tile to tile.
    static const int resident = [] {
      int occ = 0, dev = 0, cus = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &occ, fwd_fp8_kernel<D, CAUSAL, false, EXPM, SPARSE, VARLEN>, 256, 0) !=
              hipSuccess ||
          hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
      }
      return occ * cus;
    }();
    if (n_qtiles >= kF8GroupMinTiles && n_qtiles <= kF8GroupMaxTiles && resident > 0)
      group_units = std::max(8, resident / n_qtiles / 8 * 8);
  }
  if (a.lse != nullptr)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, true, EXPM, SPARSE, VARLEN>), grid, dim3(256),
                       0, stream, a.q, a.k8, a.v8t, a.scales, a.o, a.lse, a.N, Npad, a.BH,
                       n_qtiles, a.scale * kLog2e, a.rotate, a.seed, a.bmask, a.mask_stride,
                       a.sg, group_units);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, false, EXPM, SPARSE, VARLEN>), grid, dim3(256),
                       0, stream, a.q, a.k8, a.v8t, a.scales, a.o, a.lse, a.N, Npad, a.BH,
                       n_qtiles, a.scale * kLog2e, a.rotate, a.seed, a.bmask, a.mask_stride,
                       a.sg, group_units);
  return hipGetLastError();
}

template <int D, bool CAUSAL, int EXPM>
static hipError_t launch_attend_m(const Fp8Attend& a, hipStream_t stream) {
  if (a.sg.cu != nullptr) return launch_attend_s<D, CAUSAL, EXPM, false, true>(a, stream);
  return a.bmask != nullptr ? launch_attend_s<D, CAUSAL, EXPM, true, false>(a, stream)
                            : launch_attend_s<D, CAUSAL, EXPM, false, false>(a, stream);
}

template <int D, bool CAUSAL>
static hipError_t launch_attend_t(const Fp8Attend& a, int exp_mode, hipStream_t stream) {
  if (exp_mode == EXP_POLY) return launch_attend_m<D, CAUSAL, EXP_POLY>(a, stream);
  if (exp_mode == EXP_SPLIT) return launch_attend_m<D, CAUSAL, EXP_SPLIT>(a, stream);
  return launch_attend_m<D, CAUSAL, EXP_HW>(a, stream);
}

static hipError_t launch_attend(const Fp8Attend& a, int d, bool causal, int exp_mode,
                                hipStream_t stream) {
  if (d == 64)
    return causal ? launch_attend_t<64, true>(a, exp_mode, stream)
                  : launch_attend_t<64, false>(a, exp_mode, stream);
  return causal ? launch_attend_t<128, true>(a, exp_mode, stream)
                : launch_attend_t<128, false>(a, exp_mode, stream);
}

template <int D>
static void launch_prep(const void* k, const void* v, uint8_t* k8, uint8_t* v8t, float* scales,
                        int BH, int N, bool rotate, uint64_t seed, const Fp8Segs& sg,
                        hipStream_t stream) {
  const int Npad = fp8_vcols(N, sg);
  const unsigned nchunks = (unsigned)((sg.max_len + kFp8AmaxRows - 1) / kFp8AmaxRows);
  hipLaunchKernelGGL((fp8_prep_kernel<D>), dim3((unsigned)sg.nseq * nchunks, BH, 2), dim3(256),
                     0, stream, (const bf16*)k, (const bf16*)v, k8, v8t, scales, N, Npad,
                     (int)rotate, seed, sg, (int)nchunks);
}

hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                          uint8_t* k8, uint8_t* v8t, float* scales, int B, int H, int N, int d,
                          bool causal, float scale, int exp_mode, bool rotate, uint64_t seed,
                          const uint8_t* block_mask, bool per_head, const int* cu_seqlens,
                          int nseq, int max_seqlen, hipStream_t stream) {
  const int BH = B * H;
  Fp8Segs sg;
  sg.max_len = N;
  if (cu_seqlens != nullptr) {
    sg.cu = cu_seqlens;
    sg.nseq = nseq;
    sg.max_len = max_seqlen;
  }
  if (d == 64) launch_prep<64>(k, v, k8, v8t, scales, BH, N, rotate, seed, sg, stream);
  else launch_prep<128>(k, v, k8, v8t, scales, BH, N, rotate, seed, sg, stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  Fp8Attend a{(const bf16*)q, k8, v8t, scales, (bf16*)o, lse, BH, N, scale, (int)rotate, seed};
  a.sg = sg;
  if (block_mask != nullptr) {
    const long nb = (N + kMaskBlockRows - 1) / kMaskBlockRows;
    a.bmask = block_mask;
    a.mask_stride = per_head ? nb * nb : 0;
  }
  return launch_attend(a, d, causal, exp_mode, stream);
}

hipError_t launch_fwd_fp8_attend(const void* q, void* o, float* lse, const uint8_t* k8,
                                 const uint8_t* v8t, const float* scales, int B, int H, int N,
                                 int d, bool causal, float scale, int exp_mode, bool rotate,
                                 uint64_t seed, hipStream_t stream) {
  Fp8Attend a{(const bf16*)q, k8, v8t, scales, (bf16*)o, lse, B * H, N, scale, (int)rotate, seed};
  a.sg.max_len = N;
  return launch_attend(a, d, causal, exp_mode, stream);
}

}  // namespace fattn
