// Fused attention backward, bf16 in/out, fp32 accumulation, for gfx950.
//
// Gradient of ⟨O, dO⟩ for O = softmax(scale·Q·Kᵀ [causal])·V, recomputing P
// from the forward's log-sum-exp (the pages name the dS and dQ terms and the
// global atomic reduction: FlashAttention-4 gist, technical summary 2.C):
//   D  = rowsum(dO ∘ O), lse2 = LSE·log2(e)    (kernel 1, also zeroes dQ_acc)
//   P  = exp(scale·Q·Kᵀ − LSE),  dV = Pᵀ·dO,  dP = dO·Vᵀ,
//   dS = P ∘ (dP − D),  dK = scale·dSᵀ·Q,  dQ += dS·K   (kernel 2)
//   dQ = scale·dQ_acc → bf16                      (kernel 3)
//
// The statistics and the dQ accumulator are padded to Npad = N rounded up to
// 64 rows per head; padded rows carry lse2 = +∞ and D = 0, so their P (and
// therefore every contribution they make) is exactly 0 without any mask.
// Keys past N are loaded as zero rows of K and V, which makes their scores 0
// and their dQ contribution 0 (dS·K with K = 0); their dK, dV are not stored.
//
// Kernel 2 is key-stationary: a workgroup owns 128 keys (32 per wave, one
// wave per SIMD) of one head and walks the 64-query tiles, so dK and dV
// accumulate in registers of the owning wave with no atomics. dQ needs a sum
// over keys: each wave writes its dS block to LDS as dSᵀ, and after a barrier
// the workgroup multiplies the whole 64×128 dS by the 128-key K tile, so each
// dQ element gets one fp32 atomic add per workgroup and query tile (not one
// per wave).
//
// Operand orientation (32x32x16 bf16 MFMA, accumulator column = lane%32):
//   S, dP   : A = Q / dO rows from LDS, B = K / V rows held in registers,
//             so the accumulator column is the key and each lane owns one key.
//   dVᵀ, dKᵀ: A = dOᵀ / Qᵀ by the LDS transpose read, B = P / dS straight from
//             the S / dP accumulator registers (same k-slot trick as the
//             forward's P·V).
//   dQ      : A = dS by the transpose read of the dSᵀ tile, B = K by the
//             transpose read of the K tile; accumulator column = d, so the
//             atomics of one row are coalesced.
// The query tiles stream through LDS by buffer loads straight into LDS (no
// staging registers), double-buffered; the per-iteration work is split by
// 32-query halves so the exponentials of one half overlap the MFMAs of the
// other.
#include <type_traits>

#include "fattn_device.hpp"
#include "fattn_launch.h"

namespace fattn {

constexpr int kBwdWaves = 4;
constexpr int kBwdBN = 32 * kBwdWaves;  // keys per workgroup
constexpr int kBwdBM = 64;              // queries per inner step

enum : int { BG_VALU = 0x002, BG_MFMA = 0x008, BG_DS_READ = 0x100, BG_DS_WRITE = 0x200,
             BG_TRANS = 0x400 };

// ---------------------------------------------------------------------------
// Kernel 1: D_i = Σ_c dO_ic·O_ic, lse2_i = LSE_i·log2(e) (padded rows: D = 0,
// lse2 = +∞), dQ_acc = 0. One 16-byte chunk of a (padded) row per thread.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ O,
                                                     const bf16* __restrict__ dO,
                                                     const float* __restrict__ LSE,
                                                     float* __restrict__ dvec,
                                                     float* __restrict__ lse2,
                                                     float* __restrict__ dq_acc, int N, int Npad,
                                                     long rows_pad) {
  constexpr int LPR = D / 8;  // lanes per row
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long prow = t / LPR;  // padded row index (bh·Npad + n)
  const int part = (int)(t % LPR);
  const long bh = prow / Npad;
  const int n = (int)(prow - bh * Npad);
  const bool real = prow < rows_pad && n < N;
  float acc = 0.0f;
  if (real) {
    const long row = bh * N + n;
    const bf16x8 o = *(const bf16x8*)(O + row * D + part * 8);
    const bf16x8 g = *(const bf16x8*)(dO + row * D + part * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
  }
  if (prow < rows_pad) {
    const f32x4 z = {};
    *(f32x4*)(dq_acc + prow * D + part * 8) = z;
    *(f32x4*)(dq_acc + prow * D + part * 8 + 4) = z;
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
  if (prow < rows_pad && part == 0) {
    dvec[prow] = real ? acc : 0.0f;
    lse2[prow] = real ? LSE[bh * N + n] * kLog2e : INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Kernel 3: dQ = bf16(scale · dQ_acc) for the N real rows of each head.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const float* __restrict__ dq_acc,
                                                    bf16* __restrict__ dq, long n8, int N,
                                                    int Npad, float scale) {
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n8) return;
  const long row = t / (D / 8);       // bh·N + n
  const int part = (int)(t % (D / 8));
  const long bh = row / N;
  const long prow = bh * Npad + (row - bh * N);
  const f32x4 a = *(const f32x4*)(dq_acc + prow * D + part * 8);
  const f32x4 b = *(const f32x4*)(dq_acc + prow * D + part * 8 + 4);
  i32x4 w;
  w[0] = (int)pack_bf16x2(a[0] * scale, a[1] * scale);
  w[1] = (int)pack_bf16x2(a[2] * scale, a[3] * scale);
  w[2] = (int)pack_bf16x2(b[0] * scale, b[1] * scale);
  w[3] = (int)pack_bf16x2(b[2] * scale, b[3] * scale);
  *(i32x4*)(dq + row * D + part * 8) = w;
}

// s_waitcnt vmcnt(n) (expcnt, lgkmcnt not waited), n < 64.
template <int n>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

// ---------------------------------------------------------------------------
// Kernel 2: key-stationary main loop.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_main_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                     const bf16* __restrict__ V, const bf16* __restrict__ dO,
                     const float* __restrict__ lse2, const float* __restrict__ dvec,
                     float* __restrict__ dq_acc, bf16* __restrict__ dK, bf16* __restrict__ dV,
                     int N, int Npad, int BH, int n_kvtiles, float c_log2, float scale) {
  constexpr int KD = D / 16, CHUNKS = D / 8, DT = D / 32;
  constexpr int RB = D * 2;                         // bytes per Q / dO / K row
  constexpr int QT_BYTES = kBwdBM * RB;             // one Q or dO tile
  constexpr int K_BYTES = kBwdBN * RB;              // the workgroup's K tile
  constexpr int DS_RB = kBwdBM * 2;                 // bytes per dSᵀ row (128)
  constexpr int DS_BYTES = kBwdBN * DS_RB;          // dSᵀ [keys][queries]
  constexpr int KCPT = kBwdBN * CHUNKS / 256;
  constexpr int DQ_DT = 2 * DT / kBwdWaves;         // dQ d-tiles per wave (qt fixed per wave)
  constexpr int LD_LOADS = QT_BYTES / 1024 / kBwdWaves;  // 1 KB wave loads per tile per wave
  // LDS: K | Q0 | dO0 | Q1 | dO1 | dSᵀ | stats[2 stages][lse2 64 | D 64]
  __shared__ __attribute__((aligned(16))) char lds[K_BYTES + 4 * QT_BYTES + DS_BYTES +
                                                   4 * kBwdBM * 4];
  char* const k_lds = lds;
  char* const q_lds = lds + K_BYTES;               // stage s: Q at s·2·QT, dO at s·2·QT + QT
  char* const ds_lds = lds + K_BYTES + 4 * QT_BYTES;
  char* const st_lds = ds_lds + DS_BYTES;          // stage s: lse2 at s·512, D at s·512 + 256

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, c = lane & 31;

  // Workgroup → (head, key tile): heads contiguous per XCD (they share Q, dO
  // in that XCD's L2), key tiles of a head in increasing order (heaviest first
  // under the causal mask).
  const int total = n_kvtiles * BH;
  int logical = blockIdx.x;
  if ((total & 7) == 0) logical = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int bh = logical / n_kvtiles;
  const int jt = logical - bh * n_kvtiles;

  const size_t head = (size_t)bh * N * D;
  const bf16* Qh = Q + head;
  const bf16* Kh = K + head;
  const bf16* Vh = V + head;
  const bf16* dOh = dO + head;
  const float* lse_h = lse2 + (size_t)bh * Npad;
  const float* d_h = dvec + (size_t)bh * Npad;
  float* dqh = dq_acc + (size_t)bh * Npad * D;

  const int kv0 = jt * kBwdBN;
  const int kw0 = kv0 + 32 * wave;  // this wave's first key
  const int key = kw0 + c;          // this lane's key (accumulator column)

  // K tile → LDS (for the dQ product, zero rows past N), K and V rows of this
  // lane → registers (zero past N).
#pragma unroll
  for (int i = 0; i < KCPT; ++i) {
    const int ch = tid + i * 256;
    const int r = ch / CHUNKS, cc = ch % CHUNKS;
    i32x4 x = {};
    if (kv0 + r < N) x = *(const i32x4*)(Kh + (size_t)(kv0 + r) * D + cc * 8);
    *(i32x4*)(k_lds + tile_off<D>(r, cc)) = x;
  }
  bf16x8 kreg[KD], vreg[KD];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) {
    kreg[kk] = key < N ? *(const bf16x8*)(Kh + (size_t)key * D + kk * 16 + 8 * h) : bf16x8{};
    vreg[kk] = key < N ? *(const bf16x8*)(Vh + (size_t)key * D + kk * 16 + 8 * h) : bf16x8{};
  }

  // Per-lane LDS offsets (loop constants).
  int qoff[KD];  // Q / dO rows 32qt + c, chunk 2kk + h
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) qoff[kk] = tile_off<D>(c, 2 * kk + h);
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_sub = (lane & 1) * 8;
  int toff[2][DT];  // Qᵀ / dOᵀ transpose reads: rows 16ks + tr_row (+8), chunk 4dt + tr_chunk
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) toff[hf][dt] = tile_off<D>(tr_row + 8 * hf, 4 * dt + tr_chunk) + tr_sub;
  // dQ tiles of this wave: query half qtw, d-tiles dtw0 .. dtw0 + DQ_DT − 1.
  const int qtw = wave & 1;
  const int dtw0 = (wave >> 1) * DQ_DT;
  int soff[2];  // dSᵀ transpose reads: rows 16ks + tr_row (+8), chunk 4qtw + tr_chunk
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) soff[hf] = tile_off_rb<DS_RB>(tr_row + 8 * hf, 4 * qtw + tr_chunk) + tr_sub;
  int woff[4][2];  // dSᵀ writes: row 32w + c, queries 16ks + 8hf + 4h .. +3
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int qa = 16 * ks + 8 * hf + 4 * h;
      woff[ks][hf] = tile_off_rb<DS_RB>(32 * wave + c, qa >> 3) + (qa & 7) * 2;
    }

  int kToff[DQ_DT][2];  // Kᵀ transpose reads for the dQ d-tiles: rows 16ks + tr_row (+8)
#pragma unroll
  for (int i = 0; i < DQ_DT; ++i)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      kToff[i][hf] = tile_off<D>(tr_row + 8 * hf, 4 * (dtw0 + i) + tr_chunk) + tr_sub;

  const int n_qt = (N + kBwdBM - 1) / kBwdBM;
  const int i0 = CAUSAL ? kv0 / kBwdBM : 0;
  // Query tiles that straddle this key block's diagonal need the causal mask.
  const int first_unmasked = CAUSAL ? min(n_qt, (kv0 + kBwdBN + kBwdBM - 1) / kBwdBM) : i0;

  // Buffer loads of one query tile (Q, dO rows; lse2, D) straight into LDS.
  int ld_off[LD_LOADS];
#pragma unroll
  for (int i = 0; i < LD_LOADS; ++i) {
    const int r = (wave * LD_LOADS + i) * (1024 / RB) + lane / (RB / 16);
    ld_off[i] = r * RB + swz_chunk_rb<RB>(r, lane % (RB / 16)) * 16;
  }
  auto gload = [&](int it, int stage) __device__ {
    const int qs = it * kBwdBM;
    char* qb = q_lds + stage * 2 * QT_BYTES;
    buffer_to_lds<LD_LOADS>(Qh + (size_t)qs * D, (N - qs) * RB, qb, ld_off, wave * LD_LOADS);
    buffer_to_lds<LD_LOADS>(dOh + (size_t)qs * D, (N - qs) * RB, qb + QT_BYTES, ld_off,
                            wave * LD_LOADS);
    // lse2 (wave 0) and D (wave 1): 64 floats = one 4-byte element per lane.
    if (wave < 2) stats_to_lds((wave == 0 ? lse_h : d_h) + qs, st_lds + stage * 512 + wave * 256, lane);
  };

  f32x16 dk_acc[DT], dv_acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk_acc[dt] = f32x16{};
    dv_acc[dt] = f32x16{};
  }

  // P and dS of one 32-query half (accumulator rows = queries 32qt + acc_row,
  // column = key), packed as the B operands of the two 16-query steps.
  auto p_ds = [&](const f32x16& s, const f32x16& dp, const float* lse_s, const float* d_s, int qt,
                  int qs, bool masked, bf16x8& pb0, bf16x8& pb1, bf16x8& db0, bf16x8& db1) __device__ {
    i32x4 pp[2], dd[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int qrow = 32 * qt + 8 * g + 4 * h;
      const f32x4 l4 = *(const f32x4*)(lse_s + qrow);
      const f32x4 d4 = *(const f32x4*)(d_s + qrow);
      float pv[4], dsv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        float p = exp2_hw(fmaf(s[r], c_log2, -l4[e]));
        if (CAUSAL && masked && key > qs + qrow + e) p = 0.0f;
        pv[e] = p;
        dsv[e] = p * (dp[r] - d4[e]);
      }
      pp[g >> 1][2 * (g & 1)] = (int)pack_bf16x2(pv[0], pv[1]);
      pp[g >> 1][2 * (g & 1) + 1] = (int)pack_bf16x2(pv[2], pv[3]);
      dd[g >> 1][2 * (g & 1)] = (int)pack_bf16x2(dsv[0], dsv[1]);
      dd[g >> 1][2 * (g & 1) + 1] = (int)pack_bf16x2(dsv[2], dsv[3]);
    }
    pb0 = __builtin_bit_cast(bf16x8, pp[0]);
    pb1 = __builtin_bit_cast(bf16x8, pp[1]);
    db0 = __builtin_bit_cast(bf16x8, dd[0]);
    db1 = __builtin_bit_cast(bf16x8, dd[1]);
  };

  auto iteration = [&](int it, auto parity_tag, auto masked_tag) __device__ {
    constexpr int PAR = decltype(parity_tag)::value;  // stage of tile it
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int qs = it * kBwdBM;
    if (it + 1 < n_qt) gload(it + 1, PAR ^ 1);
    const char* qb = q_lds + PAR * 2 * QT_BYTES;
    const char* db = qb + QT_BYTES;
    const float* lse_s = (const float*)(st_lds + PAR * 512);
    const float* d_s = lse_s + kBwdBM;

    // S and dP of query half 0.
    f32x16 s0 = {}, dp0 = {}, s1 = {}, dp1 = {};
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      s0 = mfma32(*(const bf16x8*)(qb + qoff[kk]), kreg[kk], s0);
      dp0 = mfma32(*(const bf16x8*)(db + qoff[kk]), vreg[kk], dp0);
    }
    // S and dP of half 1 ∥ P, dS of half 0.
    bf16x8 pb[4], dsb[4];
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      s1 = mfma32(*(const bf16x8*)(qb + 32 * RB + qoff[kk]), kreg[kk], s1);
      dp1 = mfma32(*(const bf16x8*)(db + 32 * RB + qoff[kk]), vreg[kk], dp1);
    }
    p_ds(s0, dp0, lse_s, d_s, 0, qs, MASKED, pb[0], pb[1], dsb[0], dsb[1]);
    if constexpr (!MASKED) {
#pragma unroll
      for (int i = 0; i < 2 * KD; ++i) {
        __builtin_amdgcn_sched_group_barrier(BG_DS_READ, 1, 0);
        __builtin_amdgcn_sched_group_barrier(BG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(BG_VALU | BG_TRANS | BG_DS_READ, 3, 0);
      }
    }
    // dVᵀ, dKᵀ for the 16-query steps of half 0 ∥ P, dS of half 1.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x4 g0 = lds_read_tr16(db + 16 * ks * RB + toff[0][dt]);
        const bf16x4 g1 = lds_read_tr16(db + 16 * ks * RB + toff[1][dt]);
        dv_acc[dt] = mfma32(concat(g0, g1), pb[ks], dv_acc[dt]);
        const bf16x4 q0 = lds_read_tr16(qb + 16 * ks * RB + toff[0][dt]);
        const bf16x4 q1 = lds_read_tr16(qb + 16 * ks * RB + toff[1][dt]);
        dk_acc[dt] = mfma32(concat(q0, q1), dsb[ks], dk_acc[dt]);
      }
    p_ds(s1, dp1, lse_s, d_s, 1, qs, MASKED, pb[2], pb[3], dsb[2], dsb[3]);
    if constexpr (!MASKED) {
#pragma unroll
      for (int i = 0; i < 2 * DT; ++i) {
        __builtin_amdgcn_sched_group_barrier(BG_DS_READ, 2, 0);
        __builtin_amdgcn_sched_group_barrier(BG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(BG_VALU | BG_TRANS | BG_DS_READ, 3, 0);
      }
    }
    // dSᵀ → LDS (row = key, 4 queries per 8-byte write) and the half-1 steps.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const i32x4 w4 = __builtin_bit_cast(i32x4, dsb[ks]);
      i32x2 lo, hi;
      lo[0] = w4[0];
      lo[1] = w4[1];
      hi[0] = w4[2];
      hi[1] = w4[3];
      *(i32x2*)(ds_lds + woff[ks][0]) = lo;
      *(i32x2*)(ds_lds + woff[ks][1]) = hi;
    }
#pragma unroll
    for (int ks = 2; ks < 4; ++ks)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x4 g0 = lds_read_tr16(db + 16 * ks * RB + toff[0][dt]);
        const bf16x4 g1 = lds_read_tr16(db + 16 * ks * RB + toff[1][dt]);
        dv_acc[dt] = mfma32(concat(g0, g1), pb[ks], dv_acc[dt]);
        const bf16x4 q0 = lds_read_tr16(qb + 16 * ks * RB + toff[0][dt]);
        const bf16x4 q1 = lds_read_tr16(qb + 16 * ks * RB + toff[1][dt]);
        dk_acc[dt] = mfma32(concat(q0, q1), dsb[ks], dk_acc[dt]);
      }
    __syncthreads();  // dSᵀ complete

    // dQ[qtw half × this wave's d-tiles] += dS·K over the 128 keys.
    f32x16 dq[DQ_DT];
#pragma unroll
    for (int i = 0; i < DQ_DT; ++i) dq[i] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kBwdBN / 16; ++ks) {
      const bf16x4 a0 = lds_read_tr16(ds_lds + 16 * ks * DS_RB + soff[0]);
      const bf16x4 a1 = lds_read_tr16(ds_lds + 16 * ks * DS_RB + soff[1]);
      const bf16x8 a = concat(a0, a1);
#pragma unroll
      for (int i = 0; i < DQ_DT; ++i) {
        const bf16x4 b0 = lds_read_tr16(k_lds + 16 * ks * RB + kToff[i][0]);
        const bf16x4 b1 = lds_read_tr16(k_lds + 16 * ks * RB + kToff[i][1]);
        dq[i] = mfma32(a, concat(b0, b1), dq[i]);
      }
    }
    float* dqrow = dqh + (size_t)(qs + 32 * qtw + 4 * h) * D + 32 * dtw0 + c;
#pragma unroll
    for (int i = 0; i < DQ_DT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        unsafeAtomicAdd(dqrow + (8 * (r >> 2) + (r & 3)) * D + 32 * i, dq[i][r]);
    // The next tile's loads were issued before this tile's atomics; wait only
    // for them (vmcnt counts in issue order), then release both stages.
    wait_vmem_le<16 * DQ_DT>();
    __syncthreads();
  };

  gload(i0, 0);
  wait_vmem();
  __syncthreads();
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  int it = i0;
  // Masked (diagonal) tiles first, then the rest; parity follows it − i0.
  for (; it < first_unmasked; ++it) {
    if (((it - i0) & 1) == 0) iteration(it, I0{}, std::true_type{});
    else iteration(it, I1{}, std::true_type{});
  }
  if (((it - i0) & 1) == 1 && it < n_qt) {
    iteration(it, I1{}, std::false_type{});
    ++it;
  }
  for (; it + 1 < n_qt; it += 2) {
    iteration(it, I0{}, std::false_type{});
    iteration(it + 1, I1{}, std::false_type{});
  }
  if (it < n_qt) iteration(it, I0{}, std::false_type{});

  // Epilogue: lane holds dKᵀ/dVᵀ[d = 32dt + 8g + 4h + 0..3][key].
  if (key < N) {
    bf16* dk_row = dK + head + (size_t)key * D;
    bf16* dv_row = dV + head + (size_t)key * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        i32x2 wk, wv;
        wk[0] = (int)pack_bf16x2(dk_acc[dt][4 * g] * scale, dk_acc[dt][4 * g + 1] * scale);
        wk[1] = (int)pack_bf16x2(dk_acc[dt][4 * g + 2] * scale, dk_acc[dt][4 * g + 3] * scale);
        wv[0] = (int)pack_bf16x2(dv_acc[dt][4 * g], dv_acc[dt][4 * g + 1]);
        wv[1] = (int)pack_bf16x2(dv_acc[dt][4 * g + 2], dv_acc[dt][4 * g + 3]);
        *(i32x2*)(dk_row + 32 * dt + 8 * g + 4 * h) = wk;
        *(i32x2*)(dv_row + 32 * dt + 8 * g + 4 * h) = wv;
      }
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               float* dq_acc, float* dvec, float* lse2, int BH, int N,
                               float scale, hipStream_t stream) {
  const int Npad = (N + kBwdBM - 1) / kBwdBM * kBwdBM;
  const long rows_pad = (long)BH * Npad;
  {
    const long threads = rows_pad * (D / 8);
    const dim3 grid((unsigned)((threads + 255) / 256));
    hipLaunchKernelGGL((bwd_pre_kernel<D>), grid, dim3(256), 0, stream, (const bf16*)o,
                       (const bf16*)dout, lse, dvec, lse2, dq_acc, N, Npad, rows_pad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int n_kvtiles = (N + kBwdBN - 1) / kBwdBN;
    const dim3 grid(n_kvtiles * BH);
    hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL>), grid, dim3(256), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout,
                       (const float*)lse2, (const float*)dvec, dq_acc, (bf16*)dk, (bf16*)dv, N,
                       Npad, BH, n_kvtiles, scale * kLog2e, scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const long n8 = (long)BH * N * D / 8;
    const dim3 grid((unsigned)((n8 + 255) / 256));
    hipLaunchKernelGGL((bwd_dq_kernel<D>), grid, dim3(256), 0, stream, (const float*)dq_acc,
                       (bf16*)dq, n8, N, Npad, scale);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* dq_acc, float* dvec, float* lse2, int B, int H, int N, int d,
                           bool causal, float scale, hipStream_t stream) {
  const int BH = B * H;
  if (d == 64) {
    return causal ? launch_bwd_t<64, true>(q, k, v, o, lse, dout, dq, dk, dv, dq_acc, dvec, lse2, BH, N, scale, stream)
                  : launch_bwd_t<64, false>(q, k, v, o, lse, dout, dq, dk, dv, dq_acc, dvec, lse2, BH, N, scale, stream);
  }
  return causal ? launch_bwd_t<128, true>(q, k, v, o, lse, dout, dq, dk, dv, dq_acc, dvec, lse2, BH, N, scale, stream)
                : launch_bwd_t<128, false>(q, k, v, o, lse, dout, dq, dk, dv, dq_acc, dvec, lse2, BH, N, scale, stream);
}

}  // namespace fattn
