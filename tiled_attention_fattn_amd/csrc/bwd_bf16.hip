// Fused attention backward, bf16 in/out, fp32 accumulation, for gfx950.
//
// Gradient of ⟨O, dO⟩ for O = softmax(scale·Q·Kᵀ [causal])·V, recomputing P
// from the forward's log-sum-exp (the pages name the dS and dQ terms and the
// global atomic reduction: FlashAttention-4 gist, technical summary 2.C):
//   D  = rowsum(dO ∘ O)                          (kernel 1, also zeroes dQ_acc)
//   P  = exp(scale·Q·Kᵀ − LSE),  dV = Pᵀ·dO,  dP = dO·Vᵀ,
//   dS = P ∘ (dP − D),  dK = scale·dSᵀ·Q,  dQ += dS·K   (kernel 2)
//   dQ = scale·dQ_acc → bf16                      (kernel 3)
//
// Kernel 2 is key-stationary: a workgroup owns 128 keys (32 per wave) of one
// head and walks the 64-query tiles, so dK and dV accumulate in registers of
// the owning wave with no atomics. dQ needs a sum over keys: each wave writes
// its dS block to LDS as dSᵀ, and after a barrier the workgroup multiplies the
// whole 64×128 dS by the 128-key K tile, so each dQ element gets one fp32
// atomic add per workgroup and query tile (not one per wave).
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
#include "fattn_device.hpp"
#include "fattn_launch.h"

namespace fattn {

constexpr int kBwdWaves = 4;
constexpr int kBwdBN = 32 * kBwdWaves;  // keys per workgroup
constexpr int kBwdBM = 64;              // queries per inner step

// ---------------------------------------------------------------------------
// Kernel 1: D_i = Σ_c dO_ic·O_ic, and dQ_acc = 0. One 16-byte chunk per thread.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ O,
                                                     const bf16* __restrict__ dO,
                                                     float* __restrict__ dvec,
                                                     float* __restrict__ dq_acc, int rows) {
  constexpr int LPR = D / 8;  // lanes per row
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long row = t / LPR;
  const int part = (int)(t % LPR);
  float acc = 0.0f;
  if (row < rows) {
    const bf16x8 o = *(const bf16x8*)(O + row * D + part * 8);
    const bf16x8 g = *(const bf16x8*)(dO + row * D + part * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
    f32x4 z = {};
    *(f32x4*)(dq_acc + row * D + part * 8) = z;
    *(f32x4*)(dq_acc + row * D + part * 8 + 4) = z;
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
  if (row < rows && part == 0) dvec[row] = acc;
}

// ---------------------------------------------------------------------------
// Kernel 3: dQ = bf16(scale · dQ_acc), 8 elements per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_dq_kernel(const float* __restrict__ dq_acc,
                                                    bf16* __restrict__ dq, long n8, float scale) {
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n8) return;
  const f32x4 a = *(const f32x4*)(dq_acc + t * 8);
  const f32x4 b = *(const f32x4*)(dq_acc + t * 8 + 4);
  i32x4 w;
  w[0] = (int)pack_bf16x2(a[0] * scale, a[1] * scale);
  w[1] = (int)pack_bf16x2(a[2] * scale, a[3] * scale);
  w[2] = (int)pack_bf16x2(b[0] * scale, b[1] * scale);
  w[3] = (int)pack_bf16x2(b[2] * scale, b[3] * scale);
  *(i32x4*)(dq + t * 8) = w;
}

// ---------------------------------------------------------------------------
// Kernel 2: key-stationary main loop.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_main_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                     const bf16* __restrict__ V, const bf16* __restrict__ dO,
                     const float* __restrict__ LSE, const float* __restrict__ dvec,
                     float* __restrict__ dq_acc, bf16* __restrict__ dK, bf16* __restrict__ dV,
                     int N, int BH, int n_kvtiles, float c_log2, float scale) {
  constexpr int KD = D / 16, CHUNKS = D / 8, DT = D / 32;
  constexpr int QT_BYTES = kBwdBM * D * 2;          // one Q or dO tile
  constexpr int K_BYTES = kBwdBN * D * 2;           // the workgroup's K tile
  constexpr int DS_BYTES = kBwdBN * kBwdBM * 2;     // dSᵀ [keys][queries]
  constexpr int QCPT = kBwdBM * CHUNKS / 256;       // Q (and dO) chunks per thread
  constexpr int KCPT = kBwdBN * CHUNKS / 256;
  constexpr int DQ_TILES = 2 * DT / kBwdWaves;      // dQ output tiles per wave
  // LDS: K | Q0 | dO0 | Q1 | dO1 | dSᵀ | lse2[2][BM] | D[2][BM]
  __shared__ __attribute__((aligned(16))) char lds[K_BYTES + 4 * QT_BYTES + DS_BYTES +
                                                   4 * kBwdBM * 4];
  char* const k_lds = lds;
  char* const q_lds0 = lds + K_BYTES;
  char* const ds_lds = lds + K_BYTES + 4 * QT_BYTES;
  float* const stat_lds = (float*)(ds_lds + DS_BYTES);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const float* lse_h = LSE + (size_t)bh * N;
  const float* d_h = dvec + (size_t)bh * N;
  float* dqh = dq_acc + head;

  const int kv0 = jt * kBwdBN;
  const int kw0 = kv0 + 32 * wave;  // this wave's first key
  const int key = kw0 + c;          // this lane's key (accumulator column)

  // K tile → LDS (for the dQ product), K and V rows of this lane → registers.
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
    if (key < N) {
      kreg[kk] = *(const bf16x8*)(Kh + (size_t)key * D + kk * 16 + 8 * h);
      vreg[kk] = *(const bf16x8*)(Vh + (size_t)key * D + kk * 16 + 8 * h);
    } else {
      kreg[kk] = bf16x8{};
      vreg[kk] = bf16x8{};
    }
  }

  const int n_qt = (N + kBwdBM - 1) / kBwdBM;
  const int i0 = CAUSAL ? kv0 / kBwdBM : 0;

  i32x4 pq[QCPT], pdo[QCPT];
  float pst = 0.0f;  // one statistic per thread for tid < 2·BM
  auto gload = [&](int it) {
    const int qs = it * kBwdBM;
#pragma unroll
    for (int i = 0; i < QCPT; ++i) {
      const int ch = tid + i * 256;
      const int r = ch / CHUNKS, cc = ch % CHUNKS;
      if (qs + r < N) {
        pq[i] = *(const i32x4*)(Qh + (size_t)(qs + r) * D + cc * 8);
        pdo[i] = *(const i32x4*)(dOh + (size_t)(qs + r) * D + cc * 8);
      } else {
        pq[i] = i32x4{};
        pdo[i] = i32x4{};
      }
    }
    if (tid < kBwdBM) {
      pst = (qs + tid < N) ? lse_h[qs + tid] * kLog2e : INFINITY;
    } else if (tid < 2 * kBwdBM) {
      pst = (qs + tid - kBwdBM < N) ? d_h[qs + tid - kBwdBM] : 0.0f;
    }
  };
  auto lstore = [&](int stage) {
    char* qb = q_lds0 + stage * 2 * QT_BYTES;
    char* db = qb + QT_BYTES;
#pragma unroll
    for (int i = 0; i < QCPT; ++i) {
      const int ch = tid + i * 256;
      const int r = ch / CHUNKS, cc = ch % CHUNKS;
      const int off = tile_off<D>(r, cc);
      *(i32x4*)(qb + off) = pq[i];
      *(i32x4*)(db + off) = pdo[i];
    }
    // stat layout per stage: lse2[BM] then D[BM]
    if (tid < 2 * kBwdBM) stat_lds[stage * 2 * kBwdBM + tid] = pst;
  };

  f32x16 dk_acc[DT], dv_acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk_acc[dt] = f32x16{};
    dv_acc[dt] = f32x16{};
  }

  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_sub = (lane & 1) * 8;

  if (i0 < n_qt) {
    gload(i0);
    lstore(0);
  }
  __syncthreads();

  for (int it = i0; it < n_qt; ++it) {
    const int stage = (it - i0) & 1;
    const int qs = it * kBwdBM;
    if (it + 1 < n_qt) gload(it + 1);
    const char* qb = q_lds0 + stage * 2 * QT_BYTES;
    const char* db = qb + QT_BYTES;
    const float* lse2 = stat_lds + stage * 2 * kBwdBM;
    const float* dd = lse2 + kBwdBM;

    // S = Q·Kᵀ and dP = dO·Vᵀ for the 64 queries × this wave's 32 keys.
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      s[qt] = f32x16{};
      dp[qt] = f32x16{};
      const int row = qt * 32 + c;
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
        const bf16x8 a = *(const bf16x8*)(qb + tile_off<D>(row, 2 * kk + h));
        s[qt] = mfma32(a, kreg[kk], s[qt]);
        const bf16x8 g = *(const bf16x8*)(db + tile_off<D>(row, 2 * kk + h));
        dp[qt] = mfma32(g, vreg[kk], dp[qt]);
      }
    }
    // P = 2^(s·c − lse2), dS = P·(dP − D); both packed to bf16 operand slots.
    bf16x8 pb[4], dsb[4];
    const bool need_mask = (kv0 + kBwdBN > N) || (CAUSAL && kw0 + 31 > qs);
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        i32x4 pp, dd4;
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const int g = half * 2 + g2;  // group of 4 accumulator rows
          const int qrow = qt * 32 + 8 * g + 4 * h;
          const f32x4 l4 = *(const f32x4*)(lse2 + qrow);
          const f32x4 d4 = *(const f32x4*)(dd + qrow);
          float pv[4], dsv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float p = exp2_hw(fmaf(s[qt][r], c_log2, -l4[e]));
            if (need_mask) {
              const int q = qs + qrow + e;
              if (key >= N || (CAUSAL && key > q)) p = 0.0f;
            }
            pv[e] = p;
            dsv[e] = p * (dp[qt][r] - d4[e]);
          }
          pp[2 * g2] = (int)pack_bf16x2(pv[0], pv[1]);
          pp[2 * g2 + 1] = (int)pack_bf16x2(pv[2], pv[3]);
          dd4[2 * g2] = (int)pack_bf16x2(dsv[0], dsv[1]);
          dd4[2 * g2 + 1] = (int)pack_bf16x2(dsv[2], dsv[3]);
        }
        pb[2 * qt + half] = __builtin_bit_cast(bf16x8, pp);
        dsb[2 * qt + half] = __builtin_bit_cast(bf16x8, dd4);
      }
    }
    // dSᵀ → LDS for the dQ product: row = key (0..127), 4 queries per write.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const i32x4 w4 = __builtin_bit_cast(i32x4, dsb[ks]);
      // slots 0..3 hold queries 16ks + 4h + 0..3, slots 4..7 queries 16ks + 8 + 4h + 0..3
      const int krow = 32 * wave + c;
      const int q_a = 16 * ks + 4 * h;
      i32x2 lo, hi;
      lo[0] = w4[0];
      lo[1] = w4[1];
      hi[0] = w4[2];
      hi[1] = w4[3];
      *(i32x2*)(ds_lds + tile_off<64>(krow, q_a >> 3) + (q_a & 7) * 2) = lo;
      *(i32x2*)(ds_lds + tile_off<64>(krow, (q_a + 8) >> 3) + ((q_a + 8) & 7) * 2) = hi;
    }
    // dVᵀ += dOᵀ·P and dKᵀ += Qᵀ·dS (contraction over the 64 queries).
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int row = 16 * ks + tr_row;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int chunk = 4 * dt + tr_chunk;
        const bf16x4 g0 = lds_read_tr16(db + tile_off<D>(row, chunk) + tr_sub);
        const bf16x4 g1 = lds_read_tr16(db + tile_off<D>(row + 8, chunk) + tr_sub);
        dv_acc[dt] = mfma32(concat(g0, g1), pb[ks], dv_acc[dt]);
        const bf16x4 q0 = lds_read_tr16(qb + tile_off<D>(row, chunk) + tr_sub);
        const bf16x4 q1 = lds_read_tr16(qb + tile_off<D>(row + 8, chunk) + tr_sub);
        dk_acc[dt] = mfma32(concat(q0, q1), dsb[ks], dk_acc[dt]);
      }
    }
    __syncthreads();  // dSᵀ complete

    // dQ[64 × D] += dS[64 × 128]·K[128 × D]; this wave's output tiles.
#pragma unroll
    for (int ot = 0; ot < DQ_TILES; ++ot) {
      const int tile = wave * DQ_TILES + ot;
      const int qt = tile & 1, dt = tile >> 1;
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < kBwdBN / 16; ++ks) {
        const int row = 16 * ks + tr_row;
        const bf16x4 a0 = lds_read_tr16(ds_lds + tile_off<64>(row, 4 * qt + tr_chunk) + tr_sub);
        const bf16x4 a1 = lds_read_tr16(ds_lds + tile_off<64>(row + 8, 4 * qt + tr_chunk) + tr_sub);
        const bf16x4 b0 = lds_read_tr16(k_lds + tile_off<D>(row, 4 * dt + tr_chunk) + tr_sub);
        const bf16x4 b1 = lds_read_tr16(k_lds + tile_off<D>(row + 8, 4 * dt + tr_chunk) + tr_sub);
        acc = mfma32(concat(a0, a1), concat(b0, b1), acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = qs + 32 * qt + acc_row(r, h);
        if (q < N) unsafeAtomicAdd(dqh + (size_t)q * D + 32 * dt + c, acc[r]);
      }
    }
    if (it + 1 < n_qt) lstore(stage ^ 1);
    __syncthreads();
  }

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
                               float* dq_acc, float* dvec, int BH, int N, float scale,
                               hipStream_t stream) {
  const long rows = (long)BH * N;
  {
    const long threads = rows * (D / 8);
    const dim3 grid((unsigned)((threads + 255) / 256));
    hipLaunchKernelGGL((bwd_pre_kernel<D>), grid, dim3(256), 0, stream, (const bf16*)o,
                       (const bf16*)dout, dvec, dq_acc, (int)rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int n_kvtiles = (N + kBwdBN - 1) / kBwdBN;
    const dim3 grid(n_kvtiles * BH);
    hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL>), grid, dim3(256), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout, lse,
                       (const float*)dvec, dq_acc, (bf16*)dk, (bf16*)dv, N, BH, n_kvtiles,
                       scale * kLog2e, scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const long n8 = rows * D / 8;
    const dim3 grid((unsigned)((n8 + 255) / 256));
    hipLaunchKernelGGL(bwd_dq_kernel, grid, dim3(256), 0, stream, (const float*)dq_acc,
                       (bf16*)dq, n8, scale);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* dq_acc, float* dvec, int B, int H, int N, int d, bool causal,
                           float scale, hipStream_t stream) {
  const int BH = B * H;
  if (d == 64) {
    return causal ? launch_bwd_t<64, true>(q, k, v, o, lse, dout, dq, dk, dv, dq_acc, dvec, BH, N, scale, stream)
                  : launch_bwd_t<64, false>(q, k, v, o, lse, dout, dq, dk, dv, dq_acc, dvec, BH, N, scale, stream);
  }
  return causal ? launch_bwd_t<128, true>(q, k, v, o, lse, dout, dq, dk, dv, dq_acc, dvec, BH, N, scale, stream)
                : launch_bwd_t<128, false>(q, k, v, o, lse, dout, dq, dk, dv, dq_acc, dvec, BH, N, scale, stream);
}

}  // namespace fattn
