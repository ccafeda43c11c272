// Fused attention forward, bf16 in/out, fp32 accumulation, for gfx950.
//
// What is computed (FlashAttention-4 news page, "Por qué el enfoque estándar
// ya no funciona"; FlashAttention-3 page, "FlashAttention y FlashAttention-2"):
// O = softmax(scale·Q·Kᵀ [causal]) · V, one workgroup per 128 query rows of
// one head; K and V stream through LDS in 64-key tiles; the scores and the
// probabilities never leave the compute unit.
//
// Layout inside a workgroup (4 waves of 64 lanes, 32 queries per wave):
//  * Sᵀ = K·Qᵀ on 32x32x16 bf16 MFMA: the accumulator column is the query,
//    so each lane owns one query row and the row max / row sum are in-lane
//    reductions plus one exchange between the two lane halves.
//  * Oᵀ += Vᵀ·Pᵀ on the same MFMA: Pᵀ is taken straight from the Sᵀ
//    accumulator registers (the k order inside a 16-key step is free as long
//    as the Vᵀ operand uses the same order); Vᵀ comes from the row-major V tile
//    through the LDS transpose read.
//  * Online softmax in the exp2 domain with conditional rescaling
//    (FlashAttention-4 gist, technical summary 2.B): the running max used for
//    the exponent moves only when a new tile max exceeds it by more than
//    kRescaleTau, so most tiles skip the rescale of Oᵀ and l. Exact, because
//    the same max is used for O, l and LSE.
//  * K/V tiles are double-buffered: the next tile's global loads are issued
//    before the current tile's math and written to the other LDS stage after it
//    (FlashAttention-3 page, innovation 2: loads hidden behind compute).
//  * Causal: key tiles past the workgroup's last query are never loaded, and a
//    wave skips tiles that lie wholly above its diagonal.
#include "fattn_device.hpp"
#include "fattn_launch.h"

namespace fattn {

constexpr int kFwdWaves = 4;
constexpr int kFwdBM = 32 * kFwdWaves;  // query rows per workgroup
constexpr int kFwdBN = 64;              // keys per K/V tile
constexpr float kRescaleTau = 8.0f;     // log2 units: P̃ ≤ 2^8 between rescales

template <int D, bool CAUSAL, int EXPM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                     const bf16* __restrict__ V, bf16* __restrict__ O, float* __restrict__ LSE,
                     int N, int BH, int n_qtiles, float c_log2) {
  constexpr int KD = D / 16;          // MFMA k-steps over the head dimension
  constexpr int CHUNKS = D / 8;       // 16-byte chunks per row
  constexpr int TILE = kFwdBN * D * 2;
  constexpr int CPT = kFwdBN * CHUNKS / 256;  // 16-byte chunks per thread per tensor
  constexpr int NT = kFwdBN / 32;     // 32-key accumulator tiles
  constexpr int NS = kFwdBN / 16;     // 16-key PV steps
  constexpr int DT = D / 32;          // 32-wide output tiles over d
  __shared__ __attribute__((aligned(16))) char lds[2 * 2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31;

  // Workgroup → (head, query tile). Consecutive workgroup ids go to different
  // XCDs; the remap gives each XCD a contiguous run of logical tiles so the
  // tiles of one head share that XCD's L2. Causal: heaviest tiles first.
  const int total = n_qtiles * BH;
  int logical = blockIdx.x;
  if ((total & 7) == 0) logical = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int bh = logical / n_qtiles;
  int qt = logical - bh * n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;

  const size_t head = (size_t)bh * N * D;
  const bf16* Qh = Q + head;
  const bf16* Kh = K + head;
  const bf16* Vh = V + head;
  const int q_start = qt * kFwdBM;
  const int q0 = q_start + wave * 32;
  const int qi = q0 + c;

  // Qᵀ operand: lane holds Q[qi][16kk + 8h + 0..7].
  bf16x8 qreg[KD];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) {
    if (qi < N) qreg[kk] = *(const bf16x8*)(Qh + (size_t)qi * D + kk * 16 + 8 * h);
    else qreg[kk] = bf16x8{};
  }

  const int kv_end = CAUSAL ? min(N, q_start + kFwdBM) : N;
  const int n_kv = (kv_end + kFwdBN - 1) / kFwdBN;

  i32x4 pk[CPT], pv[CPT];
  auto gload = [&](int j) {
    const int key0 = j * kFwdBN;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + i * 256;
      const int r = ch / CHUNKS, cc = ch % CHUNKS;
      const int key = key0 + r;
      if (key < N) {
        pk[i] = *(const i32x4*)(Kh + (size_t)key * D + cc * 8);
        pv[i] = *(const i32x4*)(Vh + (size_t)key * D + cc * 8);
      } else {
        pk[i] = i32x4{};
        pv[i] = i32x4{};
      }
    }
  };
  auto lstore = [&](int stage) {
    char* kb = lds + stage * 2 * TILE;
    char* vb = kb + TILE;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + i * 256;
      const int r = ch / CHUNKS, cc = ch % CHUNKS;
      const int off = tile_off<D>(r, cc);
      *(i32x4*)(kb + off) = pk[i];
      *(i32x4*)(vb + off) = pv[i];
    }
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m_c = -INFINITY;  // exponent offset in use (log2 domain)
  float l_part = 0.0f;    // this lane half's share of the row sum

  // Per-lane pieces of the transpose-read addresses (see lds_read_tr16).
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_sub = (lane & 1) * 8;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int j = 0; j < n_kv; ++j) {
    const int stage = j & 1;
    if (j + 1 < n_kv) gload(j + 1);
    const char* kt = lds + stage * 2 * TILE;
    const char* vt = kt + TILE;
    const int key0 = j * kFwdBN;
    const bool active = !CAUSAL || key0 <= q0 + 31;
    if (active) {
      f32x16 s[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        s[t] = f32x16{};
        const int row = t * 32 + c;
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
          const bf16x8 a = *(const bf16x8*)(kt + tile_off<D>(row, 2 * kk + h));
          s[t] = mfma32(a, qreg[kk], s[t]);
        }
      }
      const bool need_mask = (key0 + kFwdBN > N) || (CAUSAL && key0 + kFwdBN - 1 > q0);
      if (need_mask) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + t * 32 + acc_row(r, h);
            if (key >= N || (CAUSAL && key > qi)) s[t][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
      mx = half_max(mx);
      const float mx_c = mx * c_log2;
      const bool resc = mx_c > m_c + kRescaleTau;
      if (__ballot(resc)) {
        const float m_new = resc ? mx_c : m_c;
        const float alpha = resc ? exp2_hw(m_c - m_new) : 1.0f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        l_part *= alpha;
        m_c = m_new;
      }
      // P̃ = 2^(s·c − m_c) in bf16, kept in the Pᵀ operand layout.
      bf16x8 p[NS];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          i32x4 packed;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = exp2_sel<EXPM>(fmaf(s[t][half * 8 + 2 * e], c_log2, -m_c));
            const float p1 = exp2_sel<EXPM>(fmaf(s[t][half * 8 + 2 * e + 1], c_log2, -m_c));
            l_part += p0 + p1;
            packed[e] = (int)pack_bf16x2(p0, p1);
          }
          p[2 * t + half] = __builtin_bit_cast(bf16x8, packed);
        }
      // Oᵀ += Vᵀ·Pᵀ. Slot e of step ks holds key 16ks + 8(e/4) + 4h + e%4.
#pragma unroll
      for (int ks = 0; ks < NS; ++ks) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int row = 16 * ks + tr_row;
          const int chunk = 4 * dt + tr_chunk;
          const bf16x4 lo = lds_read_tr16(vt + tile_off<D>(row, chunk) + tr_sub);
          const bf16x4 hi = lds_read_tr16(vt + tile_off<D>(row + 8, chunk) + tr_sub);
          oacc[dt] = mfma32(concat(lo, hi), p[ks], oacc[dt]);
        }
      }
    }
    if (j + 1 < n_kv) lstore(stage ^ 1);
    __syncthreads();
  }

  // Epilogue: O = Oᵀ/l (lane holds d = 32dt + 8(r/4) + 4h + r%4 of query qi).
  const float l = half_sum(l_part);
  const float inv = 1.0f / l;
  if (qi < N) {
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
    if (h == 0) LSE[(size_t)bh * N + qi] = (m_c + __builtin_log2f(l)) * kLn2;
  }
}

template <int D, bool CAUSAL, int EXPM>
static hipError_t launch_fwd_t(const void* q, const void* k, const void* v, void* o, float* lse,
                               int BH, int N, float scale, hipStream_t stream) {
  const int n_qtiles = (N + kFwdBM - 1) / kFwdBM;
  const dim3 grid(n_qtiles * BH), block(256);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, EXPM>), grid, block, 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, N, BH, n_qtiles,
                     scale * kLog2e);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fwd_d(const void* q, const void* k, const void* v, void* o, float* lse,
                               int BH, int N, bool causal, float scale, int exp_mode,
                               hipStream_t stream) {
  const bool poly = exp_mode == EXP_POLY;
  if (causal) {
    return poly ? launch_fwd_t<D, true, EXP_POLY>(q, k, v, o, lse, BH, N, scale, stream)
                : launch_fwd_t<D, true, EXP_HW>(q, k, v, o, lse, BH, N, scale, stream);
  }
  return poly ? launch_fwd_t<D, false, EXP_POLY>(q, k, v, o, lse, BH, N, scale, stream)
              : launch_fwd_t<D, false, EXP_HW>(q, k, v, o, lse, BH, N, scale, stream);
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, bool causal, float scale, int exp_mode,
                           hipStream_t stream) {
  const int BH = B * H;
  if (d == 64) return launch_fwd_d<64>(q, k, v, o, lse, BH, N, causal, scale, exp_mode, stream);
  return launch_fwd_d<128>(q, k, v, o, lse, BH, N, causal, scale, exp_mode, stream);
}

}  // namespace fattn
