// Fused attention backward, bf16 in/out, fp32 accumulation, for gfx950.
//
// Gradient of ⟨O, dO⟩ for O = softmax(scale·Q·Kᵀ [causal])·V, recomputing P
// from the forward's log-sum-exp (the pages name the dS and dQ terms:
// FlashAttention-4 gist, technical summary 2.C):
//   D  = rowsum(dO ∘ O), lse2 = LSE·log2(e)            (dQ kernel, run first;
//                                                        it stores −D for the dK/dV kernel)
//   P  = exp(scale·Q·Kᵀ − LSE),  dP = dO·Vᵀ,  dS = P ∘ (dP − D)
//   dQ = scale·dS·K                                      (dQ kernel, per query block)
//   dV = Pᵀ·dO,  dK = scale·dSᵀ·Q                       (dK/dV kernel, per key block)
//
// The statistics are padded to Npad = N rounded up to 64 rows per head;
// padded rows carry lse2 = +∞ and −D = 0, so their P (and every contribution
// they make) is exactly 0 without any mask.
//
// Block masks (SPARSE): the dK/dV kernel walks only the query tiles whose
// block row sees its key block (the mask column), the dQ kernel only the key
// tiles of the blocks its query block sees (the mask row).
//
// Packed variable-length sequences (VARLEN): both kernels run over
// (head, segment, tile) and treat each segment as a sequence of its own
// (rows offset to the segment start, length = the segment's). Rows past the
// segment end read as zero from every buffer load (Q, dO, K, V and the
// statistics alike), so they contribute nothing: their Q and dO are zero and
// so is every product they enter.
//
// dQ is a sum over keys and dK, dV are sums over queries. The dK/dV kernel
// owns a block of keys and walks the query tiles, so dK and dV accumulate in
// registers; the dQ kernel owns a block of queries and walks the key tiles (it
// recomputes S and dP, two extra products), so dQ accumulates in registers
// too. Nothing is reduced through global atomics: on gfx950 the fp32 atomic
// traffic of a fused kernel (one add per dQ element per key block and query
// tile) costs more time in the L2 than the recomputation, and without it the
// gradients are bitwise reproducible.
//
// Operand orientation (32x32x16 bf16 MFMA, accumulator column = lane%32):
//  dK/dV kernel (column = key):
//   S, dP   : A = Q / dO rows from LDS, B = K / V rows held in registers.
//   dVᵀ, dKᵀ: A = dOᵀ / Qᵀ by the LDS transpose read, B = P / dS straight from
//             the S / dP accumulator registers (the forward's P·V trick).
//  dQ kernel (column = query):
//   Sᵀ, dPᵀ : A = K / V rows from LDS, B = Q / dO rows held in registers.
//   dQᵀ     : A = Kᵀ by the LDS transpose read, B = dSᵀ from the accumulators.
// Tiles stream through LDS by buffer loads straight into LDS (no staging
// registers), double-buffered.
#include <type_traits>

#include "fattn_device.hpp"
#include "fattn_launch.h"

namespace fattn {

constexpr int kBwdWaves = 4;
constexpr int kBwdBN = 32 * kBwdWaves;  // keys per workgroup
constexpr int kBwdBM = 64;              // queries per inner step
constexpr int kLeadB = 3;               // LDS operand reads in flight ahead of the MFMAs

enum : int { BG_VALU = 0x002, BG_MFMA = 0x008, BG_DS_READ = 0x100, BG_DS_WRITE = 0x200,
             BG_TRANS = 0x400 };

// ---------------------------------------------------------------------------
// dK/dV kernel, key-stationary (launched after the dQ kernel, which writes
// the row statistics it reads).
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool VARLEN, bool SPARSE>
// d = 128 needs more than half the register file (434 of 512 per lane with
// the causal mask, 333 without: K, V and the dK, dV accumulators of its 32
// keys), so one wave per SIMD; d = 64 fits in 256, two waves per SIMD.
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 1)))
void bwd_dkdv_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                     const bf16* __restrict__ V, const bf16* __restrict__ dO,
                     const float* __restrict__ lse2, const float* __restrict__ dvec,
                     bf16* __restrict__ dK, bf16* __restrict__ dV,
                     int N, int Npad, int BH, int n_kvtiles, float c_log2, float scale,
                     const int* __restrict__ cu, int nseq, const uint8_t* __restrict__ bmask,
                     long mask_stride) {
  static_assert(!SPARSE || (kBwdBN == kMaskBlockRows && 2 * kBwdBM == kMaskBlockRows),
                "one key block per mask column, two query tiles per mask row");
  constexpr int KD = D / 16, DT = D / 32;
  constexpr int RB = D * 2;                         // bytes per Q / dO row
  constexpr int QT_BYTES = kBwdBM * RB;             // one Q or dO tile
  constexpr int LD_LOADS = QT_BYTES / 1024 / kBwdWaves;  // 1 KB wave loads per tile per wave
  // LDS: stats[2 stages][lse2 64 | −D 64] | Q0 | dO0 | Q1 | dO1. The statistics
  // come first so that their reads reach them through the 16-bit immediate
  // offset of the DS instructions (behind 64 KB of tiles every read needed an
  // address computed by a VALU op); 1 KB keeps the tiles' bank pattern.
  __shared__ __attribute__((aligned(16))) char lds[4 * kBwdBM * 4 + 4 * QT_BYTES];
  char* const st_lds = lds;                        // stage s: lse2 at s·512, −D at s·512 + 256
  char* const q_lds = lds + 4 * kBwdBM * 4;        // stage s: Q at s·2·QT, dO at s·2·QT + QT

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, c = lane & 31;

  // Workgroup → (head[, segment], key tile). Causal: tile-major from the
  // first key tile up (early key tiles see the most queries), heaviest first
  // over the whole grid, ids round-robin over the XCDs (with a multiple of 8
  // units an XCD keeps the same units from tile to tile). Otherwise heads contiguous per XCD (they
  // share Q, dO in that XCD's L2), key tiles of a head in increasing order.
  int unit, jt;
  if constexpr (CAUSAL) {
    const int units = BH * (VARLEN ? nseq : 1);
    jt = (int)(blockIdx.x / units);
    unit = blockIdx.x - jt * units;
  } else {
    const int total = n_kvtiles * BH * (VARLEN ? nseq : 1);
    int logical = blockIdx.x;
    if ((total & 7) == 0) logical = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    unit = logical / n_kvtiles;
    jt = logical - unit * n_kvtiles;
  }
  const int bh = VARLEN ? unit / nseq : unit;
  int row0 = 0, L = N;  // rows of the sequence or segment (offsets clamped to [0, N])
  if constexpr (VARLEN) {
    const int sg = unit - bh * nseq;
    row0 = min(max(cu[sg], 0), N);
    L = min(max(cu[sg + 1], row0), N) - row0;
  }
  const int kv0 = jt * kBwdBN;
  if (kv0 >= L) return;  // whole workgroup

  const size_t head = ((size_t)bh * N + row0) * D;
  const bf16* Qh = Q + head;
  const bf16* Kh = K + head;
  const bf16* Vh = V + head;
  const bf16* dOh = dO + head;
  const float* lse_h = lse2 + (size_t)bh * Npad + row0;
  const float* d_h = dvec + (size_t)bh * Npad + row0;

  const int kw0 = kv0 + 32 * wave;  // this wave's first key
  const int key = kw0 + c;          // this lane's key (accumulator column)

  // K and V rows of this lane → registers (zero past the end).
  bf16x8 kreg[KD], vreg[KD];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) {
    kreg[kk] = key < L ? *(const bf16x8*)(Kh + (size_t)key * D + kk * 16 + 8 * h) : bf16x8{};
    vreg[kk] = key < L ? *(const bf16x8*)(Vh + (size_t)key * D + kk * 16 + 8 * h) : bf16x8{};
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
  const int n_qt = (L + kBwdBM - 1) / kBwdBM;
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
    buffer_to_lds<LD_LOADS>(Qh + (size_t)qs * D, (L - qs) * RB, qb, ld_off, wave * LD_LOADS);
    buffer_to_lds<LD_LOADS>(dOh + (size_t)qs * D, (L - qs) * RB, qb + QT_BYTES, ld_off,
                            wave * LD_LOADS);
    // lse2 (wave 0) and −D (wave 1): 64 floats = one 4-byte element per lane
    // (a segment's rows only: rows past its end read as zero).
    if (wave < 2)
      stats_to_lds((wave == 0 ? lse_h : d_h) + qs, st_lds + stage * 512 + wave * 256, lane,
                   VARLEN ? min(kBwdBM, L - qs) * 4 : kBwdBM * 4);
  };

  f32x16 dk_acc[DT], dv_acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk_acc[dt] = f32x16{};
    dv_acc[dt] = f32x16{};
  }

  // P and dS of one element of a 32-query half hh (accumulator register
  // r = 4g + e: query 32hh + 8g + 4h + e, column = this lane's key), packed in
  // pairs into the B operands of the two 16-query steps of the half. The
  // half's statistics are read from LDS ahead of its steps (load_stats).
  struct HalfState {
    f32x4 l4[4], d4[4];
    float pv[2], dsv[2];
    i32x4 pp[2], dd[2];
  };
  auto load_stats = [&](const float* lse_s, const float* d_s, int hh, HalfState& hs) __device__ {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      hs.l4[g] = *(const f32x4*)(lse_s + 32 * hh + 8 * g + 4 * h);
      hs.d4[g] = *(const f32x4*)(d_s + 32 * hh + 8 * g + 4 * h);
    }
  };
  auto neg_d = [](const HalfState& hs) __device__ {
    f32x16 c;
#pragma unroll
    for (int x = 0; x < 16; ++x) c[x] = hs.d4[x / 4][x % 4];
    return c;
  };
  auto pds_step = [&](const f32x16& sv, const f32x16& dpv, int hh, int qs, bool masked,
                      HalfState& hs, int x) __device__ {
    const int g = x / 4, e = x % 4, r = x;
    const int qrow = 32 * hh + 8 * g + 4 * h;
    float p = exp2_hw(fmaf(sv[r], c_log2, -hs.l4[g][e]));
    if (CAUSAL && masked && key > qs + qrow + e) p = 0.0f;
    const float ds = p * dpv[r];  // dpv = dP − D (the chain starts at −D)
    hs.pv[e & 1] = p;
    hs.dsv[e & 1] = ds;
    if (e & 1) {
      const int w = 2 * (g & 1) + (e >> 1);
      hs.pp[g >> 1][w] = (int)pack_bf16x2(hs.pv[0], hs.pv[1]);
      hs.dd[g >> 1][w] = (int)pack_bf16x2(hs.dsv[0], hs.dsv[1]);
      // Keep the step beside its MFMA instead of letting it sink to the use.
      asm volatile("" ::"v"(hs.pp[g >> 1][w]), "v"(hs.dd[g >> 1][w]));
    }
  };

  // One query tile. The work is laid out in program order as pieces of one
  // MFMA each, separated by scheduling fences; each piece issues the LDS
  // operand read kLeadB pieces ahead and one element step of the softmax
  // gradient, so no MFMA waits for its own operand (one wave per SIMD: there
  // is no other wave to hide the LDS latency) and the VALU work sits beside
  // the MFMAs:
  //   A: S, dP of half 0 (16 MFMA)  B: S, dP of half 1 ∥ P, dS of half 0
  //   C: dVᵀ, dKᵀ of half 0 ∥ P, dS of half 1   D: dVᵀ, dKᵀ of half 1
  // itn: the next query tile in processing order (it + 1 without a block mask).
  auto iteration = [&](int it, int itn, auto parity_tag, auto masked_tag) __device__ {
    constexpr int PAR = decltype(parity_tag)::value;  // stage of tile it
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int NR = 4 * KD;  // S/dP operand reads: half i/(2KD), kk (i/2)%KD, Q or dO by i%2
    const int qs = it * kBwdBM;
    if (itn < n_qt) gload(itn, PAR ^ 1);
    const char* qb = q_lds + PAR * 2 * QT_BYTES;
    const char* db = qb + QT_BYTES;
    const float* lse_s = (const float*)(st_lds + PAR * 512);
    const float* d_s = lse_s + kBwdBM;

    auto sread = [&](int i) __device__ {
      const int hh = i / (2 * KD), kk = (i / 2) % KD;
      return *(const bf16x8*)((i % 2 ? db : qb) + hh * 32 * RB + qoff[kk]);
    };
    f32x16 sd[2][2];  // [half][S, dP]
    bf16x8 ra[NR];
    HalfState hs0, hs1;
    load_stats(lse_s, d_s, 0, hs0);
#pragma unroll
    for (int i = 0; i < kLeadB; ++i) ra[i] = sread(i);
    load_stats(lse_s, d_s, 1, hs1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int hh = i / (2 * KD), kk = (i / 2) % KD, w = i % 2;
      // The dP chain starts from −D of its rows, so it ends at dP − D.
      const f32x16 c0 = w ? neg_d(hh ? hs1 : hs0) : f32x16{};
      sd[hh][w] = mfma32(ra[i], w ? vreg[kk] : kreg[kk], kk == 0 ? c0 : sd[hh][w]);
      if (i + kLeadB < NR) ra[i + kLeadB] = sread(i + kLeadB);
      if (hh == 1) {
        // 16 element steps of half 0 over the 2KD pieces of phase B.
#pragma unroll
        for (int x = (i - 2 * KD) * 16 / (2 * KD); x < (i - 2 * KD + 1) * 16 / (2 * KD); ++x)
          pds_step(sd[0][0], sd[0][1], 0, qs, MASKED, hs0, x);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    bf16x8 pb[4], dsb[4];
    pb[0] = __builtin_bit_cast(bf16x8, hs0.pp[0]);
    pb[1] = __builtin_bit_cast(bf16x8, hs0.pp[1]);
    dsb[0] = __builtin_bit_cast(bf16x8, hs0.dd[0]);
    dsb[1] = __builtin_bit_cast(bf16x8, hs0.dd[1]);

    // dVᵀ += dOᵀ·P, dKᵀ += Qᵀ·dS: piece i = ks (i / 2DT), d tile (i / 2) % DT,
    // dV or dK by i % 2; two transpose reads each.
    constexpr int NT = 8 * DT;
    bf16x4 ta[NT][2];
    auto tread = [&](int i) __device__ {
      const int ks = i / (2 * DT), dt = (i / 2) % DT;
      const char* base = (i % 2 ? qb : db) + 16 * ks * RB;
      ta[i][0] = lds_read_tr16(base + toff[0][dt]);
      ta[i][1] = lds_read_tr16(base + toff[1][dt]);
    };
#pragma unroll
    for (int i = 0; i < kLeadB; ++i) tread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int ks = i / (2 * DT), dt = (i / 2) % DT;
      if (ks == 2 && i % (2 * DT) == 0) {
        pb[2] = __builtin_bit_cast(bf16x8, hs1.pp[0]);
        pb[3] = __builtin_bit_cast(bf16x8, hs1.pp[1]);
        dsb[2] = __builtin_bit_cast(bf16x8, hs1.dd[0]);
        dsb[3] = __builtin_bit_cast(bf16x8, hs1.dd[1]);
      }
      const bf16x8 a = concat(ta[i][0], ta[i][1]);
      if (i % 2) dk_acc[dt] = mfma32(a, dsb[ks], dk_acc[dt]);
      else dv_acc[dt] = mfma32(a, pb[ks], dv_acc[dt]);
      if (i + kLeadB < NT) tread(i + kLeadB);
      if (ks < 2) {
        // 16 element steps of half 1 over the 4DT pieces of phase C.
#pragma unroll
        for (int x = i * 16 / (4 * DT); x < (i + 1) * 16 / (4 * DT); ++x)
          pds_step(sd[1][0], sd[1][1], 1, qs, MASKED, hs1, x);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Both stages are free once every wave is done with this tile and the
    // next tile's loads have landed.
    wait_vmem();
    __syncthreads();
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if constexpr (!SPARSE) {
    gload(i0, 0);
    wait_vmem();
    __syncthreads();
    int it = i0;
    // Masked (diagonal) tiles first, then the rest; parity follows it − i0.
    for (; it < first_unmasked; ++it) {
      if (((it - i0) & 1) == 0) iteration(it, it + 1, I0{}, std::true_type{});
      else iteration(it, it + 1, I1{}, std::true_type{});
    }
    if (((it - i0) & 1) == 1 && it < n_qt) {
      iteration(it, it + 1, I1{}, std::false_type{});
      ++it;
    }
    for (; it + 1 < n_qt; it += 2) {
      iteration(it, it + 1, I0{}, std::false_type{});
      iteration(it + 1, it + 2, I1{}, std::false_type{});
    }
    if (it < n_qt) iteration(it, it + 1, I0{}, std::false_type{});
  } else {
    // Only the query tiles whose block row sees this key block (its column
    // of the mask); stages alternate by position. A key block no query sees
    // keeps dK = dV = 0.
    uint64_t mb[kMaskWords];
    const int nb = (N + kMaskBlockRows - 1) / kMaskBlockRows;
    load_mask_bits(bmask + bh * mask_stride + jt, nb, nb, lane, mb);
    int a = next_mask_tile(mb, i0, n_qt);
    if (a < n_qt) {
      gload(a, 0);
      wait_vmem();
      __syncthreads();
      int b = next_mask_tile(mb, a + 1, n_qt);
      for (int pos = 0; a < n_qt; ++pos) {
        if (pos & 1) {
          if (a < first_unmasked) iteration(a, b, I1{}, std::true_type{});
          else iteration(a, b, I1{}, std::false_type{});
        } else {
          if (a < first_unmasked) iteration(a, b, I0{}, std::true_type{});
          else iteration(a, b, I0{}, std::false_type{});
        }
        a = b;
        b = next_mask_tile(mb, b + 1, n_qt);
      }
    }
  }

  // Epilogue: lane holds dKᵀ/dVᵀ[d = 32dt + 8g + 4h + 0..3][key].
  if (key < L) {
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

// ---------------------------------------------------------------------------
// dQ kernel, query-stationary. A workgroup owns 128 queries of one head
// (32 per wave, one per lane column) and walks the 64-key tiles up to its
// diagonal: Sᵀ = K·Qᵀ and dPᵀ = V·dOᵀ with Q, dO in registers, then
// dS = P ∘ (dP − D) packed as the B operand of dQᵀ += Kᵀ·dSᵀ.
// ---------------------------------------------------------------------------
constexpr int kDqWaves = 4;
constexpr int kDqBM = 32 * kDqWaves;  // queries per workgroup
constexpr int kDqBN = 64;             // keys per tile

template <int D, bool CAUSAL, bool VARLEN, bool SPARSE>
// Two waves per SIMD at d = 128 (up to 256 registers), three at d = 64 (168).
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2, D == 64 ? 3 : 2)))
void bwd_dq_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                   const bf16* __restrict__ V, const bf16* __restrict__ dO,
                   const bf16* __restrict__ O, const float* __restrict__ LSE,
                   float* __restrict__ lse2, float* __restrict__ dvec,
                   bf16* __restrict__ dQ, int N, int Npad, int BH, int n_qtiles, float c_log2,
                   float scale, const int* __restrict__ cu, int nseq,
                   const uint8_t* __restrict__ bmask, long mask_stride) {
  static_assert(!SPARSE || (kDqBM == kMaskBlockRows && 2 * kDqBN == kMaskBlockRows),
                "one query block per mask row, two key tiles per mask column");
  constexpr int KD = D / 16, RB = D * 2, TILE = kDqBN * RB, DT = D / 32;
  constexpr int LOADS = TILE / 1024 / kDqWaves;  // 1 KB wave loads per tensor per tile
  // LDS: K slots 0, 1 then V slots 0, 1, row-major with the 64-bank swizzle.
  __shared__ __attribute__((aligned(16))) char lds[4 * TILE];
  char* const k_lds = lds;
  char* const v_lds = lds + 2 * TILE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, c = lane & 31;

  // Workgroup → (head[, segment], query tile). Causal: tile-major from the
  // last query tile down, heaviest first over the whole grid (as in the
  // forward). Otherwise XCD-aware: each XCD gets a contiguous run of tiles.
  int unit, qt;
  if constexpr (CAUSAL) {
    const int units = BH * (VARLEN ? nseq : 1);
    const int step = (int)(blockIdx.x / units);
    unit = blockIdx.x - step * units;
    qt = n_qtiles - 1 - step;
  } else {
    const int total = n_qtiles * BH * (VARLEN ? nseq : 1);
    int logical = blockIdx.x;
    if ((total & 7) == 0) logical = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    unit = logical / n_qtiles;
    qt = logical - unit * n_qtiles;
  }
  const int bh = VARLEN ? unit / nseq : unit;
  int row0 = 0, L = N;  // rows of the sequence or segment (offsets clamped to [0, N])
  if constexpr (VARLEN) {
    const int sg = unit - bh * nseq;
    row0 = min(max(cu[sg], 0), N);
    L = min(max(cu[sg + 1], row0), N) - row0;
  }
  const int q_start = qt * kDqBM;
  if (q_start >= L) return;  // whole workgroup

  const size_t head = ((size_t)bh * N + row0) * D;
  const bf16* Qh = Q + head;
  const bf16* Kh = K + head;
  const bf16* Vh = V + head;
  const bf16* dOh = dO + head;
  const int qi = q_start + 32 * wave + c;  // this lane's query
  const bool qv = qi < L;

  // Qᵀ and dOᵀ operands: lane holds row qi, elements 16kk + 8h + 0..7.
  bf16x8 qr[KD], dor[KD];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) {
    qr[kk] = qv ? *(const bf16x8*)(Qh + (size_t)qi * D + kk * 16 + 8 * h) : bf16x8{};
    dor[kk] = qv ? *(const bf16x8*)(dOh + (size_t)qi * D + kk * 16 + 8 * h) : bf16x8{};
  }

  // Row statistics of this lane's query, for this kernel and for the dK/dV
  // kernel that runs after it: D = rowsum(dO∘O) and lse2 = LSE·log2(e).
  // D is summed in one fixed order: an FMA chain over each 16-byte chunk
  // of the row, then pairs of chunks combined as a butterfly over the chunk
  // index (bits 3, 2, 1 of chunk 2kk + h are bits of kk, in-lane; bit 0 is
  // the lane half). Rows in [L, Npad) of the last tile get D = 0 and
  // lse2 = +∞, so that their P, and every contribution they make, is 0.
  float dq_d = 0.0f;
  {
    const bf16* Oh = O + head;
    float part[KD];
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      const bf16x8 o = qv ? *(const bf16x8*)(Oh + (size_t)qi * D + kk * 16 + 8 * h) : bf16x8{};
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)dor[kk][e], acc);
      part[kk] = acc;
    }
#pragma unroll
    for (int m = KD / 2; m >= 1; m >>= 1)
#pragma unroll
      for (int kk = 0; kk < m; ++kk) part[kk] = part[kk] + part[kk + m];
    dq_d = half_sum(part[0]);
  }
  const float l2 = qv ? LSE[(size_t)bh * N + row0 + qi] * kLog2e : INFINITY;
  if (!qv) dq_d = 0.0f;
  if (h == 0 && (VARLEN ? qv : row0 + qi < Npad)) {
    lse2[(size_t)bh * Npad + row0 + qi] = l2;
    dvec[(size_t)bh * Npad + row0 + qi] = -dq_d;
  }

  // Per-lane LDS offsets: K / V rows (A operands of Sᵀ, dPᵀ) and the Kᵀ
  // transpose reads (A operand of dQᵀ).
  int koff[KD];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) koff[kk] = tile_off<D>(c, 2 * kk + h);
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_sub = (lane & 1) * 8;
  int toff[2][DT];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) toff[hf][dt] = tile_off<D>(tr_row + 8 * hf, 4 * dt + tr_chunk) + tr_sub;

  const int kv_end = CAUSAL ? min(L, q_start + kDqBM) : L;
  const int n_kv = (kv_end + kDqBN - 1) / kDqBN;
  const int first_masked = CAUSAL ? min(q_start / kDqBN, L / kDqBN) : L / kDqBN;

  int ld_off[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int r = (wave * LOADS + i) * (1024 / RB) + lane / (RB / 16);
    ld_off[i] = r * RB + swz_chunk_rb<RB>(r, lane % (RB / 16)) * 16;
  }
  auto gload = [&](int j, int slot) __device__ {
    const int key0 = j * kDqBN;
    buffer_to_lds<LOADS>(Kh + (size_t)key0 * D, (L - key0) * RB, k_lds + slot * TILE, ld_off,
                         wave * LOADS);
    buffer_to_lds<LOADS>(Vh + (size_t)key0 * D, (L - key0) * RB, v_lds + slot * TILE, ld_off,
                         wave * LOADS);
  };

  f32x16 dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x16{};

  // jn: the next key tile in processing order (j + 1 without a block mask).
  auto iteration = [&](int j, int jn, auto parity_tag, auto masked_tag) __device__ {
    constexpr int PAR = decltype(parity_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    if (jn < n_kv) gload(jn, PAR ^ 1);
    const char* kt = k_lds + PAR * TILE;
    const char* vt = v_lds + PAR * TILE;
    const int key0 = j * kDqBN;
    // Program-order pieces with LDS operand reads kLeadB MFMAs ahead: Sᵀ, dPᵀ
    // of keys 0..31, their dS; Sᵀ, dPᵀ of keys 32..63, their dS; then dQᵀ.
    // (Two waves share each SIMD: the other wave's MFMAs cover this wave's
    // dS steps, which keeps only one key half's scores live.)
    constexpr int NR = 4 * KD;  // piece i: key half t = i/(2KD), kk = (i/2)%KD, S or dP by i%2
    auto sread = [&](int i) __device__ {
      const int t = i / (2 * KD), kk = (i / 2) % KD;
      return *(const bf16x8*)((i % 2 ? vt : kt) + t * 32 * RB + koff[kk]);
    };
    // dS of one element pair (registers 2x, 2x+1 of key half t), packed.
    i32x4 dw[4];
    auto ds_step = [&](const f32x16& sv, const f32x16& dpv, int t, int x) __device__ {
      float ds[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int r = 2 * x + b;
        float p = exp2_hw(fmaf(sv[r], c_log2, -l2));
        if (MASKED) {
          const int key = key0 + t * 32 + acc_row(r, h);
          if (key >= L || (CAUSAL && key > qi)) p = 0.0f;
        }
        ds[b] = p * (dpv[r] - dq_d);
      }
      dw[2 * t + x / 4][x % 4] = (int)pack_bf16x2(ds[0], ds[1]);
    };
    bf16x8 ra[NR];
#pragma unroll
    for (int i = 0; i < kLeadB; ++i) ra[i] = sread(i);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x16 sd[2];  // S, dP of key half t
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 2 * KD * t; i < 2 * KD * (t + 1); ++i) {
        const int kk = (i / 2) % KD, w = i % 2;
        sd[w] = mfma32(ra[i], w ? dor[kk] : qr[kk], kk == 0 ? f32x16{} : sd[w]);
        if (i + kLeadB < NR) ra[i + kLeadB] = sread(i + kLeadB);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) ds_step(sd[0], sd[1], t, x);
    }
    // dQᵀ += Kᵀ·dSᵀ: Kᵀ operands by transpose reads of the K tile.
    constexpr int NT = 4 * DT;  // piece i: step ks = i/DT, d tile i%DT
    bf16x4 ta[NT][2];
    auto tread = [&](int i) __device__ {
      const char* base = kt + 16 * (i / DT) * RB;
      ta[i][0] = lds_read_tr16(base + toff[0][i % DT]);
      ta[i][1] = lds_read_tr16(base + toff[1][i % DT]);
    };
#pragma unroll
    for (int i = 0; i < kLeadB; ++i) tread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int ks = i / DT, dt = i % DT;
      dq[dt] = mfma32(concat(ta[i][0], ta[i][1]), __builtin_bit_cast(bf16x8, dw[ks]), dq[dt]);
      if (i + kLeadB < NT) tread(i + kLeadB);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmem();
    __syncthreads();
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if constexpr (!SPARSE) {
    gload(0, 0);
    wait_vmem();
    __syncthreads();
    int j = 0;
    for (; j + 1 < first_masked; j += 2) {
      iteration(j, j + 1, I0{}, std::false_type{});
      iteration(j + 1, j + 2, I1{}, std::false_type{});
    }
    for (; j < n_kv; ++j) {
      if (j & 1) iteration(j, j + 1, I1{}, std::integral_constant<bool, true>{});
      else iteration(j, j + 1, I0{}, std::integral_constant<bool, true>{});
    }
  } else {
    // Only the key tiles of the blocks this query block sees (its row of the
    // mask); slots alternate by position. A block row that sees nothing
    // keeps dQ = 0.
    uint64_t mb[kMaskWords];
    const int nb = (N + kMaskBlockRows - 1) / kMaskBlockRows;
    load_mask_bits(bmask + bh * mask_stride + (long)qt * nb, 1, nb, lane, mb);
    int a = next_mask_tile(mb, 0, n_kv);
    if (a < n_kv) {
      gload(a, 0);
      wait_vmem();
      __syncthreads();
      int b = next_mask_tile(mb, a + 1, n_kv);
      for (int pos = 0; a < n_kv; ++pos) {
        if (pos & 1) {
          if (a >= first_masked) iteration(a, b, I1{}, std::true_type{});
          else iteration(a, b, I1{}, std::false_type{});
        } else {
          if (a >= first_masked) iteration(a, b, I0{}, std::true_type{});
          else iteration(a, b, I0{}, std::false_type{});
        }
        a = b;
        b = next_mask_tile(mb, b + 1, n_kv);
      }
    }
  }

  // Epilogue: dQ = scale·dQᵀ (lane holds d = 32dt + 8(r/4) + 4h + r%4).
  if (qv) {
    bf16* row = dQ + head + (size_t)qi * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        i32x2 w;
        w[0] = (int)pack_bf16x2(dq[dt][4 * g] * scale, dq[dt][4 * g + 1] * scale);
        w[1] = (int)pack_bf16x2(dq[dt][4 * g + 2] * scale, dq[dt][4 * g + 3] * scale);
        *(i32x2*)(row + 32 * dt + 8 * g + 4 * h) = w;
      }
  }
}

// Launch variants: dense, packed segments (varlen) or block mask.
enum { BWD_DENSE = 0, BWD_VARLEN = 1, BWD_SPARSE = 2 };
struct BwdAux {
  const int* cu = nullptr;
  int nseq = 1;
  int max_len = 0;
  const uint8_t* bmask = nullptr;
  long mask_stride = 0;
};

template <int D, bool CAUSAL, int MODE>
static hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               float* dvec, float* lse2, int BH, int N, float scale,
                               const BwdAux& x, hipStream_t stream) {
  constexpr bool VARLEN = MODE == BWD_VARLEN, SPARSE = MODE == BWD_SPARSE;
  const int Npad = (N + kBwdRowPad - 1) / kBwdRowPad * kBwdRowPad;
  const int len = VARLEN ? x.max_len : N;  // longest sequence the grid covers
  const int units = BH * (VARLEN ? x.nseq : 1);
  {
    // dQ, and the row statistics D and lse2 that the dK/dV kernel reads.
    const int n_qtiles = (len + kDqBM - 1) / kDqBM;
    const dim3 grid(n_qtiles * units);
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, VARLEN, SPARSE>), grid, dim3(256), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout,
                       (const bf16*)o, lse, lse2, dvec, (bf16*)dq, N, Npad, BH, n_qtiles,
                       scale * kLog2e, scale, x.cu, x.nseq, x.bmask, x.mask_stride);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int n_kvtiles = (len + kBwdBN - 1) / kBwdBN;
    const dim3 grid(n_kvtiles * units);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, VARLEN, SPARSE>), grid, dim3(256), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout,
                       (const float*)lse2, (const float*)dvec, (bf16*)dk, (bf16*)dv, N,
                       Npad, BH, n_kvtiles, scale * kLog2e, scale, x.cu, x.nseq, x.bmask,
                       x.mask_stride);
  }
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_bwd_m(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               float* dvec, float* lse2, int BH, int N, int d, bool causal,
                               float scale, const BwdAux& x, hipStream_t stream) {
  if (d == 64) {
    return causal ? launch_bwd_t<64, true, MODE>(q, k, v, o, lse, dout, dq, dk, dv, dvec, lse2, BH, N, scale, x, stream)
                  : launch_bwd_t<64, false, MODE>(q, k, v, o, lse, dout, dq, dk, dv, dvec, lse2, BH, N, scale, x, stream);
  }
  return causal ? launch_bwd_t<128, true, MODE>(q, k, v, o, lse, dout, dq, dk, dv, dvec, lse2, BH, N, scale, x, stream)
                : launch_bwd_t<128, false, MODE>(q, k, v, o, lse, dout, dq, dk, dv, dvec, lse2, BH, N, scale, x, stream);
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* dvec, float* lse2, int B, int H, int N, int d, bool causal,
                           float scale, hipStream_t stream) {
  return launch_bwd_m<BWD_DENSE>(q, k, v, o, lse, dout, dq, dk, dv, dvec, lse2, B * H, N, d,
                                 causal, scale, BwdAux{}, stream);
}

hipError_t launch_bwd_bf16_varlen(const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, const void* dout, void* dq, void* dk,
                                  void* dv, float* dvec, float* lse2, const int* cu_seqlens,
                                  int nseq, int max_seqlen, int B, int H, int N, int d,
                                  bool causal, float scale, hipStream_t stream) {
  BwdAux x;
  x.cu = cu_seqlens;
  x.nseq = nseq;
  x.max_len = max_seqlen;
  return launch_bwd_m<BWD_VARLEN>(q, k, v, o, lse, dout, dq, dk, dv, dvec, lse2, B * H, N, d,
                                  causal, scale, x, stream);
}

hipError_t launch_bwd_bf16_blocksparse(const void* q, const void* k, const void* v,
                                       const void* o, const float* lse, const void* dout,
                                       void* dq, void* dk, void* dv, float* dvec, float* lse2,
                                       const uint8_t* block_mask, bool per_head, int B, int H,
                                       int N, int d, bool causal, float scale,
                                       hipStream_t stream) {
  BwdAux x;
  x.bmask = block_mask;
  const long nb = (N + kMaskBlockRows - 1) / kMaskBlockRows;
  x.mask_stride = per_head ? nb * nb : 0;
  return launch_bwd_m<BWD_SPARSE>(q, k, v, o, lse, dout, dq, dk, dv, dvec, lse2, B * H, N, d,
                                  causal, scale, x, stream);
}

}  // namespace fattn
