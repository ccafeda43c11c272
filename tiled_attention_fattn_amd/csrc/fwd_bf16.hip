// Fused attention forward, bf16 in/out, fp32 accumulation, for gfx950.
//
// What is computed (FlashAttention-4 news page, "Por qué el enfoque estándar
// ya no funciona"; FlashAttention-3 page, "FlashAttention y FlashAttention-2"):
// O = softmax(scale·Q·Kᵀ [causal]) · V, one workgroup per block of query rows of
// one head; K and V stream through LDS in 64-key tiles; the scores and the
// probabilities never leave the compute unit.
//
// Layout inside a workgroup (32 queries per wave; 8 waves for plain
// non-causal attention, one workgroup per compute unit, or 4 waves and two
// workgroups per compute unit otherwise; either way each SIMD holds two
// waves whose VALU and MFMA phases interleave):
//  * Sᵀ = K·Qᵀ on 32x32x16 bf16 MFMA: the accumulator column is the query,
//    so each lane owns one query row and the row reductions are in-lane plus
//    one exchange between the two lane halves. K comes from LDS, Q stays in
//    registers for the whole loop.
//  * Oᵀ += Vᵀ·Pᵀ on the same MFMA: Pᵀ is taken straight from the Sᵀ
//    accumulator registers (the k order inside a 16-key step is free as long
//    as the Vᵀ operand uses the same order); Vᵀ comes from the row-major V tile
//    through the LDS transpose read.
//  * Software pipeline over 64-key tiles: the exponentials of tile j run
//    beside the MFMAs of S(j+1), then PV(j) (FlashAttention-4 news page,
//    "Cómo Together AI resolvió el problema": overlap the tensor units, the
//    exponential units and memory). The loop body is written in program
//    order as pieces of one MFMA each between scheduling fences: every piece
//    issues the LDS operand read of the MFMA three pieces ahead, and each S
//    piece also carries its share of the softmax of tile j, so neither an
//    MFMA's operand latency nor the exponentials stall the MFMA pipe.
//  * Online softmax in the exp2 domain with conditional rescaling
//    (FlashAttention-4 gist, technical summary 2.B): the exponent offset
//    moves only when a tile's probabilities would exceed 2^τ, detected from
//    the tile's row sum (see guard below), so the common tile needs neither
//    a row max nor a rescale of Oᵀ and l. Exact, because the same offset is
//    used for O, l and LSE.
//  * Row sums are accumulated in fp32 from the probabilities before their
//    rounding to bf16 for the PV product.
//  * K/V tiles stream into LDS by buffer loads that write LDS directly,
//    double-buffered and issued an iteration ahead (FlashAttention-3 page,
//    innovation 2: loads hidden behind compute).
//  * Causal: key tiles past the workgroup's last query are never loaded; the
//    element mask is applied only on tiles that cross the diagonal.
//  * Packed variable-length sequences (VARLEN): the grid runs over (head,
//    segment, query tile) and each workgroup works on its segment as on a
//    sequence of its own (base rows offset to the segment start, length =
//    the segment's), so no tile ever mixes two segments.
//  * Block masks (SPARSE): each workgroup is one 128-query block; it reads
//    its row of the 128×128-block mask once (as 64-bit ballots) and runs the
//    same schedule over the visible 64-key tiles only.
#include <algorithm>
#include <type_traits>

#include "fattn_device.hpp"
#include "fattn_launch.h"

namespace fattn {

constexpr int kFwdQW = 32;                  // queries per wave
// Waves per workgroup (WAVES): 4 (128 queries, two workgroups per compute
// unit), or 8 (256 queries sharing every K/V tile, one workgroup per compute
// unit), which halves the bytes the tile loads write into LDS per MFMA. The
// launch picks 8 only for plain non-causal attention with d = 128 and
// N >= 4096: under the causal mask the diagonal work grows with the query
// block, and for d = 64 or shorter sequences the halved workgroup count
// costs more than it saves (measured).
constexpr int kFwdWideMinN = 4096;
// d = 64 needs 168 vector registers per lane, so three waves fit on each SIMD
// (three 4-wave workgroups per compute unit, 96 KB of LDS); d = 128 needs 256.
constexpr int kFwdBN = 64;                  // keys per K/V tile
constexpr float kRescaleTau = 8.0f;         // log2 units: P̃ ≤ 2^8 between rescales
constexpr float kSumGuard = 256.0f;         // 2^kRescaleTau
constexpr int kLead = 3;                    // LDS operand reads in flight ahead of the MFMAs
constexpr int kMaskBlock = kMaskBlockRows;  // block-mask granularity (queries and keys)
// Causal issue groups (see the workgroup mapping): used for d = 128 when a
// unit has between these many query tiles. Longer sequences reuse each K/V
// tile across enough query tiles that cache locality between them no longer
// matters, very short ones have too little K/V for it to matter, and at
// d = 64 (three workgroups per compute unit) the groups were slower (all
// measured).
constexpr int kCausalGroupMinTiles = 4, kCausalGroupMaxTiles = 16;


// Running softmax state of one 32-query sub-tile (per lane: one query).
template <int DT>
struct SubTile {
  f32x16 o[DT];
  float m_c;     // exponent offset in use (log2 domain)
  float l_part;  // this lane half's share of the row sum
};

// Masks the scores of a 64-key tile for ragged N and the causal diagonal.
template <bool CAUSAL>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int key0, int N, int qi, int h) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + t * 32 + acc_row(r, h);
      if (key >= N || (CAUSAL && key > qi)) s[t][r] = -INFINITY;
    }
}

// P̃ = 2^(s·c − m_c) packed to bf16 in the Pᵀ operand layout (slot e of
// step ks: key 16ks + 8(e/4) + 4h + e%4). Returns this lane half's fp32 sum
// of P̃ (taken before the rounding to bf16, so the LSE keeps fp32 accuracy).
template <int EXPM>
__device__ __forceinline__ float softmax_exp(const f32x16 (&s)[2], float c_log2, float m_c,
                                             bf16x8 (&p)[4]) {
  float la = 0.0f, lb = 0.0f;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      i32x4 packed;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // SPLIT: the pair e = 3 of every group of four goes to the polynomial.
        constexpr int M = EXPM == EXP_SPLIT ? EXP_HW : EXPM;
        const float x0 = fmaf(s[t][half * 8 + 2 * e], c_log2, -m_c);
        const float x1 = fmaf(s[t][half * 8 + 2 * e + 1], c_log2, -m_c);
        const float p0 = (EXPM == EXP_SPLIT && e == 3) ? exp2_poly(x0) : exp2_sel<M>(x0);
        const float p1 = (EXPM == EXP_SPLIT && e == 3) ? exp2_poly(x1) : exp2_sel<M>(x1);
        la += p0;
        lb += p1;
        packed[e] = (int)pack_bf16x2(p0, p1);
      }
      p[2 * t + half] = __builtin_bit_cast(bf16x8, packed);
    }
  return la + lb;
}

// One element pair x (0..15) of softmax_exp: tile t = x/8, register half
// (x/4)%2, pair e = x%4; same arithmetic, for interleaving with MFMAs.
template <int EXPM>
__device__ __forceinline__ void softmax_exp_pair(const f32x16 (&s)[2], float c_log2, float m_c,
                                                 int x, i32x4 (&pk)[4], float& la, float& lb) {
  const int t = x / 8, half = (x / 4) % 2, e = x % 4;
  constexpr int M = EXPM == EXP_SPLIT ? EXP_HW : EXPM;
  const float x0 = fmaf(s[t][half * 8 + 2 * e], c_log2, -m_c);
  const float x1 = fmaf(s[t][half * 8 + 2 * e + 1], c_log2, -m_c);
  const float p0 = (EXPM == EXP_SPLIT && e == 3) ? exp2_poly(x0) : exp2_sel<M>(x0);
  const float p1 = (EXPM == EXP_SPLIT && e == 3) ? exp2_poly(x1) : exp2_sel<M>(x1);
  la += p0;
  lb += p1;
  pk[2 * t + half][e] = (int)pack_bf16x2(p0, p1);
}

template <int D, bool CAUSAL, int EXPM, bool VARLEN, bool SPARSE, int WAVES>
__global__ __launch_bounds__(64 * WAVES)
__attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2, D == 64 ? 3 : 2)))
void fwd_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                     const bf16* __restrict__ V, bf16* __restrict__ O, float* __restrict__ LSE,
                     int N, int BH, int n_qtiles, float c_log2, const int* __restrict__ cu,
                     int nseq, const uint8_t* __restrict__ bmask, long mask_stride,
                     int group_units) {
  static_assert(!(VARLEN && SPARSE), "block masks apply to whole sequences");
  static_assert(WAVES == 4 || (WAVES == 8 && !CAUSAL && !VARLEN && !SPARSE),
                "eight waves only for plain non-causal attention");
  constexpr int kFwdWaves = WAVES;
  constexpr int kFwdBM = kFwdQW * kFwdWaves;  // query rows per workgroup
  static_assert(!SPARSE || kFwdBM == kMaskBlock, "one query tile per mask block row");
  constexpr int KD = D / 16;          // MFMA k-steps over the head dimension
  constexpr int RB = D * 2;           // bytes per K/V row
  constexpr int TILE = kFwdBN * RB;
  constexpr int NS = kFwdBN / 16;     // 16-key PV steps
  constexpr int DT = D / 32;          // 32-wide output tiles over d
  // LDS: K slots 0, 1 then V slots 0, 1.
  __shared__ __attribute__((aligned(16))) char lds[4 * TILE];
  char* const k_lds = lds;
  char* const v_lds = lds + 2 * TILE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int h = lane >> 5, c = lane & 31;

  // Workgroup → (head[, segment], query tile).
  //  * Causal: tile-major from the last query tile down, so the heaviest
  //    tiles (a tile's work grows with its index) of every head and segment
  //    are issued before any lighter one, longest-processing-time first
  //    (within a group of units, below); consecutive ids run round-robin over
  //    the XCDs, so (with a multiple of 8 units) an XCD keeps the same
  //    (head, segment) units from tile to tile.
  //  * Packed segments without the mask: longest segment first (every tile
  //    of a segment costs its length): the workgroup's rank r picks the r-th
  //    longest segment, heads interleaved within a rank.
  //  * Otherwise the remap gives each XCD a contiguous run of tiles so the
  //    tiles of one head share that XCD's L2.
  int unit, qt;
  if constexpr (CAUSAL) {
    // Units are issued in groups of group_units (chosen by the launch), each
    // group tile-major as above: for short sequences one group fills the
    // resident workgroups once, so the few units on each XCD keep their K
    // and V in its L2 while all their tiles run.
    const int units = BH * (VARLEN ? nseq : 1);
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
    unit = b * nseq + segment_of_rank(cu, nseq, N, r, lane);
  } else {
    const int total = n_qtiles * BH;
    int logical = blockIdx.x;
    if ((total & 7) == 0) logical = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    unit = logical / n_qtiles;
    qt = logical - unit * n_qtiles;
  }
  const int bh = VARLEN ? unit / nseq : unit;
  // Rows [row0, row0 + L) of the head: the whole head, or one segment (its
  // offsets clamped to [0, N] so that no offset can address outside the head).
  int row0 = 0, L = N;
  if constexpr (VARLEN) {
    const int sg = unit - bh * nseq;
    row0 = min(max(cu[sg], 0), N);
    L = min(max(cu[sg + 1], row0), N) - row0;
  }
  const int q_start = qt * kFwdBM;
  if (q_start >= L) return;  // whole workgroup: a segment shorter than the grid's longest

  const size_t head = ((size_t)bh * N + row0) * D;
  const bf16* Qh = Q + head;
  const bf16* Kh = K + head;
  const bf16* Vh = V + head;
  const int q0 = q_start + wave * kFwdQW;
  const int qi = q0 + c;  // this lane's query

  // Qᵀ operand: lane holds Q[qi][16kk + 8h + 0..7].
  bf16x8 qr[KD];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk)
    qr[kk] = qi < L ? *(const bf16x8*)(Qh + (size_t)qi * D + kk * 16 + 8 * h) : bf16x8{};

  // Per-lane LDS offsets, constant over the loop (the swizzle depends on the
  // row only through bits that do not change between the 32-row tiles or the
  // 16-row PV steps).
  int koff[KD];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) koff[kk] = tile_off<D>(c, 2 * kk + h);
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_sub = (lane & 1) * 8;
  int voff[2][DT];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      voff[hf][dt] = tile_off<D>(tr_row + 8 * hf, 4 * dt + tr_chunk) + tr_sub;

  const int kv_end = CAUSAL ? min(L, q_start + kFwdBM) : L;
  const int n_kv = (kv_end + kFwdBN - 1) / kFwdBN;
  // First tile whose scores need the element mask (ragged end or diagonal).
  const int first_masked = CAUSAL ? min(q_start / kFwdBN, L / kFwdBN) : L / kFwdBN;

  // Global → LDS without staging registers: each wave moves 1 KB (64 lanes ×
  // 16 B) per load straight into LDS at a wave-uniform base. The source is a
  // buffer resource starting at the tile's first row and ending at row L (the
  // end of the sequence or segment), so rows past L read as zero (range
  // check) and the per-lane byte offset is a loop constant; the swizzle is
  // applied on the source side (the XOR swizzle is its own inverse).
  constexpr int ROWS_PER_LOAD = 1024 / RB;          // rows per 1 KB wave load
  constexpr int LOADS = TILE / 1024 / kFwdWaves;    // wave loads per tensor per tile
  int ld_off[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int r = (wave * LOADS + i) * ROWS_PER_LOAD + lane / (RB / 16);
    ld_off[i] = r * RB + swz_chunk_rb<RB>(r, lane % (RB / 16)) * 16;
  }
  auto gload = [&](const bf16* src, char* dst_tile, int j) __device__ {
    const int key0 = j * kFwdBN;
    buffer_to_lds<LOADS>(src + (size_t)key0 * D, (L - key0) * RB, dst_tile, ld_off, wave * LOADS);
  };

  SubTile<DT> st;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) st.o[dt] = f32x16{};
  st.l_part = 0.0f;

  auto scores = [&](const char* kt, f32x16 (&s)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KD; ++kk)
        s[t] = mfma32(*(const bf16x8*)(kt + t * 32 * RB + koff[kk]), qr[kk], s[t]);
    }
  };
  auto tile_max = [&](const f32x16 (&s)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    return half_max(mx) * c_log2;
  };

  // Key tiles in processing order: all of [0, n_kv), or under a block mask
  // only those whose 128-key block is visible to this 128-query block (the
  // workgroup's row of the mask; a tile of 64 keys lies in block j/2). The
  // row is read once into four 64-bit ballots (up to 256 blocks), so the
  // walk over it is scalar work that waits on no memory.
  uint64_t mb[kMaskWords] = {};
  if constexpr (SPARSE) {
    const int nb = (N + kMaskBlock - 1) / kMaskBlock;
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
      if (h == 0) LSE[(size_t)bh * N + row0 + qi] = -INFINITY;
    }
    return;
  }

  // Prologue: K(c0), K(c1), V(c0) in flight; S(c0); running max from it.
  // The second barrier lets the first iteration refill K slot 0 only once
  // every wave has read K(c0) from it.
  gload(Kh, k_lds, c0);
  if (c1 < n_kv) gload(Kh, k_lds + TILE, c1);
  gload(Vh, v_lds, c0);
  wait_vmem();
  __syncthreads();
  f32x16 s[2];
  scores(k_lds, s);
  if (c0 >= first_masked) mask_tile<CAUSAL>(s, c0 * kFwdBN, L, qi, h);
  st.m_c = tile_max(s);
  __syncthreads();

  // Conditional rescale (FlashAttention-4 gist, technical summary 2.B). The
  // offset m_c stays put while every P̃ of a tile is at most 2^τ. A lane
  // half's tile sum bounds each of its P̃, so the test needs neither the row
  // max nor the scores once the exponentials are taken: only when some sum
  // exceeds 2^τ (rare once m_c is near the row max) does the wave take the
  // exact branch. That branch rebuilds S(j) bit for bit (same operands, same
  // accumulation order; K(j) is re-read from global memory because its LDS
  // slot already receives K(j+2)), moves m_c to the row max, rescales Oᵀ and
  // l and recomputes P̃(j).
  auto guard = [&](int j, bf16x8 (&p)[NS], float& lt) __device__ {
    if (__ballot(lt > kSumGuard)) {
      const int key0 = j * kFwdBN;
      f32x16 s[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int key = key0 + t * 32 + c;
        const bf16* krow = Kh + (size_t)min(key, L - 1) * D + 8 * h;
        s[t] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
          bf16x8 a = *(const bf16x8*)(krow + kk * 16);
          if (key >= L) a = bf16x8{};
          s[t] = mfma32(a, qr[kk], s[t]);
        }
      }
      if (j >= first_masked) mask_tile<CAUSAL>(s, key0, L, qi, h);
      const float m_new = fmaxf(st.m_c, tile_max(s));
      const float alpha = exp2_hw(st.m_c - m_new);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[dt][r] *= alpha;
      st.l_part *= alpha;
      st.m_c = m_new;
      lt = softmax_exp<EXPM>(s, c_log2, st.m_c, p);
    }
    st.l_part += lt;
  };

  // Iteration j: exp(S(j)) ∥ S(j+1) on the MFMA pipe, the guard, then PV(j),
  // laid out in program order as pieces of one MFMA each separated by
  // scheduling fences. Each piece issues the LDS operand read of the MFMA
  // kLead pieces ahead (the reads of the first PV MFMAs ride on the last S
  // pieces), so no MFMA waits for its own operand, and the S pieces carry
  // one element pair of the softmax of tile j each. The last iteration (no
  // tile j+1) is peeled.
  constexpr int NSP = 2 * KD;     // S pieces: key half t = i%2, k-step kk = i/2
  static_assert(16 % NSP == 0, "softmax pairs must spread evenly over the S pieces");
  constexpr int NPV = NS * DT;    // PV pieces: key step ks = i/DT, d tile dt = i%DT
  auto kread = [&](const char* kt, int i) __device__ {
    return *(const bf16x8*)(kt + (i % 2) * 32 * RB + koff[i / 2]);
  };
  auto vread = [&](const char* vt, int i, bf16x4 (&ta)[NPV][2]) __device__ {
    const char* base = vt + 16 * (i / DT) * RB;
    ta[i][0] = lds_read_tr16(base + voff[0][i % DT]);
    ta[i][1] = lds_read_tr16(base + voff[1][i % DT]);
  };
  // Tiles j (this iteration), jn and jn2 (the next two in processing order;
  // j + 1 and j + 2 without a block mask); PAR is the position's parity.
  auto iteration = [&](int j, int jn, int jn2, auto parity_tag, auto has_next_tag) __device__ {
    constexpr int PAR = decltype(parity_tag)::value;  // a compile-time slot index
    constexpr bool HAS_NEXT = decltype(has_next_tag)::value;
    // Loads for later iterations: K(jn2) into the K slot that held K(j)
    // (consumed by S(j) one iteration ago), V(jn) into the V slot that held
    // the previous tile's V (consumed by its PV one iteration ago).
    if constexpr (HAS_NEXT) {
      if (jn2 < n_kv) gload(Kh, k_lds + PAR * TILE, jn2);
      gload(Vh, v_lds + (PAR ^ 1) * TILE, jn);
    }
    const char* kt = k_lds + (PAR ^ 1) * TILE;
    const char* vt = v_lds + PAR * TILE;
    // An empty asm statement on the exponent offset at every call site, so
    // the exp2 arguments of this iteration are formed inside it: otherwise
    // the compiler forms them once above the branch between the last two
    // iterations and spills them, and each spill reload's wait on the
    // vector-memory counter also waits for the tile loads issued above.
    asm volatile("" : "+v"(st.m_c));
    i32x4 pk[4];
    float la = 0.0f, lb = 0.0f;
    f32x16 ns[2];
    bf16x4 ta[NPV][2];
    if constexpr (HAS_NEXT) {
      bf16x8 ra[NSP];
#pragma unroll
      for (int i = 0; i < kLead; ++i) ra[i] = kread(kt, i);
#pragma unroll
      for (int i = 0; i < NSP; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        // The two key halves alternate, so no MFMA waits for the one before.
        const int t = i % 2, kk = i / 2;
        ns[t] = mfma32(ra[i], qr[kk], kk == 0 ? f32x16{} : ns[t]);
        if (i + kLead < NSP) ra[i + kLead] = kread(kt, i + kLead);
        else vread(vt, i + kLead - NSP, ta);
        // 16 element pairs over the NSP pieces; each kept beside its MFMA
        // instead of sinking to its use.
#pragma unroll
        for (int x = i * 16 / NSP; x < (i + 1) * 16 / NSP; ++x) {
          softmax_exp_pair<EXPM>(s, c_log2, st.m_c, x, pk, la, lb);
          asm volatile("" ::"v"(pk[x / 4][x % 4]), "v"(la), "v"(lb));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (jn >= first_masked) mask_tile<CAUSAL>(ns, jn * kFwdBN, L, qi, h);
    } else {
#pragma unroll
      for (int i = 0; i < kLead; ++i) vread(vt, i, ta);
#pragma unroll
      for (int x = 0; x < 16; ++x) softmax_exp_pair<EXPM>(s, c_log2, st.m_c, x, pk, la, lb);
    }
    bf16x8 p[NS];
#pragma unroll
    for (int ks = 0; ks < NS; ++ks) p[ks] = __builtin_bit_cast(bf16x8, pk[ks]);
    float lt = la + lb;
    guard(j, p, lt);

    // PV(j): Vᵀ operands by transpose reads, kLead pieces ahead. The PV
    // pieces run at the lower wave priority: when the other wave of the SIMD
    // is in its S/softmax phase, that phase (VALU-heavy, with the loads) is
    // issued first and the PV MFMAs fill the matrix pipe around it.
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const int ks = i / DT, dt = i % DT;
      st.o[dt] = mfma32(concat(ta[i][0], ta[i][1]), p[ks], st.o[dt]);
      if (i + kLead < NPV) vread(vt, i + kLead, ta);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    if constexpr (HAS_NEXT) {
      s[0] = ns[0];
      s[1] = ns[1];
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

  // Epilogue: O = Oᵀ/l (lane holds d = 32dt + 8(r/4) + 4h + r%4 of its query).
  const float l = half_sum(st.l_part);
  const float inv = 1.0f / l;
  if (qi < L) {
    bf16* Orow = O + head + (size_t)qi * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        i32x2 w;
        w[0] = (int)pack_bf16x2(st.o[dt][4 * g] * inv, st.o[dt][4 * g + 1] * inv);
        w[1] = (int)pack_bf16x2(st.o[dt][4 * g + 2] * inv, st.o[dt][4 * g + 3] * inv);
        *(i32x2*)(Orow + 32 * dt + 8 * g + 4 * h) = w;
      }
    if (h == 0) LSE[(size_t)bh * N + row0 + qi] = (st.m_c + __builtin_log2f(l)) * kLn2;
  }
}

// Launch variants: dense, packed segments (varlen) or block mask.
enum { FWD_DENSE = 0, FWD_VARLEN = 1, FWD_SPARSE = 2 };
struct FwdAux {
  const int* cu = nullptr;  // varlen: segment offsets
  int nseq = 1;
  int max_len = 0;          // varlen: longest segment the grid covers
  const uint8_t* bmask = nullptr;  // block mask rows of 128 queries
  long mask_stride = 0;     // elements between the masks of consecutive heads (0: shared)
};

template <int D, bool CAUSAL, int EXPM, int MODE, int WAVES>
static hipError_t launch_fwd_w(const void* q, const void* k, const void* v, void* o, float* lse,
                               int BH, int N, float scale, const FwdAux& x, hipStream_t stream) {
  constexpr int bm = kFwdQW * WAVES;
  const auto kernel =
      fwd_bf16_kernel<D, CAUSAL, EXPM, MODE == FWD_VARLEN, MODE == FWD_SPARSE, WAVES>;
  const int n_qtiles = ((MODE == FWD_VARLEN ? x.max_len : N) + bm - 1) / bm;
  const int units = BH * (MODE == FWD_VARLEN ? x.nseq : 1);
  int group_units = units;
  if constexpr (CAUSAL) {
    // One group = the workgroups the device keeps resident (queried once per
    // kernel instance), rounded down to whole units, a multiple of 8 (the
    // XCD count) so that each XCD holds the same units from tile to tile.
    static const int resident = [kernel] {
      int occ = 0, dev = 0, cus = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, 64 * WAVES, 0) !=
              hipSuccess ||
          hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
      }
      return occ * cus;
    }();
    if (D == 128 && n_qtiles >= kCausalGroupMinTiles && n_qtiles <= kCausalGroupMaxTiles &&
        resident > 0)
      group_units = std::max(8, resident / n_qtiles / 8 * 8);
  }
  hipLaunchKernelGGL(kernel, dim3(n_qtiles * units), dim3(64 * WAVES), 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, N, BH,
                     n_qtiles, scale * kLog2e, x.cu, x.nseq, x.bmask, x.mask_stride,
                     group_units);
  return hipGetLastError();
}

template <int D, bool CAUSAL, int EXPM, int MODE>
static hipError_t launch_fwd_t(const void* q, const void* k, const void* v, void* o, float* lse,
                               int BH, int N, float scale, const FwdAux& x, hipStream_t stream) {
  if constexpr (D == 128 && !CAUSAL && MODE == FWD_DENSE) {
    if (N >= kFwdWideMinN)
      return launch_fwd_w<D, CAUSAL, EXPM, MODE, 8>(q, k, v, o, lse, BH, N, scale, x, stream);
  }
  return launch_fwd_w<D, CAUSAL, EXPM, MODE, 4>(q, k, v, o, lse, BH, N, scale, x, stream);
}

template <int D, bool CAUSAL, int MODE>
static hipError_t launch_fwd_e(const void* q, const void* k, const void* v, void* o, float* lse,
                               int BH, int N, float scale, int exp_mode, const FwdAux& x,
                               hipStream_t stream) {
  if (exp_mode == EXP_POLY)
    return launch_fwd_t<D, CAUSAL, EXP_POLY, MODE>(q, k, v, o, lse, BH, N, scale, x, stream);
  if (exp_mode == EXP_SPLIT)
    return launch_fwd_t<D, CAUSAL, EXP_SPLIT, MODE>(q, k, v, o, lse, BH, N, scale, x, stream);
  return launch_fwd_t<D, CAUSAL, EXP_HW, MODE>(q, k, v, o, lse, BH, N, scale, x, stream);
}

template <int MODE>
static hipError_t launch_fwd_m(const void* q, const void* k, const void* v, void* o, float* lse,
                               int BH, int N, int d, bool causal, float scale, int exp_mode,
                               const FwdAux& x, hipStream_t stream) {
  if (d == 64) {
    return causal ? launch_fwd_e<64, true, MODE>(q, k, v, o, lse, BH, N, scale, exp_mode, x, stream)
                  : launch_fwd_e<64, false, MODE>(q, k, v, o, lse, BH, N, scale, exp_mode, x, stream);
  }
  return causal ? launch_fwd_e<128, true, MODE>(q, k, v, o, lse, BH, N, scale, exp_mode, x, stream)
                : launch_fwd_e<128, false, MODE>(q, k, v, o, lse, BH, N, scale, exp_mode, x, stream);
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, bool causal, float scale, int exp_mode,
                           hipStream_t stream) {
  return launch_fwd_m<FWD_DENSE>(q, k, v, o, lse, B * H, N, d, causal, scale, exp_mode, FwdAux{},
                                 stream);
}

hipError_t launch_fwd_bf16_varlen(const void* q, const void* k, const void* v, void* o,
                                  float* lse, const int* cu_seqlens, int nseq, int max_seqlen,
                                  int B, int H, int N, int d, bool causal, float scale,
                                  int exp_mode, hipStream_t stream) {
  FwdAux x;
  x.cu = cu_seqlens;
  x.nseq = nseq;
  x.max_len = max_seqlen;
  return launch_fwd_m<FWD_VARLEN>(q, k, v, o, lse, B * H, N, d, causal, scale, exp_mode, x,
                                  stream);
}

hipError_t launch_fwd_bf16_blocksparse(const void* q, const void* k, const void* v, void* o,
                                       float* lse, const uint8_t* block_mask, bool per_head,
                                       int B, int H, int N, int d, bool causal, float scale,
                                       int exp_mode, hipStream_t stream) {
  FwdAux x;
  x.bmask = block_mask;
  const long nb = (N + kMaskBlock - 1) / kMaskBlock;
  x.mask_stride = per_head ? nb * nb : 0;
  return launch_fwd_m<FWD_SPARSE>(q, k, v, o, lse, B * H, N, d, causal, scale, exp_mode, x,
                                  stream);
}

}  // namespace fattn
