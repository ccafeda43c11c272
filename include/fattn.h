/*
 * libfattn — fused exact attention for AMD Instinct MI355X (gfx950).
 *
 * Computes O = softmax(scale · Q·Kᵀ [causal mask]) · V tile by tile with an
 * online softmax, keeps the N×N score matrix on chip, saves the per-row
 * log-sum-exp, and forms dQ, dK, dV in the backward pass by recomputing P
 * from that log-sum-exp. An fp8 forward rotates Q and K with a random-sign
 * Hadamard matrix before e4m3 quantisation ("incoherent processing").
 *
 * Sources (web pages describing the method):
 *  - "FlashAttention-4: cómo Together AI aceleró la atención en GPU
 *    Blackwell" (news.hamidun.com) — section "Por qué el enfoque estándar ya
 *    no funciona": the problem is the two products S = Q·Kᵀ and O = P·V with
 *    a softmax between them.
 *  - "FlashAttention-3 (ES)" (systems-analysis.ru) — "FlashAttention y
 *    FlashAttention-2": tiling into on-chip memory and fusion, so no
 *    intermediate reaches global memory; innovation 3: fp8 with incoherent
 *    processing by a random orthogonal (Hadamard) matrix.
 *  - "FlashAttention-4: Algorithm and Kernel Pipelining Co-Design for
 *    Asymmetric Hardware Scaling" (gist.science) — technical summary 2.B
 *    (software exp2 on FMA units, conditional rescaling past a threshold),
 *    2.C (backward: dS, dQ and global atomic reductions); the Portuguese
 *    summary of the same paper, "Significado e Impacto", names variable-length
 *    (varlen) attention as a variant the design enables.
 *
 * Conventions for every entry point
 *  - Tensors are device pointers to contiguous [B, H, N, d] arrays (d fastest)
 *    of bfloat16 (2-byte storage) unless stated otherwise; LSE and the
 *    backward statistics are float32 [B, H, N]. Every pointer must be 16-byte
 *    aligned. The caller owns all memory; the library never allocates device
 *    memory and never synchronises.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    asynchronously; the return value is the enqueue status only. Device
 *    faults surface at the caller's next synchronisation.
 *  - Supported: B, H, N ≥ 1 with B·H·N·d < 2^31 elements per tensor,
 *    d ∈ {64, 128}, any N (ragged tails are masked), causal ∈ {0, 1} with the
 *    reading that key j is visible to query i iff j ≤ i, finite scale > 0.
 *  - All argument checks run on the host before any HIP call, so a rejected
 *    call has no effect on the device.
 *  - Calls are re-entrant; concurrent calls that share output or workspace
 *    buffers race.
 */
#ifndef FATTN_H
#define FATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FATTN_OK = 0,
  FATTN_EINVAL = 1,      /* null/misaligned pointer, B/H/N < 1, bad scale, bad flag */
  FATTN_ENOTSUP = 2,     /* d not in {64, 128}; tensor too large for 32-bit indexing */
  FATTN_EWORKSPACE = 3,  /* workspace pointer null or smaller than required */
  FATTN_EHIP = 4,        /* a HIP runtime call failed; see fattn_last_error() */
  FATTN_EDEVICE = 5      /* the current device is not gfx950 */
} fattn_status;

/* Which exp2 the softmax uses (the bf16 and fp8 forward kernels). */
typedef enum {
  FATTN_EXP_AUTO = 0,    /* the variant measured fastest on gfx950: hardware,
                            for both forwards and both head dimensions */
  FATTN_EXP_HW = 1,      /* v_exp_f32 on the transcendental unit */
  FATTN_EXP_POLY = 2,    /* Cody–Waite split + degree-3 polynomial on FMA units */
  FATTN_EXP_SPLIT = 3    /* a static quarter of the exponentials (one in four
                            element pairs) on the polynomial, the rest on
                            the hardware unit */
} fattn_exp_mode;

/*
 * Forward, bfloat16 in and out.
 *   q, k, v  [B,H,N,d] bf16 inputs.
 *   o        [B,H,N,d] bf16 output, O = softmax(scale·Q·Kᵀ [mask])·V,
 *            rounded to nearest even.
 *   lse      [B,H,N] fp32 output, natural-log log-sum-exp of the masked,
 *            scaled scores of each row (required: the backward consumes it).
 *   exp_mode one of fattn_exp_mode.
 * The softmax keeps an exponent offset and an fp32 row sum per row and
 * rescales the partial output only when some probability of a tile would
 * exceed 2^8 relative to the offset in use (FlashAttention-4 gist,
 * technical summary 2.B), which is exact.
 */
fattn_status fattn_fwd(const void* q, const void* k, const void* v, void* o,
                       float* lse, int B, int H, int N, int d, int causal,
                       float scale, int exp_mode, void* stream);

/*
 * Backward, bfloat16 in and out, from the forward's saved O and LSE.
 *   dout        [B,H,N,d] bf16 upstream gradient dO.
 *   dq, dk, dv  [B,H,N,d] bf16 outputs.
 *   workspace   device memory of at least fattn_bwd_workspace_bytes(B,H,N,d)
 *               bytes, 256-byte aligned; contents on entry are ignored.
 *               Layout (Npad = N rounded up to 64): fp32 −D, D = rowsum(dO∘O),
 *               [B,H,Npad] at offset 0, then fp32 LSE·log2(e) [B,H,Npad]
 *               (padded rows: 0, +∞), each piece 256-byte aligned; with
 *               packed sequences (fattn_bwd_varlen) only the rows of the
 *               segments are written.
 * The gradients are the standard ones of the softmax attention (FlashAttention-4
 * gist, technical summary 2.C, names dS = P∘(dP − D) and the dQ reduction):
 * dV = Pᵀ·dO, dP = dO·Vᵀ, dS = P∘(dP − D), dQ = scale·dS·K, dK = scale·dSᵀ·Q,
 * with P recomputed from the saved LSE. That summary reduces dQ with global
 * atomics; here dK and dV are accumulated by the workgroup that owns their
 * key block and dQ by the workgroup that owns its query block (which
 * recomputes the scores): no global atomics, so all three gradients are
 * bitwise reproducible. Errors: EINVAL/ENOTSUP as fattn_fwd; EWORKSPACE for a
 * NULL, misaligned or too small workspace; EDEVICE, EHIP.
 */
size_t fattn_bwd_workspace_bytes(int B, int H, int N, int d);
fattn_status fattn_bwd(const void* q, const void* k, const void* v,
                       const void* o, const float* lse, const void* dout,
                       void* dq, void* dk, void* dv, int B, int H, int N, int d,
                       int causal, float scale, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * fattn_bwd without a workspace argument, for callers that cannot allocate
 * device memory: work recorded under graph capture, tight serving loops,
 * harnesses that forbid allocation. The row statistics live in a
 * library-owned static device buffer of FATTN_NOALLOC_WORKSPACE_BYTES bytes
 * per GPU (held from the first use on that GPU until the process ends, its
 * device address looked up on the first call on each device); the call
 * itself allocates nothing. Inputs, outputs and results as fattn_bwd.
 * Limits: fattn_bwd_workspace_bytes(B,H,N,d) must not exceed
 * FATTN_NOALLOC_WORKSPACE_BYTES (B·H·ceil(N/64)·64 <= 2^21 rows, e.g.
 * B·H = 64 at N = 32768), else FATTN_EWORKSPACE and nothing is launched.
 * Every call on one GPU shares that GPU's buffer: calls that overlap on one
 * GPU (other streams, other threads) race and give wrong gradients; the
 * buffer keeps the last call's contents (each call overwrites all it reads).
 * Errors otherwise as fattn_bwd; EHIP if the buffer's address cannot be
 * looked up.
 */
#define FATTN_NOALLOC_WORKSPACE_BYTES ((size_t)16 << 20)
fattn_status fattn_bwd_noalloc(const void* q, const void* k, const void* v,
                               const void* o, const float* lse, const void* dout,
                               void* dq, void* dk, void* dv, int B, int H, int N,
                               int d, int causal, float scale, void* stream);

/*
 * Packed variable-length sequences (varlen), bf16 forward and backward.
 *   cu_seqlens  device int32 [nseq + 1], non-decreasing offsets into the N rows
 *               of every head: rows [cu_seqlens[s], cu_seqlens[s+1]) form
 *               segment s, and a query attends only to the keys of its own
 *               segment (and, when causal, to those at or before its row).
 *               The same offsets apply to every (b, h).
 *   nseq        number of segments, >= 1.
 *   max_seqlen  an upper bound on every segment's length, 1..N: it sizes the
 *               launch grid (B·H·nseq·ceil(max_seqlen/128) workgroups,
 *               ENOTSUP past 2^31 − 1).
 * Everything else as fattn_fwd / fattn_bwd (same workspace). Each segment is
 * computed exactly as fattn_fwd / fattn_bwd would compute it as a sequence of
 * its own. The offsets live in device memory, so they are not checked on the
 * host: the kernels clamp them to [0, N] (no access outside the tensors for
 * any contents), and the caller must keep cu_seqlens[0] = 0,
 * cu_seqlens[nseq] = N and every length <= max_seqlen — rows outside every
 * segment, and rows of a segment past max_seqlen, are not written.
 */
fattn_status fattn_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                              float* lse, const int32_t* cu_seqlens, int nseq,
                              int max_seqlen, int B, int H, int N, int d, int causal,
                              float scale, int exp_mode, void* stream);
fattn_status fattn_bwd_varlen(const void* q, const void* k, const void* v,
                              const void* o, const float* lse, const void* dout,
                              void* dq, void* dk, void* dv,
                              const int32_t* cu_seqlens, int nseq, int max_seqlen,
                              int B, int H, int N, int d, int causal, float scale,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-sparse bf16 forward.
 *   block_mask  device uint8, one entry per block of 128 queries × 128 keys:
 *               [nb][nb] shared by every (b, h) (per_head = 0) or
 *               [B·H][nb][nb] (per_head = 1), nb = ceil(N/128), row-major
 *               (query block, key block). Non-zero: the keys of the key block
 *               are visible to the queries of the query block (subject also
 *               to the causal mask); zero: they are not, and their K/V tiles
 *               are never loaded.
 * A query that sees no key gets O = 0 and LSE = −∞ (the convention of the
 * plain definition for an empty row). Everything else as fattn_fwd. The mask
 * lives in device memory and is read as given (the caller sizes it).
 * Supports N <= 32768 (ENOTSUP beyond).
 * fattn_bwd_blocksparse: the backward of fattn_fwd_blocksparse from its O and
 * LSE, same mask, same workspace as fattn_bwd; key blocks that no query sees
 * get dK = dV = 0, queries that see no key get dQ = 0.
 */
fattn_status fattn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o,
                                   float* lse, const uint8_t* block_mask, int per_head,
                                   int B, int H, int N, int d, int causal, float scale,
                                   int exp_mode, void* stream);
fattn_status fattn_bwd_blocksparse(const void* q, const void* k, const void* v,
                                   const void* o, const float* lse, const void* dout,
                                   void* dq, void* dk, void* dv,
                                   const uint8_t* block_mask, int per_head, int B, int H,
                                   int N, int d, int causal, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Forward with fp8 (OCP e4m3fn) operands and bf16 in/out
 * (FlashAttention-3 page, innovation 3).
 *   q, k, v     [B,H,N,d] bf16 inputs; o [B,H,N,d] bf16 output.
 *   lse         optional [B,H,N] fp32 output (NULL to skip).
 *   exp_mode    one of fattn_exp_mode, for the exponentials of the softmax
 *               (FlashAttention-4 gist, technical summary 2.B).
 *   rotate      1: Q' = Q·R, K' = K·R with R = diag(s)·H_d/√d, H_d the
 *               Sylvester Hadamard matrix, s_i = ±1 from the top bit of the
 *               i-th SplitMix64 output for state `seed`; 0: no rotation.
 *   workspace   at least fattn_fwd_fp8_workspace_bytes(B,H,N,d) bytes,
 *               256-byte aligned. Layout (see fattn_fwd_fp8_workspace_layout):
 *               e4m3 K8 [B,H,N,d], e4m3 V8 stored transposed per head as
 *               [B,H,d,Npad] (Npad = N rounded up to 64, zero padded; inside
 *               each block of 64 keys, position p = 32a + s holds key
 *               32(s/16) + 8((s%16)/4) + 4a + s%4, the order in which the
 *               kernel's P operand holds keys), then fp32 scales
 *               [B·H][⌈N/128⌉][2]: the (K', V) pair of each chunk of 128
 *               keys (keys 128c .. 128c + 127).
 * K' and Q' are quantised as code = e4m3(x·448/amax), the exact ratio
 * rounded to nearest even, with scale amax/448 (1 where amax = 0): K' with
 * one amax per (b, h) and chunk of 128 keys, Q' with one amax per row (each
 * query row meets the keys only through its own scores). V takes one power
 * of two per (b, h) and chunk, 2^e with e the least integer ≥ −126 such
 * that amax ≤ 448·2^e (1 where amax = 0), and code = e4m3(v·2^−e), an
 * exact scaling; the PV product applies 2^e as the fp8 MFMA's block scale.
 * Q' keeps a second e4m3 term for its quantisation residual,
 * Q8lo = e4m3(16·(x·448/amax − decode(Q8))), so that
 * Q' ≈ scale_q·(Q8 + Q8lo/16); the scores use both terms (two fp8 MFMAs).
 * Q' is rotated and quantised inside the attention kernel (each workgroup
 * its own rows) and never stored.
 * The softmax stores each unnormalised probability P̃ = 2^(s − m) in e4m3
 * as P̃·2^(7−k) ≤ 256, with m the row's first tile max and k ≥ 0 the least
 * integer that keeps every stored value of the row so far within that
 * bound; the matrix core multiplies 2^k back (the P operand's block scale),
 * so the partial output is rescaled only when k would pass 32 (m then moves
 * to the row max). O is normalised by the sum of the quantised P̃ of its
 * row.
 * Additionally requires B·H ≤ 65535 (ENOTSUP otherwise).
 * Validated range (GPU parity tests against float64 attention): d ∈ {64,
 * 128}, N from 1 to 32768, causal and not. Error against exact attention,
 * relative RMS of O: within 6e-2 for N(0,1) inputs up to N = 32768 and for
 * inputs with 0.1% of the Q and K entries scaled by 20 at N = 4096 (every
 * element of B=4, H=16). With such outliers the e4m3 operands alone already
 * cost about 5.5% at N = 32768 (the quantised operands with exact P against
 * exact attention), so there the output is held to 4e-2 of that operand
 * model instead. Longer sequences run but are not validated.
 */
size_t fattn_fwd_fp8_workspace_bytes(int B, int H, int N, int d);
fattn_status fattn_fwd_fp8_workspace_layout(int B, int H, int N, int d,
                                            size_t* off_k8, size_t* off_v8t,
                                            size_t* off_scales);
fattn_status fattn_fwd_fp8(const void* q, const void* k, const void* v, void* o,
                           float* lse, int B, int H, int N, int d, int causal,
                           float scale, int exp_mode, int rotate, uint64_t seed,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * The attention step of fattn_fwd_fp8 alone (FlashAttention-3 page,
 * "Nuevas capacidades…" (FP8): the fp8 matrix products with the softmax
 * between them), on a workspace that a previous fattn_fwd_fp8 call with the
 * same B, H, N, d, rotate and seed filled: it reads the e4m3 operands K8,
 * V8ᵀ and their scales from the workspace, rotates and quantises q itself
 * (bf16 [B,H,N,d], as fattn_fwd_fp8 does) and writes o (and lse if
 * non-NULL) exactly as that call did for the same q, causal, scale and
 * exp_mode. The workspace is only read.
 * For re-running attention on keys and values already quantised, and for
 * timing the attention step apart from the K/V quantisation.
 * Errors as fattn_fwd_fp8 (a workspace never filled gives meaningless o,
 * not an error).
 */
fattn_status fattn_fwd_fp8_attend(const void* q, void* o, float* lse, int B, int H, int N,
                                  int d, int causal, float scale, int exp_mode, int rotate,
                                  uint64_t seed, const void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Block-sparse fp8 forward: fattn_fwd_fp8 restricted by a block mask
 * (FlashAttention-4 gist, closing summary: block-sparse named among the
 * variants the design admits; FlashAttention-3 page, innovation 3 for the
 * fp8 operands). block_mask and per_head exactly as for
 * fattn_fwd_blocksparse (uint8 over 128-query × 128-key blocks, device
 * memory, read as given; key blocks a query block does not see are never
 * loaded). The quantisation is that of fattn_fwd_fp8: K' and V with one
 * scale per (b, h) and chunk of 128 keys, taken over all of the chunk's keys
 * whether visible or not, and Q' per row; the workspace is filled the same
 * way, so a later
 * fattn_fwd_fp8_attend on it computes dense attention of the same operands.
 * A query that sees no key gets O = 0 and LSE = −∞. With every block set
 * the result equals fattn_fwd_fp8's. Supports N <= 32768 (ENOTSUP beyond);
 * everything else, errors included, as fattn_fwd_fp8.
 */
fattn_status fattn_fwd_fp8_blocksparse(const void* q, const void* k, const void* v, void* o,
                                       float* lse, const uint8_t* block_mask, int per_head,
                                       int B, int H, int N, int d, int causal, float scale,
                                       int exp_mode, int rotate, uint64_t seed,
                                       void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * fp8 forward over packed variable-length sequences: fattn_fwd_fp8 with the
 * segments of fattn_fwd_varlen (cu_seqlens, nseq, max_seqlen as there; FA4
 * gist, closing summary: varlen named among the variants the design admits;
 * FlashAttention-3 page, innovation 3 for the fp8 operands). Each segment
 * is a sequence of its own, also for the quantisation: K' and V get one
 * scale per (b, h, segment) and chunk of 128 of that segment's rows counted
 * from its first, Q' one per row as always, so each segment's O and LSE and
 * its K8, V8ᵀ and scales are exactly those fattn_fwd_fp8 gives
 * for that segment alone (same rotate, seed, causal, scale, exp_mode).
 *   workspace   at least fattn_fwd_fp8_varlen_workspace_bytes(B, H, N, d,
 *               nseq, max_seqlen) bytes, 256-byte aligned: K8 as for
 *               fattn_fwd_fp8; V8ᵀ [B,H,d,Npad] with Npad = roundup(N, 64) +
 *               64·nseq, segment s in the 64-key blocks from column
 *               roundup(cu[s], 64) + 64·s on (same key order); scales
 *               [B·H][nseq][⌈max_seqlen/128⌉][2] (the chunks a segment
 *               has; the rest are not written).
 * The offsets are read on the device and clamped to [0, N], and every
 * segment is cut to its first max_seqlen rows (the caller keeps lengths
 * within max_seqlen; rows outside every segment, or past that cut, are not
 * written). Additionally ENOTSUP when d·Npad ≥ 2^31 or
 * nseq·⌈max_seqlen/64⌉ ≥ 2^31. Errors otherwise as fattn_fwd_varlen and
 * fattn_fwd_fp8.
 */
size_t fattn_fwd_fp8_varlen_workspace_bytes(int B, int H, int N, int d, int nseq,
                                            int max_seqlen);
fattn_status fattn_fwd_fp8_varlen(const void* q, const void* k, const void* v, void* o,
                                  float* lse, const int32_t* cu_seqlens, int nseq,
                                  int max_seqlen, int B, int H, int N, int d, int causal,
                                  float scale, int exp_mode, int rotate, uint64_t seed,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* fattn_strerror(int status);
/* Detail of the last error on the calling thread (argument or HIP message). */
const char* fattn_last_error(void);
/* Library version as major*10000 + minor*100 + patch. */
int fattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FATTN_H */
