// Internal launcher interface between the C-ABI host code (fattn_host.cpp)
// and the kernel translation units. Arguments are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fattn {

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, bool causal, float scale, int exp_mode,
                           hipStream_t stream);

// Packed variable-length sequences: rows [cu_seqlens[s], cu_seqlens[s+1]) of
// every head form segment s (device int32 [nseq+1]); max_seqlen bounds the
// segment lengths the grid covers.
hipError_t launch_fwd_bf16_varlen(const void* q, const void* k, const void* v, void* o,
                                  float* lse, const int* cu_seqlens, int nseq, int max_seqlen,
                                  int B, int H, int N, int d, bool causal, float scale,
                                  int exp_mode, hipStream_t stream);

// Block-sparse forward: block_mask uint8 [⌈N/128⌉][⌈N/128⌉] (one for all
// heads) or [B*H][⌈N/128⌉][⌈N/128⌉] (per_head); non-zero = visible.
hipError_t launch_fwd_bf16_blocksparse(const void* q, const void* k, const void* v, void* o,
                                       float* lse, const uint8_t* block_mask, bool per_head,
                                       int B, int H, int N, int d, bool causal, float scale,
                                       int exp_mode, hipStream_t stream);

// Backward: `dvec` and `lse2` fp32 [B,H,Npad] live in the caller's workspace
// (Npad = N rounded up to kBwdRowPad).
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* dvec, float* lse2, int B, int H, int N, int d, bool causal,
                           float scale, hipStream_t stream);

hipError_t launch_bwd_bf16_varlen(const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, const void* dout, void* dq, void* dk,
                                  void* dv, float* dvec, float* lse2, const int* cu_seqlens,
                                  int nseq, int max_seqlen, int B, int H, int N, int d,
                                  bool causal, float scale, hipStream_t stream);

hipError_t launch_bwd_bf16_blocksparse(const void* q, const void* k, const void* v,
                                       const void* o, const float* lse, const void* dout,
                                       void* dq, void* dk, void* dv, float* dvec, float* lse2,
                                       const uint8_t* block_mask, bool per_head, int B, int H,
                                       int N, int d, bool causal, float scale,
                                       hipStream_t stream);

constexpr int kBwdRowPad = 64;

// fp8 forward: k8 e4m3 [B,H,N,d]; v8t e4m3 [B,H,d,Npad]; scales fp32
// [B*H(*nseq)][ceil(rows/128)][2] (K, V per 128-key chunk; rows = N, or
// max_seqlen with packed segments). Q is rotated and quantised (one scale
// per row) inside the attention kernel.
// block_mask: optional uint8 mask over 128×128 blocks ([nb][nb], or
// [B·H][nb][nb] when per_head), as for launch_fwd_bf16_blocksparse.
// cu_seqlens: optional packed segments (nseq, max_seqlen), as for
// launch_fwd_bf16_varlen; then V8ᵀ has roundup(N, 64) + 64·nseq columns per
// head. Not both.
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                          uint8_t* k8, uint8_t* v8t, float* scales, int B, int H, int N, int d,
                          bool causal, float scale, int exp_mode, bool rotate, uint64_t seed,
                          const uint8_t* block_mask, bool per_head, const int* cu_seqlens,
                          int nseq, int max_seqlen, hipStream_t stream);

// fp8 attention only (the last launch of launch_fwd_fp8) on the K/V operands
// a previous launch_fwd_fp8 of the same shape left in k8/v8t/scales; Q is
// read in bf16 as in launch_fwd_fp8.
hipError_t launch_fwd_fp8_attend(const void* q, void* o, float* lse, const uint8_t* k8,
                                 const uint8_t* v8t, const float* scales, int B, int H, int N,
                                 int d, bool causal, float scale, int exp_mode, bool rotate,
                                 uint64_t seed, hipStream_t stream);

// Library-owned backward workspace (static_ws.hip): its capacity, and its
// device address on `device`, which must be the current device (looked up on
// the first call for that device, then cached).
constexpr size_t kStaticWorkspaceBytes = (size_t)16 << 20;
hipError_t static_workspace(int device, void** ptr);

constexpr int kFp8Npad = 64;
constexpr int kFp8AmaxRows = 128;  // keys per K/V scale chunk

}  // namespace fattn
