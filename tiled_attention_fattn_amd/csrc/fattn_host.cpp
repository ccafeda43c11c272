// C-ABI entry points of libfattn: argument validation (host only, before any
// HIP call), the gfx950 device check, workspace carving and kernel launch on
// the caller's stream. Allocates nothing, never synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/fattn.h"
#include "fattn_launch.h"

namespace {

thread_local char g_last_error[512] = "";

fattn_status fail(fattn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Shape checks shared by every entry point.
fattn_status check_shape(int B, int H, int N, int d, int causal, float scale) {
  if (B < 1 || H < 1 || N < 1)
    return fail(FATTN_EINVAL, "B, H and N must be >= 1 (got B=%d H=%d N=%d)", B, H, N);
  if (d != 64 && d != 128) return fail(FATTN_ENOTSUP, "head dimension d=%d not supported (64 or 128)", d);
  if (causal != 0 && causal != 1) return fail(FATTN_EINVAL, "causal must be 0 or 1 (got %d)", causal);
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(FATTN_EINVAL, "scale must be finite and > 0 (got %g)", (double)scale);
  const unsigned long long elems = (unsigned long long)B * H * N * d;
  if (elems >= (1ull << 31))
    return fail(FATTN_ENOTSUP, "tensor of %llu elements exceeds 2^31-1", elems);
  return FATTN_OK;
}

fattn_status check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(FATTN_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(FATTN_EINVAL, "%s is not 16-byte aligned", name);
  return FATTN_OK;
}

// gfx950 check, cached per device id.
std::mutex g_dev_mu;
int g_dev_ok[64];  // 0 unknown, 1 gfx950, 2 other

fattn_status check_device(int* dev_out = nullptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FATTN_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(FATTN_EDEVICE, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(FATTN_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_dev_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    if (g_dev_ok[dev] == 2) return fail(FATTN_EDEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  if (g_dev_ok[dev] != 1) return fail(FATTN_EDEVICE, "device %d is not gfx950", dev);
  if (dev_out) *dev_out = dev;
  return FATTN_OK;
}

fattn_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
  g_last_error[0] = '\0';
  return FATTN_OK;
}

#define FATTN_TRY(x)                    \
  do {                                  \
    fattn_status s_ = (x);              \
    if (s_ != FATTN_OK) return s_;      \
  } while (0)

struct Fp8Layout {
  size_t k8, v8t, scales, total;
};

// nseq = 0: no packed segments (one per head, all N rows). With segments
// V8ᵀ has 64 more columns per segment and the scales one set per (head,
// segment) over max_seqlen rows. Scales: a (K, V) fp32 pair per 128-key
// chunk.
Fp8Layout fp8_layout(int B, int H, int N, int d, int nseq = 0, int max_seqlen = 0) {
  const size_t bh = (size_t)B * H;
  const size_t units = bh * (nseq > 0 ? nseq : 1);
  const size_t npad = round_up((size_t)N, fattn::kFp8Npad) + (size_t)fattn::kFp8Npad * nseq;
  const size_t rows = nseq > 0 ? (size_t)max_seqlen : (size_t)N;
  Fp8Layout L;
  L.k8 = 0;
  L.v8t = round_up(L.k8 + bh * N * d, 256);
  L.scales = round_up(L.v8t + bh * d * npad, 256);
  const size_t nchunks = (rows + fattn::kFp8AmaxRows - 1) / fattn::kFp8AmaxRows;
  L.total = round_up(L.scales + 2 * units * nchunks * sizeof(float), 256);
  return L;
}

fattn_status check_varlen(const int32_t* cu_seqlens, int nseq, int max_seqlen, int B, int H,
                          int N) {
  if (cu_seqlens == nullptr) return fail(FATTN_EINVAL, "cu_seqlens is NULL");
  if (((uintptr_t)cu_seqlens & 3) != 0) return fail(FATTN_EINVAL, "cu_seqlens is not 4-byte aligned");
  if (nseq < 1) return fail(FATTN_EINVAL, "nseq must be >= 1 (got %d)", nseq);
  if (max_seqlen < 1 || max_seqlen > N)
    return fail(FATTN_EINVAL, "max_seqlen must be in [1, N=%d] (got %d)", N, max_seqlen);
  // Grid of (head, segment, 128-row tile) workgroups.
  const unsigned long long wgs = (unsigned long long)B * H * nseq * ((max_seqlen + 127) / 128);
  if (wgs >= (1ull << 31))
    return fail(FATTN_ENOTSUP, "%llu workgroups (B*H*nseq*ceil(max_seqlen/128)) exceed 2^31-1", wgs);
  return FATTN_OK;
}

fattn_status check_exp_mode(int exp_mode) {
  if (exp_mode < FATTN_EXP_AUTO || exp_mode > FATTN_EXP_SPLIT)
    return fail(FATTN_EINVAL, "exp_mode must be 0, 1, 2 or 3 (got %d)", exp_mode);
  return FATTN_OK;
}

}  // namespace

extern "C" {

fattn_status fattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int N, int d, int causal, float scale, int exp_mode, void* stream) {
  FATTN_TRY(check_ptr(q, "q"));
  FATTN_TRY(check_ptr(k, "k"));
  FATTN_TRY(check_ptr(v, "v"));
  FATTN_TRY(check_ptr(o, "o"));
  FATTN_TRY(check_ptr(lse, "lse"));
  FATTN_TRY(check_shape(B, H, N, d, causal, scale));
  FATTN_TRY(check_exp_mode(exp_mode));
  FATTN_TRY(check_device());
  const int mode = exp_mode == FATTN_EXP_AUTO ? FATTN_EXP_HW : exp_mode;
  return hip_status(fattn::launch_fwd_bf16(q, k, v, o, lse, B, H, N, d, causal != 0, scale, mode,
                                           (hipStream_t)stream),
                    "fattn_fwd launch");
}

fattn_status fattn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int32_t* cu_seqlens, int nseq, int max_seqlen, int B, int H,
                              int N, int d, int causal, float scale, int exp_mode, void* stream) {
  FATTN_TRY(check_ptr(q, "q"));
  FATTN_TRY(check_ptr(k, "k"));
  FATTN_TRY(check_ptr(v, "v"));
  FATTN_TRY(check_ptr(o, "o"));
  FATTN_TRY(check_ptr(lse, "lse"));
  FATTN_TRY(check_shape(B, H, N, d, causal, scale));
  FATTN_TRY(check_varlen(cu_seqlens, nseq, max_seqlen, B, H, N));
  FATTN_TRY(check_exp_mode(exp_mode));
  FATTN_TRY(check_device());
  const int mode = exp_mode == FATTN_EXP_AUTO ? FATTN_EXP_HW : exp_mode;
  return hip_status(fattn::launch_fwd_bf16_varlen(q, k, v, o, lse, cu_seqlens, nseq, max_seqlen,
                                                  B, H, N, d, causal != 0, scale, mode,
                                                  (hipStream_t)stream),
                    "fattn_fwd_varlen launch");
}

fattn_status fattn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o,
                                   float* lse, const uint8_t* block_mask, int per_head, int B,
                                   int H, int N, int d, int causal, float scale, int exp_mode,
                                   void* stream) {
  FATTN_TRY(check_ptr(q, "q"));
  FATTN_TRY(check_ptr(k, "k"));
  FATTN_TRY(check_ptr(v, "v"));
  FATTN_TRY(check_ptr(o, "o"));
  FATTN_TRY(check_ptr(lse, "lse"));
  FATTN_TRY(check_shape(B, H, N, d, causal, scale));
  if (block_mask == nullptr) return fail(FATTN_EINVAL, "block_mask is NULL");
  if (per_head != 0 && per_head != 1)
    return fail(FATTN_EINVAL, "per_head must be 0 or 1 (got %d)", per_head);
  if (N > 32768) return fail(FATTN_ENOTSUP, "block-sparse forward supports N <= 32768 (got %d)", N);
  FATTN_TRY(check_exp_mode(exp_mode));
  FATTN_TRY(check_device());
  const int mode = exp_mode == FATTN_EXP_AUTO ? FATTN_EXP_HW : exp_mode;
  return hip_status(fattn::launch_fwd_bf16_blocksparse(q, k, v, o, lse, block_mask,
                                                       per_head != 0, B, H, N, d, causal != 0,
                                                       scale, mode, (hipStream_t)stream),
                    "fattn_fwd_blocksparse launch");
}

size_t fattn_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
  const size_t n = (size_t)B * H * round_up((size_t)N, fattn::kBwdRowPad);
  return 2 * round_up(n * sizeof(float), 256);
}

fattn_status fattn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                       int causal, float scale, void* workspace, size_t workspace_bytes,
                       void* stream) {
  FATTN_TRY(check_ptr(q, "q"));
  FATTN_TRY(check_ptr(k, "k"));
  FATTN_TRY(check_ptr(v, "v"));
  FATTN_TRY(check_ptr(o, "o"));
  FATTN_TRY(check_ptr(lse, "lse"));
  FATTN_TRY(check_ptr(dout, "dout"));
  FATTN_TRY(check_ptr(dq, "dq"));
  FATTN_TRY(check_ptr(dk, "dk"));
  FATTN_TRY(check_ptr(dv, "dv"));
  FATTN_TRY(check_shape(B, H, N, d, causal, scale));
  if (workspace == nullptr) return fail(FATTN_EWORKSPACE, "workspace is NULL");
  if (!aligned256(workspace)) return fail(FATTN_EWORKSPACE, "workspace is not 256-byte aligned");
  const size_t need = fattn_bwd_workspace_bytes(B, H, N, d);
  if (workspace_bytes < need)
    return fail(FATTN_EWORKSPACE, "workspace of %zu bytes, %zu required", workspace_bytes, need);
  FATTN_TRY(check_device());
  const size_t n = (size_t)B * H * round_up((size_t)N, fattn::kBwdRowPad);
  float* dvec = (float*)workspace;
  float* lse2 = (float*)((char*)dvec + round_up(n * sizeof(float), 256));
  return hip_status(fattn::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, dvec, lse2, B, H, N,
                                           d, causal != 0, scale, (hipStream_t)stream),
                    "fattn_bwd launch");
}

fattn_status fattn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              const int32_t* cu_seqlens, int nseq, int max_seqlen, int B, int H,
                              int N, int d, int causal, float scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
  FATTN_TRY(check_ptr(q, "q"));
  FATTN_TRY(check_ptr(k, "k"));
  FATTN_TRY(check_ptr(v, "v"));
  FATTN_TRY(check_ptr(o, "o"));
  FATTN_TRY(check_ptr(lse, "lse"));
  FATTN_TRY(check_ptr(dout, "dout"));
  FATTN_TRY(check_ptr(dq, "dq"));
  FATTN_TRY(check_ptr(dk, "dk"));
  FATTN_TRY(check_ptr(dv, "dv"));
  FATTN_TRY(check_shape(B, H, N, d, causal, scale));
  FATTN_TRY(check_varlen(cu_seqlens, nseq, max_seqlen, B, H, N));
  if (workspace == nullptr) return fail(FATTN_EWORKSPACE, "workspace is NULL");
  if (!aligned256(workspace)) return fail(FATTN_EWORKSPACE, "workspace is not 256-byte aligned");
  const size_t need = fattn_bwd_workspace_bytes(B, H, N, d);
  if (workspace_bytes < need)
    return fail(FATTN_EWORKSPACE, "workspace of %zu bytes, %zu required", workspace_bytes, need);
  FATTN_TRY(check_device());
  const size_t n = (size_t)B * H * round_up((size_t)N, fattn::kBwdRowPad);
  float* dvec = (float*)workspace;
  float* lse2 = (float*)((char*)dvec + round_up(n * sizeof(float), 256));
  return hip_status(fattn::launch_bwd_bf16_varlen(q, k, v, o, lse, dout, dq, dk, dv, dvec, lse2,
                                                  cu_seqlens, nseq, max_seqlen, B, H, N, d,
                                                  causal != 0, scale, (hipStream_t)stream),
                    "fattn_bwd_varlen launch");
}

fattn_status fattn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o,
                                   const float* lse, const void* dout, void* dq, void* dk,
                                   void* dv, const uint8_t* block_mask, int per_head, int B,
                                   int H, int N, int d, int causal, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  FATTN_TRY(check_ptr(q, "q"));
  FATTN_TRY(check_ptr(k, "k"));
  FATTN_TRY(check_ptr(v, "v"));
  FATTN_TRY(check_ptr(o, "o"));
  FATTN_TRY(check_ptr(lse, "lse"));
  FATTN_TRY(check_ptr(dout, "dout"));
  FATTN_TRY(check_ptr(dq, "dq"));
  FATTN_TRY(check_ptr(dk, "dk"));
  FATTN_TRY(check_ptr(dv, "dv"));
  FATTN_TRY(check_shape(B, H, N, d, causal, scale));
  if (block_mask == nullptr) return fail(FATTN_EINVAL, "block_mask is NULL");
  if (per_head != 0 && per_head != 1)
    return fail(FATTN_EINVAL, "per_head must be 0 or 1 (got %d)", per_head);
  if (N > 32768) return fail(FATTN_ENOTSUP, "block-sparse backward supports N <= 32768 (got %d)", N);
  if (workspace == nullptr) return fail(FATTN_EWORKSPACE, "workspace is NULL");
  if (!aligned256(workspace)) return fail(FATTN_EWORKSPACE, "workspace is not 256-byte aligned");
  const size_t need = fattn_bwd_workspace_bytes(B, H, N, d);
  if (workspace_bytes < need)
    return fail(FATTN_EWORKSPACE, "workspace of %zu bytes, %zu required", workspace_bytes, need);
  FATTN_TRY(check_device());
  const size_t n = (size_t)B * H * round_up((size_t)N, fattn::kBwdRowPad);
  float* dvec = (float*)workspace;
  float* lse2 = (float*)((char*)dvec + round_up(n * sizeof(float), 256));
  return hip_status(fattn::launch_bwd_bf16_blocksparse(q, k, v, o, lse, dout, dq, dk, dv, dvec,
                                                       lse2, block_mask, per_head != 0, B, H, N,
                                                       d, causal != 0, scale,
                                                       (hipStream_t)stream),
                    "fattn_bwd_blocksparse launch");
}

fattn_status fattn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               int B, int H, int N, int d, int causal, float scale,
                               void* stream) {
  static_assert(FATTN_NOALLOC_WORKSPACE_BYTES == fattn::kStaticWorkspaceBytes,
                "the header states the static workspace's capacity");
  FATTN_TRY(check_ptr(q, "q"));
  FATTN_TRY(check_ptr(k, "k"));
  FATTN_TRY(check_ptr(v, "v"));
  FATTN_TRY(check_ptr(o, "o"));
  FATTN_TRY(check_ptr(lse, "lse"));
  FATTN_TRY(check_ptr(dout, "dout"));
  FATTN_TRY(check_ptr(dq, "dq"));
  FATTN_TRY(check_ptr(dk, "dk"));
  FATTN_TRY(check_ptr(dv, "dv"));
  FATTN_TRY(check_shape(B, H, N, d, causal, scale));
  const size_t need = fattn_bwd_workspace_bytes(B, H, N, d);
  if (need > fattn::kStaticWorkspaceBytes)
    return fail(FATTN_EWORKSPACE,
                "B=%d H=%d N=%d needs %zu bytes of workspace; the library's static workspace "
                "holds %zu (use fattn_bwd with a caller workspace)",
                B, H, N, need, fattn::kStaticWorkspaceBytes);
  int dev = 0;
  FATTN_TRY(check_device(&dev));
  void* ws = nullptr;
  const hipError_t e = fattn::static_workspace(dev, &ws);
  if (e != hipSuccess)
    return fail(FATTN_EHIP, "static workspace of device %d: %s", dev, hipGetErrorString(e));
  const size_t n = (size_t)B * H * round_up((size_t)N, fattn::kBwdRowPad);
  float* dvec = (float*)ws;
  float* lse2 = (float*)((char*)dvec + round_up(n * sizeof(float), 256));
  return hip_status(fattn::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, dvec, lse2, B, H, N,
                                           d, causal != 0, scale, (hipStream_t)stream),
                    "fattn_bwd_noalloc launch");
}

size_t fattn_fwd_fp8_workspace_bytes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
  return fp8_layout(B, H, N, d).total;
}

fattn_status fattn_fwd_fp8_workspace_layout(int B, int H, int N, int d, size_t* off_k8,
                                            size_t* off_v8t, size_t* off_scales) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return fail(FATTN_EINVAL, "B, H, N and d must be >= 1");
  const Fp8Layout L = fp8_layout(B, H, N, d);
  if (off_k8) *off_k8 = L.k8;
  if (off_v8t) *off_v8t = L.v8t;
  if (off_scales) *off_scales = L.scales;
  return FATTN_OK;
}

// fattn_fwd_fp8, fattn_fwd_fp8_blocksparse and fattn_fwd_fp8_varlen: one
// validation and launch path (block_mask and cu_seqlens NULL for dense
// attention; the callers set at most one of them).
static fattn_status fwd_fp8_impl(const char* name, const void* q, const void* k, const void* v,
                                 void* o, float* lse, const uint8_t* block_mask, int per_head,
                                 const int32_t* cu_seqlens, int nseq, int max_seqlen, int B,
                                 int H, int N, int d, int causal, float scale, int exp_mode,
                                 int rotate, uint64_t seed, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  FATTN_TRY(check_ptr(q, "q"));
  FATTN_TRY(check_ptr(k, "k"));
  FATTN_TRY(check_ptr(v, "v"));
  FATTN_TRY(check_ptr(o, "o"));
  if (lse != nullptr && !aligned16(lse)) return fail(FATTN_EINVAL, "lse is not 16-byte aligned");
  FATTN_TRY(check_shape(B, H, N, d, causal, scale));
  FATTN_TRY(check_exp_mode(exp_mode));
  if (rotate != 0 && rotate != 1) return fail(FATTN_EINVAL, "rotate must be 0 or 1 (got %d)", rotate);
  if ((long long)B * H > 65535)
    return fail(FATTN_ENOTSUP, "fp8 forward supports B*H <= 65535 (got %lld)", (long long)B * H);
  if (block_mask != nullptr) {
    if (per_head != 0 && per_head != 1)
      return fail(FATTN_EINVAL, "per_head must be 0 or 1 (got %d)", per_head);
    if (N > 32768)
      return fail(FATTN_ENOTSUP, "block-sparse forward supports N <= 32768 (got %d)", N);
  }
  const bool varlen = cu_seqlens != nullptr;
  if (varlen) {
    FATTN_TRY(check_varlen(cu_seqlens, nseq, max_seqlen, B, H, N));
    // V8ᵀ rows of d·(roundup(N, 64) + 64·nseq) bytes per head, addressed
    // with 32-bit offsets; 64-key blocks per segment in one grid dimension.
    const unsigned long long vcols =
        (unsigned long long)round_up((size_t)N, fattn::kFp8Npad) + 64ull * nseq;
    if ((unsigned long long)d * vcols >= (1ull << 31))
      return fail(FATTN_ENOTSUP, "d*(N+64*nseq) = %llu bytes of V8 per head exceed 2^31-1",
                  (unsigned long long)d * vcols);
    if ((unsigned long long)nseq * ((max_seqlen + 63) / 64) >= (1ull << 31))
      return fail(FATTN_ENOTSUP, "nseq*ceil(max_seqlen/64) exceeds 2^31-1");
  }
  if (workspace == nullptr) return fail(FATTN_EWORKSPACE, "workspace is NULL");
  if (!aligned256(workspace)) return fail(FATTN_EWORKSPACE, "workspace is not 256-byte aligned");
  const Fp8Layout L = varlen ? fp8_layout(B, H, N, d, nseq, max_seqlen) : fp8_layout(B, H, N, d);
  if (workspace_bytes < L.total)
    return fail(FATTN_EWORKSPACE, "workspace of %zu bytes, %zu required", workspace_bytes, L.total);
  FATTN_TRY(check_device());
  char* ws = (char*)workspace;
  return hip_status(fattn::launch_fwd_fp8(q, k, v, o, lse, (uint8_t*)(ws + L.k8),
                                          (uint8_t*)(ws + L.v8t), (float*)(ws + L.scales),
                                          B, H, N, d, causal != 0, scale,
                                          exp_mode == FATTN_EXP_AUTO ? FATTN_EXP_HW : exp_mode,
                                          rotate != 0, seed, block_mask, per_head != 0,
                                          cu_seqlens, nseq, max_seqlen, (hipStream_t)stream),
                    name);
}

fattn_status fattn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int N, int d, int causal, float scale, int exp_mode, int rotate,
                           uint64_t seed, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_fp8_impl("fattn_fwd_fp8 launch", q, k, v, o, lse, nullptr, 0, nullptr, 0, 0, B, H,
                      N, d, causal, scale, exp_mode, rotate, seed, workspace, workspace_bytes,
                      stream);
}

fattn_status fattn_fwd_fp8_blocksparse(const void* q, const void* k, const void* v, void* o,
                                       float* lse, const uint8_t* block_mask, int per_head, int B,
                                       int H, int N, int d, int causal, float scale, int exp_mode,
                                       int rotate, uint64_t seed, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (block_mask == nullptr) return fail(FATTN_EINVAL, "block_mask is NULL");
  return fwd_fp8_impl("fattn_fwd_fp8_blocksparse launch", q, k, v, o, lse, block_mask, per_head,
                      nullptr, 0, 0, B, H, N, d, causal, scale, exp_mode, rotate, seed, workspace,
                      workspace_bytes, stream);
}

size_t fattn_fwd_fp8_varlen_workspace_bytes(int B, int H, int N, int d, int nseq,
                                            int max_seqlen) {
  if (B < 1 || H < 1 || N < 1 || d < 1 || nseq < 1 || max_seqlen < 1) return 0;
  return fp8_layout(B, H, N, d, nseq, max_seqlen).total;
}

fattn_status fattn_fwd_fp8_varlen(const void* q, const void* k, const void* v, void* o,
                                  float* lse, const int32_t* cu_seqlens, int nseq,
                                  int max_seqlen, int B, int H, int N, int d, int causal,
                                  float scale, int exp_mode, int rotate, uint64_t seed,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (cu_seqlens == nullptr) return fail(FATTN_EINVAL, "cu_seqlens is NULL");
  return fwd_fp8_impl("fattn_fwd_fp8_varlen launch", q, k, v, o, lse, nullptr, 0, cu_seqlens,
                      nseq, max_seqlen, B, H, N, d, causal, scale, exp_mode, rotate, seed,
                      workspace, workspace_bytes, stream);
}

fattn_status fattn_fwd_fp8_attend(const void* q, void* o, float* lse, int B, int H, int N, int d,
                                  int causal, float scale, int exp_mode, int rotate, uint64_t seed,
                                  const void* workspace, size_t workspace_bytes, void* stream) {
  FATTN_TRY(check_ptr(q, "q"));
  FATTN_TRY(check_ptr(o, "o"));
  if (lse != nullptr && !aligned16(lse)) return fail(FATTN_EINVAL, "lse is not 16-byte aligned");
  FATTN_TRY(check_shape(B, H, N, d, causal, scale));
  FATTN_TRY(check_exp_mode(exp_mode));
  if (rotate != 0 && rotate != 1) return fail(FATTN_EINVAL, "rotate must be 0 or 1 (got %d)", rotate);
  if ((long long)B * H > 65535)
    return fail(FATTN_ENOTSUP, "fp8 forward supports B*H <= 65535 (got %lld)", (long long)B * H);
  if (workspace == nullptr) return fail(FATTN_EWORKSPACE, "workspace is NULL");
  if (!aligned256(workspace)) return fail(FATTN_EWORKSPACE, "workspace is not 256-byte aligned");
  const Fp8Layout L = fp8_layout(B, H, N, d);
  if (workspace_bytes < L.total)
    return fail(FATTN_EWORKSPACE, "workspace of %zu bytes, %zu required", workspace_bytes, L.total);
  FATTN_TRY(check_device());
  const char* ws = (const char*)workspace;
  return hip_status(fattn::launch_fwd_fp8_attend(q, o, lse, (const uint8_t*)(ws + L.k8),
                                                 (const uint8_t*)(ws + L.v8t),
                                                 (const float*)(ws + L.scales), B, H, N, d,
                                                 causal != 0, scale,
                                                 exp_mode == FATTN_EXP_AUTO ? FATTN_EXP_HW : exp_mode,
                                                 rotate != 0, seed, (hipStream_t)stream),
                    "fattn_fwd_fp8_attend launch");
}

const char* fattn_strerror(int status) {
  switch (status) {
    case FATTN_OK: return "success";
    case FATTN_EINVAL: return "invalid argument";
    case FATTN_ENOTSUP: return "unsupported shape or option";
    case FATTN_EWORKSPACE: return "workspace missing or too small";
    case FATTN_EHIP: return "HIP runtime error";
    case FATTN_EDEVICE: return "device is not gfx950";
    default: return "unknown status";
  }
}

const char* fattn_last_error(void) { return g_last_error; }

int fattn_version(void) { return 400; }

}  // extern "C"
