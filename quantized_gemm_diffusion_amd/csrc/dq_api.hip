// dq_api.hip -- the C ABI of libdq (declared in include/dq.h): argument
// checks on the host, then one or two kernel launches on the caller's stream.
// Nothing here allocates device memory or synchronizes.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "dq.h"
#include "attention.h"
#include "dq_internal.h"
#include "embed.h"
#include "row_stats.h"

namespace {

thread_local char g_err[256] = "";

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = 0;
  return DQ_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int block_bytes(int type) { return type == DQ_Q4_K ? dq::Q4K_BLOCK : dq::Q6K_BLOCK; }

int check_type(int type) {
  if (type != DQ_Q4_K && type != DQ_Q6_K)
    return fail(DQ_EUNSUPPORTED, "unsupported weight type %d (Q4_K = 12, Q6_K = 14)", type);
  return DQ_OK;
}

int check_k(int64_t K) {
  if (K <= 0 || K % dq::QK)
    return fail(DQ_EINVAL, "K = %lld must be a positive multiple of 256", (long long)K);
  if (K > (int64_t)1 << 24) return fail(DQ_EINVAL, "K = %lld too large", (long long)K);
  return DQ_OK;
}

int launched(hipError_t e, const char *what) {
  if (e != hipSuccess)
    return fail(DQ_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr int64_t kMaxRows = (int64_t)1 << 30;

}  // namespace

extern "C" {

const char *dq_status_string(int status) {
  switch (status) {
    case DQ_OK: return "DQ_OK";
    case DQ_EINVAL: return "DQ_EINVAL";
    case DQ_EUNSUPPORTED: return "DQ_EUNSUPPORTED";
    case DQ_EWORKSPACE: return "DQ_EWORKSPACE";
    case DQ_EHIP: return "DQ_EHIP";
    default: return "DQ_UNKNOWN";
  }
}

const char *dq_last_error(void) { return g_err; }

int dq_packed_size(int type, int64_t N, int64_t K, size_t *bytes) {
  if (int s = check_type(type)) return s;
  if (int s = check_k(K)) return s;
  if (N < 0 || N > kMaxRows) return fail(DQ_EINVAL, "N = %lld out of range", (long long)N);
  if (!bytes) return fail(DQ_EINVAL, "bytes is NULL");
  const int64_t ntiles = (N + dq::TILE_N - 1) / dq::TILE_N;
  *bytes = (size_t)ntiles * dq::TILE_N * (size_t)(K / dq::QK) * (size_t)block_bytes(type);
  return ok();
}

int dq_repack_weights(int type, int64_t N, int64_t K, const void *gguf, void *packed,
                      hipStream_t stream) {
  size_t bytes = 0;
  if (int s = dq_packed_size(type, N, K, &bytes)) return s;
  if (N == 0) return ok();
  if (!gguf || !packed) return fail(DQ_EINVAL, "gguf or packed is NULL");
  if (!aligned(packed, 16)) return fail(DQ_EINVAL, "packed must be 16-byte aligned");
  const uint8_t *s = static_cast<const uint8_t *>(gguf);
  const uint8_t *p = static_cast<const uint8_t *>(packed);
  const size_t src_bytes = (size_t)N * (size_t)(K / dq::QK) * (size_t)block_bytes(type);
  if (s < p + bytes && p < s + src_bytes) return fail(DQ_EINVAL, "gguf and packed overlap");
  if (K / dq::QK > 65535) return fail(DQ_EINVAL, "K too large for the repack grid");
  return launched(dq::launch_repack(type, N, K, s, static_cast<uint8_t *>(packed), stream),
                  "dq_repack_weights");
}

// Bytes of the quantized-activation records of M rows of length K; the GEMM
// addresses them with 32-bit offsets.
static int act_bytes(int64_t M, int64_t K, size_t *bytes) {
  const int64_t nmb = (M + dq::ACT_ROWS - 1) / dq::ACT_ROWS;
  const int64_t total = nmb * (K / dq::QK) * dq::ACT_RECORD;
  if (total > INT32_MAX)
    return fail(DQ_EINVAL, "M = %lld x K = %lld too large for one activation buffer",
                (long long)M, (long long)K);
  *bytes = (size_t)total;
  return DQ_OK;
}

int dq_act_size(int64_t M, int64_t K, size_t *bytes) {
  if (int s = check_k(K)) return s;
  if (M < 0 || M > kMaxRows) return fail(DQ_EINVAL, "M = %lld out of range", (long long)M);
  if (!bytes) return fail(DQ_EINVAL, "bytes is NULL");
  if (int s = act_bytes(M, K, bytes)) return s;
  return ok();
}

int dq_quantize_act(int64_t M, int64_t K, const float *x, int64_t ldx, void *qa,
                    hipStream_t stream) {
  size_t bytes = 0;
  if (int s = dq_act_size(M, K, &bytes)) return s;
  if (ldx < K) return fail(DQ_EINVAL, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  if (M == 0) return ok();
  if (!x || !qa) return fail(DQ_EINVAL, "NULL pointer argument");
  if (!aligned(qa, 16) || !aligned(x, 4))
    return fail(DQ_EINVAL, "qa must be 16-byte aligned, x 4-byte aligned");
  return launched(dq::launch_quantize(M, K, x, ldx, nullptr, 0, static_cast<uint8_t *>(qa),
                                      nullptr, stream),
                  "dq_quantize_act");
}

int dq_swiglu_quantize_act(int64_t M, int64_t F, const float *gu, int64_t ldgu, void *qa,
                           hipStream_t stream) {
  size_t bytes = 0;
  if (int s = dq_act_size(M, F, &bytes)) return s;
  if (ldgu < 2 * F)
    return fail(DQ_EINVAL, "ldgu = %lld < 2F = %lld", (long long)ldgu, (long long)(2 * F));
  if (M == 0) return ok();
  if (!gu || !qa) return fail(DQ_EINVAL, "NULL pointer argument");
  if (!aligned(qa, 16) || !aligned(gu, 4))
    return fail(DQ_EINVAL, "qa must be 16-byte aligned, gu 4-byte aligned");
  return launched(dq::launch_swiglu_quantize(M, F, gu, ldgu, static_cast<uint8_t *>(qa), stream),
                  "dq_swiglu_quantize_act");
}

int dq_rmsnorm_quantize_act(int64_t M, int64_t K, const float *x, int64_t ldx,
                            const float *gamma, float eps, void *qa, hipStream_t stream) {
  size_t bytes = 0;
  if (int s = dq_act_size(M, K, &bytes)) return s;
  if (ldx < K) return fail(DQ_EINVAL, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  if (K > (int64_t)dq::NORM_MAX_BLOCKS * dq::QK)
    return fail(DQ_EINVAL, "K = %lld too large for the RMSNorm producer (at most %lld)",
                (long long)K, (long long)dq::NORM_MAX_BLOCKS * dq::QK);
  if (!(eps >= 0.0f) || !isfinite(eps)) return fail(DQ_EINVAL, "eps must be finite and >= 0");
  if (M == 0) return ok();
  if (!x || !gamma || !qa) return fail(DQ_EINVAL, "NULL pointer argument");
  if (!aligned(qa, 16) || !aligned(x, 4) || !aligned(gamma, 4))
    return fail(DQ_EINVAL, "qa must be 16-byte aligned, x and gamma 4-byte aligned");
  return launched(dq::launch_rmsnorm_quantize(M, K, x, ldx, gamma, eps, static_cast<uint8_t *>(qa),
                                              stream),
                  "dq_rmsnorm_quantize_act");
}

static int check_gemm(int type, int64_t M, int64_t N, int64_t K, const void *qa,
                      const void *packed) {
  if (int s = check_type(type)) return s;
  if (int s = check_k(K)) return s;
  if (M < 0 || M > kMaxRows) return fail(DQ_EINVAL, "M = %lld out of range", (long long)M);
  if (N < 0 || N > kMaxRows) return fail(DQ_EINVAL, "N = %lld out of range", (long long)N);
  size_t bytes = 0;
  if (int s = act_bytes(M, K, &bytes)) return s;
  // the canvas GEMM's one-dimensional grid: at most (N/32) x (M/16) workgroups
  // of at most 512 work-items, all numbered in 32 bits
  const int64_t ncg = (N + 2 * dq::TILE_N - 1) / (2 * dq::TILE_N);
  const int64_t nmb = (M + dq::ACT_ROWS - 1) / dq::ACT_ROWS;
  if (ncg * nmb * 512 > (int64_t)UINT32_MAX)
    return fail(DQ_EINVAL, "M or N too large for the GEMM grid");
  if ((K / dq::QK) * (int64_t)dq::Q6K_TILE > INT32_MAX)
    return fail(DQ_EINVAL, "K too large for the GEMM's 32-bit tile offsets");
  if (M == 0 || N == 0) return DQ_OK;
  if (!qa || !packed) return fail(DQ_EINVAL, "NULL pointer argument");
  if (!aligned(qa, 16) || !aligned(packed, 16))
    return fail(DQ_EINVAL, "qa and packed must be 16-byte aligned");
  return DQ_OK;
}

int dq_qgemm(int type, int64_t M, int64_t N, int64_t K, const void *qa, const void *packed,
             float *y, int64_t ldy, hipStream_t stream) {
  if (int s = check_gemm(type, M, N, K, qa, packed)) return s;
  if (ldy < N) return fail(DQ_EINVAL, "ldy = %lld < N = %lld", (long long)ldy, (long long)N);
  if (M == 0 || N == 0) return ok();
  if (!y || !aligned(y, 4)) return fail(DQ_EINVAL, "y is NULL or not 4-byte aligned");
  return launched(dq::launch_qgemm(type, 0, M, N, K, static_cast<const uint8_t *>(qa),
                                   static_cast<const uint8_t *>(packed), y, ldy, nullptr, nullptr,
                                   stream),
                  "dq_qgemm");
}

int dq_qgemm_swiglu(int type, int64_t M, int64_t F, int64_t K, const void *qa,
                    const void *packed, float *h, int64_t ldh, hipStream_t stream) {
  if (F < 0 || F % 16 != 0 || F > kMaxRows / 2)
    return fail(DQ_EINVAL, "F = %lld is not a multiple of 16 in range", (long long)F);
  if (int s = check_gemm(type, M, 2 * F, K, qa, packed)) return s;
  if (ldh < F) return fail(DQ_EINVAL, "ldh = %lld < F = %lld", (long long)ldh, (long long)F);
  if (M == 0 || F == 0) return ok();
  if (!h || !aligned(h, 4)) return fail(DQ_EINVAL, "h is NULL or not 4-byte aligned");
  return launched(dq::launch_qgemm(type, 4, M, 2 * F, K, static_cast<const uint8_t *>(qa),
                                   static_cast<const uint8_t *>(packed), h, ldh, nullptr, nullptr,
                                   stream),
                  "dq_qgemm_swiglu");
}

// Workspace: [flags int32 x M | pad to 256] [quantized-activation records]
static size_t rows_ws_flags(int64_t M) { return ((size_t)M * 4 + 255) & ~(size_t)255; }

int dq_qgemm_rows_workspace(int64_t M, int64_t K, size_t *bytes) {
  if (int s = check_k(K)) return s;
  if (M < 0 || M > kMaxRows) return fail(DQ_EINVAL, "M = %lld out of range", (long long)M);
  if (!bytes) return fail(DQ_EINVAL, "bytes is NULL");
  size_t act = 0;
  if (int s = act_bytes(M, K, &act)) return s;
  *bytes = rows_ws_flags(M) + act;
  return ok();
}

// Arguments of the gathered-row projection, checked; M == 0 or N == 0 is a
// valid no-op (returns DQ_OK with *noop set).
static int check_rows(int type, int64_t L, int64_t M, int64_t N, int64_t K, const float *canvas,
                      int64_t ldc, const int32_t *idx, const void *packed, const float *y,
                      int64_t ldy, bool *noop) {
  *noop = true;
  if (int s = check_type(type)) return s;
  if (int s = check_k(K)) return s;
  if (L < 0 || L > kMaxRows) return fail(DQ_EINVAL, "L = %lld out of range", (long long)L);
  if (M < 0 || M > kMaxRows) return fail(DQ_EINVAL, "M = %lld out of range", (long long)M);
  if (N < 0 || N > kMaxRows) return fail(DQ_EINVAL, "N = %lld out of range", (long long)N);
  if (ldc < K) return fail(DQ_EINVAL, "ldc = %lld < K = %lld", (long long)ldc, (long long)K);
  if (ldy < N) return fail(DQ_EINVAL, "ldy = %lld < N = %lld", (long long)ldy, (long long)N);
  if (M == 0 || N == 0) return DQ_OK;
  if (!canvas || !idx || !packed || !y) return fail(DQ_EINVAL, "NULL pointer argument");
  if (!aligned(canvas, 4) || !aligned(idx, 4) || !aligned(y, 4) || !aligned(packed, 16))
    return fail(DQ_EINVAL, "canvas, idx, y must be 4-byte aligned, packed 16-byte aligned");
  *noop = false;
  return DQ_OK;
}

// The launches of the gathered-row projection: flags[M] and the records qa of
// the gathered rows are device memory the caller of this function provides.
static int rows_launch(int type, int64_t L, int64_t M, int64_t N, int64_t K, const float *canvas,
                       int64_t ldc, const int32_t *idx, const void *packed, float *y, int64_t ldy,
                       int32_t *flags, uint8_t *qa, hipStream_t stream, const char *who) {
  if (int s = check_gemm(type, M, N, K, qa, packed)) return s;
  hipError_t e = hipSuccess;
  if (dq::launch_rows_gather_row1(type, M, N, K, canvas, ldc, idx, L, flags,
                                  static_cast<const uint8_t *>(packed), y, 0.0f, nullptr, stream,
                                  e))
    return launched(e, who);
  e = dq::launch_quantize(M, K, canvas, ldc, idx, L, qa, flags, stream);
  if (e != hipSuccess) return launched(e, who);
  return launched(dq::launch_qgemm(type, 1, M, N, K, qa, static_cast<const uint8_t *>(packed), y,
                                   ldy, nullptr, nullptr, stream),
                  who);
}

int dq_qgemm_rows(int type, int64_t L, int64_t M, int64_t N, int64_t K, const float *canvas,
                  int64_t ldc, const int32_t *idx, const void *packed, float *y, int64_t ldy,
                  void *ws, size_t ws_bytes, hipStream_t stream) {
  bool noop = true;
  if (int s = check_rows(type, L, M, N, K, canvas, ldc, idx, packed, y, ldy, &noop)) return s;
  if (noop) return ok();
  size_t need = 0;
  if (int s = dq_qgemm_rows_workspace(M, K, &need)) return s;
  if (!ws || ws_bytes < need)
    return fail(DQ_EWORKSPACE, "workspace needs %zu bytes, got %zu", need, ws ? ws_bytes : 0);
  if (!aligned(ws, 256)) return fail(DQ_EINVAL, "workspace must be 256-byte aligned");
  uint8_t *w = static_cast<uint8_t *>(ws);
  return rows_launch(type, L, M, N, K, canvas, ldc, idx, packed, y, ldy,
                     reinterpret_cast<int32_t *>(w), w + rows_ws_flags(M), stream,
                     "dq_qgemm_rows");
}

// ---------------------------------------------------------------------------
// dq_qgemm_rows_noalloc: the gathered-row projection with its workspace in a
// file-scope device array (one copy per GPU, held until the process ends)
// instead of caller memory.  The array's name is a host-side stand-in; its
// device address is looked up once per device, with that device current, and
// only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[DQ_NOALLOC_SCRATCH_BYTES];

static int scratch_address(hipStream_t stream, uint8_t **out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DQ_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DQ_EHIP, "device %d out of range", dev);
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(DQ_EHIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if ((int)sdev != dev)
      return fail(DQ_EINVAL, "stream belongs to device %d, the current device is %d", (int)sdev,
                  dev);
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DQ_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = static_cast<uint8_t *>(addr[dev]);
  return DQ_OK;
}

int dq_qgemm_rows_noalloc(int type, int64_t L, int64_t M, int64_t N, int64_t K,
                          const float *canvas, int64_t ldc, const int32_t *idx,
                          const void *packed, float *y, int64_t ldy, int32_t *flags,
                          hipStream_t stream) {
  bool noop = true;
  if (int s = check_rows(type, L, M, N, K, canvas, ldc, idx, packed, y, ldy, &noop)) return s;
  if (noop) return ok();
  if (flags && !aligned(flags, 4)) return fail(DQ_EINVAL, "flags must be 4-byte aligned");
  size_t act = 0;
  if (int s = act_bytes(M, K, &act)) return s;
  const size_t fbytes = flags ? 0 : rows_ws_flags(M);
  if (fbytes + act > (size_t)DQ_NOALLOC_SCRATCH_BYTES)
    return fail(DQ_EWORKSPACE,
                "M = %lld rows of K = %lld need %zu bytes of scratch, more than the %u built in",
                (long long)M, (long long)K, fbytes + act, (unsigned)DQ_NOALLOC_SCRATCH_BYTES);
  uint8_t *w = nullptr;
  if (int s = scratch_address(stream, &w)) return s;
  int32_t *f = flags ? flags : reinterpret_cast<int32_t *>(w);
  return rows_launch(type, L, M, N, K, canvas, ldc, idx, packed, y, ldy, f, w + fbytes, stream,
                     "dq_qgemm_rows_noalloc");
}

static int check_beta(float beta) {
  if (!(beta > 0.0f) || !isfinite(beta)) return fail(DQ_EINVAL, "beta must be finite and > 0");
  return DQ_OK;
}

static size_t stats_part_bytes(int64_t M, int64_t npart) {
  return (size_t)M * (size_t)npart * sizeof(float4);
}

int dq_logits_stats_workspace(int64_t M, int64_t N, size_t *bytes) {
  if (M < 0 || M > kMaxRows) return fail(DQ_EINVAL, "M = %lld out of range", (long long)M);
  if (N < 1 || N > kMaxRows) return fail(DQ_EINVAL, "N = %lld out of range", (long long)N);
  if (!bytes) return fail(DQ_EINVAL, "bytes is NULL");
  *bytes = stats_part_bytes(M, dq::logits_stats_parts(N));
  return ok();
}

int dq_logits_stats(int64_t M, int64_t N, const float *y, int64_t ldy, float beta,
                    int32_t *token, float *stats, void *ws, size_t ws_bytes, hipStream_t stream) {
  size_t need = 0;
  if (int s = dq_logits_stats_workspace(M, N, &need)) return s;
  if (ldy < N) return fail(DQ_EINVAL, "ldy = %lld < N = %lld", (long long)ldy, (long long)N);
  if (int s = check_beta(beta)) return s;
  const int npart = dq::logits_stats_parts(N);
  // one workgroup of 256 work-items per (row, partial), numbered in 32 bits
  if (M * npart * 256 > (int64_t)UINT32_MAX) return fail(DQ_EINVAL, "too many rows for one launch");
  if (M == 0) return ok();
  if (!y || !token || !stats) return fail(DQ_EINVAL, "NULL pointer argument");
  if (!aligned(y, 4) || !aligned(token, 4) || !aligned(stats, 4))
    return fail(DQ_EINVAL, "y, token and stats must be 4-byte aligned");
  if (!ws || ws_bytes < need)
    return fail(DQ_EWORKSPACE, "workspace needs %zu bytes, got %zu", need, ws ? ws_bytes : 0);
  if (!aligned(ws, 16)) return fail(DQ_EINVAL, "workspace must be 16-byte aligned");
  float4 *part = static_cast<float4 *>(ws);
  hipError_t e = dq::launch_logits_stats_partial(M, N, y, ldy, beta, npart, part, stream);
  if (e != hipSuccess) return launched(e, "dq_logits_stats (partials)");
  return launched(dq::launch_row_stats_finish(M, npart, part, token, stats, stream),
                  "dq_logits_stats (finish)");
}

// Workspace: [flags | quantized-activation records | partial states], the
// first two as for dq_qgemm_rows, the states 16-byte aligned after them.
int dq_qgemm_rows_sample_workspace(int64_t M, int64_t N, int64_t K, size_t *bytes) {
  size_t rows = 0;
  if (N < 1 || N > kMaxRows) return fail(DQ_EINVAL, "N = %lld out of range", (long long)N);
  if (int s = dq_qgemm_rows_workspace(M, K, &rows)) return s;
  *bytes = rows + stats_part_bytes(M, dq::qgemm_stats_parts(M, N, K));
  return ok();
}

int dq_qgemm_rows_sample(int type, int64_t L, int64_t M, int64_t N, int64_t K,
                         const float *canvas, int64_t ldc, const int32_t *idx, const void *packed,
                         float beta, int32_t *token, float *stats, void *ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (int s = check_type(type)) return s;
  if (int s = check_k(K)) return s;
  if (L < 0 || L > kMaxRows) return fail(DQ_EINVAL, "L = %lld out of range", (long long)L);
  if (M < 0 || M > kMaxRows) return fail(DQ_EINVAL, "M = %lld out of range", (long long)M);
  if (N < 1 || N > kMaxRows) return fail(DQ_EINVAL, "N = %lld out of range", (long long)N);
  if (ldc < K) return fail(DQ_EINVAL, "ldc = %lld < K = %lld", (long long)ldc, (long long)K);
  if (int s = check_beta(beta)) return s;
  // the finish launch: one 256-wide workgroup per row
  if (M * 256 > (int64_t)UINT32_MAX) return fail(DQ_EINVAL, "too many rows for one launch");
  if (M == 0) return ok();
  if (!canvas || !idx || !packed || !token || !stats)
    return fail(DQ_EINVAL, "NULL pointer argument");
  if (!aligned(canvas, 4) || !aligned(idx, 4) || !aligned(token, 4) || !aligned(stats, 4) ||
      !aligned(packed, 16))
    return fail(DQ_EINVAL,
                "canvas, idx, token, stats must be 4-byte aligned, packed 16-byte aligned");
  size_t need = 0, rows = 0;
  if (int s = dq_qgemm_rows_sample_workspace(M, N, K, &need)) return s;
  if (int s = dq_qgemm_rows_workspace(M, K, &rows)) return s;
  if (!ws || ws_bytes < need)
    return fail(DQ_EWORKSPACE, "workspace needs %zu bytes, got %zu", need, ws ? ws_bytes : 0);
  if (!aligned(ws, 256)) return fail(DQ_EINVAL, "workspace must be 256-byte aligned");
  uint8_t *w = static_cast<uint8_t *>(ws);
  uint8_t *qa = w + rows_ws_flags(M);
  if (int s = check_gemm(type, M, N, K, qa, packed)) return s;
  int32_t *flags = reinterpret_cast<int32_t *>(w);
  float4 *part = reinterpret_cast<float4 *>(w + rows);
  const int npart = dq::qgemm_stats_parts(M, N, K);
  hipError_t e = hipSuccess;
  if (!dq::launch_rows_gather_row1(type, M, N, K, canvas, ldc, idx, L, flags,
                                   static_cast<const uint8_t *>(packed), nullptr, beta, part,
                                   stream, e)) {
    e = dq::launch_quantize(M, K, canvas, ldc, idx, L, qa, flags, stream);
    if (e != hipSuccess) return launched(e, "dq_qgemm_rows_sample (gather-quantize)");
    e = dq::launch_qgemm_stats(type, M, N, K, qa, static_cast<const uint8_t *>(packed), beta,
                               part, npart, stream);
  }
  if (e != hipSuccess) return launched(e, "dq_qgemm_rows_sample (gemm)");
  return launched(dq::launch_row_stats_finish(M, npart, part, token, stats, stream),
                  "dq_qgemm_rows_sample (finish)");
}

static int check_attention_shape(int64_t L, int64_t H, int64_t Hkv, int64_t D) {
  if (D != dq::ATTN_HEAD_DIM)
    return fail(DQ_EUNSUPPORTED, "head dimension %lld (only 128 is built)", (long long)D);
  if (L < 0 || L > ((int64_t)1 << 20)) return fail(DQ_EINVAL, "L = %lld out of range", (long long)L);
  if (H <= 0 || Hkv <= 0 || H % Hkv || H > 4096)
    return fail(DQ_EINVAL, "H = %lld, Hkv = %lld: need 0 < Hkv, Hkv divides H <= 4096",
                (long long)H, (long long)Hkv);
  // one kv head's key blocks are addressed with 32-bit offsets
  if (dq::attention_workspace_bytes(L, 1) > (int64_t)INT32_MAX)
    return fail(DQ_EINVAL, "L = %lld too long", (long long)L);
  return DQ_OK;
}

int dq_attention_workspace(int64_t L, int64_t H, int64_t Hkv, int64_t D, size_t *bytes) {
  if (int s = check_attention_shape(L, H, Hkv, D)) return s;
  if (!bytes) return fail(DQ_EINVAL, "bytes is NULL");
  *bytes = (size_t)dq::attention_workspace_bytes(L, Hkv);
  return ok();
}

int dq_attention(int64_t L, int64_t H, int64_t Hkv, int64_t D, const float *qkv, int64_t ldqkv,
                 const float *rope, int rope_mode, float *out, int64_t ldo, void *ws,
                 size_t ws_bytes, hipStream_t stream) {
  if (int s = check_attention_shape(L, H, Hkv, D)) return s;
  if (rope_mode < 0 || rope_mode > 2) return fail(DQ_EINVAL, "rope_mode %d not 0, 1 or 2", rope_mode);
  if (ldqkv < (H + 2 * Hkv) * D || ldqkv % 4)
    return fail(DQ_EINVAL, "ldqkv = %lld: need >= (H + 2 Hkv) D and a multiple of 4",
                (long long)ldqkv);
  if (ldo < H * D) return fail(DQ_EINVAL, "ldo = %lld < H D", (long long)ldo);
  if (L == 0) return ok();
  if (!qkv || !out || (rope_mode && !rope)) return fail(DQ_EINVAL, "NULL pointer argument");
  if (!aligned(qkv, 16) || !aligned(out, 4) || (rope_mode && !aligned(rope, 8)))
    return fail(DQ_EINVAL, "qkv must be 16-byte aligned, out 4-byte, rope 8-byte");
  const size_t need = (size_t)dq::attention_workspace_bytes(L, Hkv);
  if (!ws || ws_bytes < need)
    return fail(DQ_EWORKSPACE, "workspace needs %zu bytes, got %zu", need, ws ? ws_bytes : 0);
  if (!aligned(ws, 16)) return fail(DQ_EINVAL, "workspace must be 16-byte aligned");
  return launched(dq::launch_attention(L, H, Hkv, qkv, ldqkv, rope, rope_mode,
                                       static_cast<uint8_t *>(ws), out, ldo, stream),
                  "dq_attention");
}

int dq_row_bytes(int type, int64_t K, size_t *bytes) {
  if (type != 0 && type != 1 && type != 8 && type != 12 && type != 13 && type != 14 &&
      type != 30)
    return fail(DQ_EUNSUPPORTED, "GGUF type %d is not decoded (0, 1, 8, 12, 13, 14, 30 are)",
                type);
  if (K <= 0 || K % 256 || K > ((int64_t)1 << 24))
    return fail(DQ_EINVAL, "K = %lld must be a positive multiple of 256", (long long)K);
  if (!bytes) return fail(DQ_EINVAL, "bytes is NULL");
  *bytes = (size_t)dq::embed_row_bytes(type, K);
  return ok();
}

int dq_embed_rows(int type, int64_t N, int64_t K, const void *table, const int32_t *ids,
                  int64_t M, float *out, int64_t ldo, int32_t *flags, hipStream_t stream) {
  size_t rb = 0;
  if (int s = dq_row_bytes(type, K, &rb)) return s;
  if (N < 0 || N > kMaxRows) return fail(DQ_EINVAL, "N = %lld out of range", (long long)N);
  if (M < 0 || M > kMaxRows) return fail(DQ_EINVAL, "M = %lld out of range", (long long)M);
  if (ldo < K) return fail(DQ_EINVAL, "ldo = %lld < K = %lld", (long long)ldo, (long long)K);
  // one wave per (row, 256 values), four to a workgroup, numbered in 32 bits
  if (M * (K / 256) / 4 >= (int64_t)UINT32_MAX) return fail(DQ_EINVAL, "M x K too large");
  if (M == 0) return ok();
  if (!table || !ids || !out) return fail(DQ_EINVAL, "NULL pointer argument");
  if (!aligned(table, 16) || !aligned(ids, 4) || !aligned(out, 4) || (flags && !aligned(flags, 4)))
    return fail(DQ_EINVAL, "table must be 16-byte aligned, ids, out and flags 4-byte");
  return launched(dq::launch_embed_rows(type, N, K, static_cast<const uint8_t *>(table), ids, M,
                                        out, ldo, flags, stream),
                  "dq_embed_rows");
}

int dq_debug_superblock_sums(int type, int64_t M, int64_t N, int64_t K, const void *qa,
                             const void *packed, int32_t *S, int32_t *Mn, hipStream_t stream) {
  if (int s = check_gemm(type, M, N, K, qa, packed)) return s;
  if (M == 0 || N == 0) return ok();
  if (!S || !Mn || !aligned(S, 4) || !aligned(Mn, 4))
    return fail(DQ_EINVAL, "S and Mn must be non-NULL and 4-byte aligned");
  if ((int64_t)M * N * (K / dq::QK) > ((int64_t)1 << 40))
    return fail(DQ_EINVAL, "debug output too large");
  return launched(dq::launch_qgemm(type, 2, M, N, K, static_cast<const uint8_t *>(qa),
                                   static_cast<const uint8_t *>(packed), nullptr, N, S, Mn, stream),
                  "dq_debug_superblock_sums");
}

int dq_debug_subdots(int type, int64_t M, int64_t N, int64_t K, const void *qa,
                     const void *packed, int32_t *dots, hipStream_t stream) {
  if (int s = check_gemm(type, M, N, K, qa, packed)) return s;
  if (M == 0 || N == 0) return ok();
  if (!dots || !aligned(dots, 4)) return fail(DQ_EINVAL, "dots must be non-NULL and 4-byte aligned");
  const int J = type == DQ_Q4_K ? 8 : 16;
  if ((int64_t)M * N * (K / dq::QK) * J > ((int64_t)1 << 40))
    return fail(DQ_EINVAL, "debug output too large");
  // one launch per sub-block position, each storing that sub-block's dots
  for (int sub = 0; sub < J; ++sub) {
    const hipError_t e = dq::launch_qgemm(type, 2, M, N, K, static_cast<const uint8_t *>(qa),
                                          static_cast<const uint8_t *>(packed), nullptr, N, dots,
                                          dots, stream, sub);
    if (e != hipSuccess) return launched(e, "dq_debug_subdots");
  }
  return ok();
}

}  // extern "C"
