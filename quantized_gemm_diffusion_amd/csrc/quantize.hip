// quantize.hip -- f32 activations -> int8 codes, one binary32 scale per 256
// values, and int32 code sums per 32 (mojo-dllm "Architecture" page, "Source
// map": activation quantization, int8 with one scale per 256).  The gathered
// variant reads canvas row idx[m] for output row m ("A forward pass", steps
// 3-4: only the requested positions reach the output projection).
//
// One wave64 per (row, 256-block): each lane owns 4 consecutive values.  The
// block's max |x| is reduced across the wave (max is exact in any order),
// then every lane applies inv = 127/amax (IEEE division), rint (ties to even)
// and a clamp to [-127, 127]; the 8 lanes of each 32-group sum their codes.
// All arithmetic is binary32 with no contraction, so codes match any other
// binary32 implementation of the same steps bit for bit.
#include "dq_internal.h"

// every step below is one binary32 operation; nothing may be fused
#pragma clang fp contract(off)

namespace dq {
namespace {

constexpr int WAVES_PER_BLOCK = 4;

template <bool VEC, bool GATHER>
__global__ __launch_bounds__(256) void quantize_kernel(int64_t M, int nb, const float *__restrict__ x,
                                                       int64_t ldx, const int32_t *__restrict__ idx,
                                                       int64_t L, int8_t *__restrict__ q,
                                                       float *__restrict__ d,
                                                       int32_t *__restrict__ bsum,
                                                       int32_t *__restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * WAVES_PER_BLOCK + (threadIdx.x >> 6);
  if (item >= M * nb) return;  // whole wave exits together
  const int64_t m = item / nb;
  const int b = (int)(item - m * nb);
  const int64_t K = (int64_t)nb * QK;

  int64_t src = m;
  bool valid = true;
  if (GATHER) {
    const int32_t r = idx[m];
    valid = r >= 0 && (int64_t)r < L;
    src = valid ? r : 0;
    if (b == 0 && lane == 0) err[m] = valid ? 0 : 1;
  }

  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
    const float *xr = x + src * ldx + (int64_t)b * QK + 4 * lane;
    if (VEC) {
      const f32x4 t = *reinterpret_cast<const f32x4 *>(xr);
      v[0] = t[0];
      v[1] = t[1];
      v[2] = t[2];
      v[3] = t[3];
    } else {
      v[0] = xr[0];
      v[1] = xr[1];
      v[2] = xr[2];
      v[3] = xr[3];
    }
  }

  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));

  int c[4] = {0, 0, 0, 0};
  if (amax != 0.0f) {
    const float inv = 127.0f / amax;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float r = __builtin_rintf(v[i] * inv);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      c[i] = (int)r;
    }
  }
  const uint32_t packed = (uint32_t)(c[0] & 255) | ((uint32_t)(c[1] & 255) << 8) |
                          ((uint32_t)(c[2] & 255) << 16) | ((uint32_t)(c[3] & 255) << 24);
  *reinterpret_cast<uint32_t *>(q + m * K + (int64_t)b * QK + 4 * lane) = packed;

  int s = c[0] + c[1] + c[2] + c[3];
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  s += __shfl_xor(s, 4, 64);
  if ((lane & 7) == 0) bsum[m * (K / 32) + (int64_t)b * 8 + (lane >> 3)] = s;
  if (lane == 0) d[m * nb + b] = amax != 0.0f ? amax / 127.0f : 0.0f;
}

}  // namespace

hipError_t launch_quantize(int64_t M, int64_t K, const float *x, int64_t ldx, const int32_t *idx,
                           int64_t L, int8_t *q, float *d, int32_t *bsum, int32_t *err,
                           hipStream_t stream) {
  const int nb = (int)(K / QK);
  const int64_t items = M * nb;
  const int64_t blocks = (items + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  const bool vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (ldx % 4 == 0);
  dim3 grid((unsigned)blocks), block(64 * WAVES_PER_BLOCK);
  if (idx) {
    if (vec)
      hipLaunchKernelGGL((quantize_kernel<true, true>), grid, block, 0, stream, M, nb, x, ldx,
                         idx, L, q, d, bsum, err);
    else
      hipLaunchKernelGGL((quantize_kernel<false, true>), grid, block, 0, stream, M, nb, x, ldx,
                         idx, L, q, d, bsum, err);
  } else {
    if (vec)
      hipLaunchKernelGGL((quantize_kernel<true, false>), grid, block, 0, stream, M, nb, x, ldx,
                         idx, L, q, d, bsum, err);
    else
      hipLaunchKernelGGL((quantize_kernel<false, false>), grid, block, 0, stream, M, nb, x, ldx,
                         idx, L, q, d, bsum, err);
  }
  return hipGetLastError();
}

}  // namespace dq
