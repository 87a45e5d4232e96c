// embed.hip -- embedding rows: the rows of a GGUF table selected by token id,
// decoded to f32 (mojo-dllm "Architecture" page, "A forward pass", step 1:
// embedding rows are decoded from the memory-mapped Q4_K table, one row per
// token; "Source map": scalar F32 / F16 / BF16 / Q8_0 / Q4_K / Q5_K / Q6_K
// decoders).  The table is in GGUF bytes as loaded (not repacked): N rows of
// row_bytes(type, K) bytes.  Every decoded value is the exactly rounded
// binary32 of its definition:
//   F32, F16, BF16, Q8_0 (d q) and Q6_K (d (sc (q - 32)), the integer product
//   first) are exact in binary32; Q4_K and Q5_K form d sc q and dmin m exactly
//   and round their difference once.
// One wave per (row, 256 consecutive values); lane l decodes values 4l .. 4l+3
// and stores them as one 16-byte segment.  HBM-bound: the selected rows'
// bytes in, 4 bytes per value out.
#include "embed.h"

#include "dq_internal.h"

namespace dq {
namespace {

__device__ inline float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(bits16 & 0xffffu));
}

__device__ inline uint32_t ld_u16(const uint8_t *p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8);
}

// 6-bit scale and min of sub-block j from the 12 packed bytes s (Q4_K, Q5_K).
__device__ inline void scale_min(const uint8_t *s, int j, int &sc, int &mn) {
  if (j < 4) {
    sc = s[j] & 63;
    mn = s[j + 4] & 63;
  } else {
    sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
    mn = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
  }
}

// d sc q - dmin m with both products exact in binary32, one rounding.
__device__ inline float kq_value(float dsc, int q, float dm) {
  return __fsub_rn(__fmul_rn(dsc, (float)q), dm);
}

template <int TYPE>
__device__ inline void decode4(const uint8_t *row, int sp, int lane, float v[4]) {
  const int i0 = 256 * sp + 4 * lane;  // first value of this lane in the row
  if (TYPE == 0) {                     // F32
    const float4 x = *reinterpret_cast<const float4 *>(row + 4 * (int64_t)i0);
    v[0] = x.x, v[1] = x.y, v[2] = x.z, v[3] = x.w;
  } else if (TYPE == 1 || TYPE == 30) {  // F16, BF16
    const uint2 x = *reinterpret_cast<const uint2 *>(row + 2 * (int64_t)i0);
    const uint32_t h[4] = {x.x & 0xffffu, x.x >> 16, x.y & 0xffffu, x.y >> 16};
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = TYPE == 1 ? h2f(h[e]) : __uint_as_float(h[e] << 16);
  } else if (TYPE == 8) {  // Q8_0: 34-byte blocks of 32, 2-byte aligned
    const uint8_t *blk = row + (int64_t)(i0 / 32) * 34;
    const float d = h2f(ld_u16(blk));
    const int o = 2 + (i0 % 32);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __fmul_rn(d, (float)(int8_t)blk[o + e]);
  } else if (TYPE == 12 || TYPE == 13) {  // Q4_K, Q5_K
    constexpr int BB = TYPE == 12 ? 144 : 176;
    constexpr int QS = TYPE == 12 ? 16 : 48;
    const uint8_t *blk = row + (int64_t)sp * BB;
    const int i = 4 * lane, c = i / 64, r = i % 64, j = i / 32;
    int sc, mn;
    scale_min(blk + 4, j, sc, mn);
    const float dsc = __fmul_rn(h2f(ld_u16(blk)), (float)sc);
    const float dm = __fmul_rn(h2f(ld_u16(blk + 2)), (float)mn);
    const uint32_t qs = *reinterpret_cast<const uint32_t *>(blk + QS + 32 * c + (r % 32));
    const int sh = r >= 32 ? 4 : 0;
    uint32_t hb = 0;
    if (TYPE == 13) hb = *reinterpret_cast<const uint32_t *>(blk + 16 + (r % 32));
    const int bit = 2 * c + (r >= 32 ? 1 : 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int q = (qs >> (8 * e + sh)) & 15;
      if (TYPE == 13) q |= ((hb >> (8 * e + bit)) & 1) << 4;
      v[e] = kq_value(dsc, q, dm);
    }
  } else {  // Q6_K: 210-byte blocks, 2-byte aligned
    const uint8_t *blk = row + (int64_t)sp * 210;
    const int i = 4 * lane, h = i / 128, quarter = (i % 128) / 32, l0 = i % 32;
    const float d = h2f(ld_u16(blk + 208));
    const int sc = (int8_t)blk[192 + i / 16];
    const uint8_t *ql = blk + 64 * h + l0 + ((quarter & 1) ? 32 : 0);
    const uint8_t *qh = blk + 128 + 32 * h + l0;
    const int qsh = quarter >= 2 ? 4 : 0, hsh = 2 * quarter;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int q = ((ql[e] >> qsh) & 15) | (((qh[e] >> hsh) & 3) << 4);
      v[e] = __fmul_rn(d, (float)(sc * (q - 32)));
    }
  }
}

template <int TYPE>
__global__ __launch_bounds__(256) void embed_rows_kernel(int64_t N, int64_t K,
                                                         const uint8_t *__restrict__ table,
                                                         int64_t row_bytes,
                                                         const int32_t *__restrict__ ids,
                                                         int64_t M, float *__restrict__ out,
                                                         int64_t ldo, int32_t *__restrict__ flag,
                                                         int out_vec) {
  const int lane = threadIdx.x & 63;
  const int64_t spans = K / 256;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= M * spans) return;
  const int64_t i = w / spans;
  const int sp = (int)(w - i * spans);
  const int64_t id = ids[i];
  const bool ok = id >= 0 && id < N;
  if (flag && sp == 0 && lane == 0) flag[i] = ok ? 0 : 1;
  float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (ok) decode4<TYPE>(table + id * row_bytes, sp, lane, v);
  float *o = out + i * ldo + 256 * (int64_t)sp + 4 * lane;
  if (out_vec) {
    *reinterpret_cast<float4 *>(o) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = v[e];
  }
}

template <int TYPE>
hipError_t launch_type(int64_t N, int64_t K, const uint8_t *table, const int32_t *ids,
                       int64_t M, float *out, int64_t ldo, int32_t *flag, hipStream_t stream) {
  const int64_t waves = M * (K / 256);
  const int out_vec = (reinterpret_cast<uintptr_t>(out) % 16 == 0) && (ldo % 4 == 0);
  hipLaunchKernelGGL(embed_rows_kernel<TYPE>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                     stream, N, K, table, embed_row_bytes(TYPE, K), ids, M, out, ldo, flag,
                     out_vec);
  return hipGetLastError();
}

}  // namespace

int64_t embed_row_bytes(int type, int64_t K) {
  if (K <= 0 || K % 256) return 0;
  switch (type) {
    case 0: return 4 * K;
    case 1:
    case 30: return 2 * K;
    case 8: return K / 32 * 34;
    case 12: return K / 256 * 144;
    case 13: return K / 256 * 176;
    case 14: return K / 256 * 210;
    default: return 0;
  }
}

hipError_t launch_embed_rows(int type, int64_t N, int64_t K, const uint8_t *table,
                             const int32_t *ids, int64_t M, float *out, int64_t ldo,
                             int32_t *flag, hipStream_t stream) {
  switch (type) {
    case 0: return launch_type<0>(N, K, table, ids, M, out, ldo, flag, stream);
    case 1: return launch_type<1>(N, K, table, ids, M, out, ldo, flag, stream);
    case 8: return launch_type<8>(N, K, table, ids, M, out, ldo, flag, stream);
    case 12: return launch_type<12>(N, K, table, ids, M, out, ldo, flag, stream);
    case 13: return launch_type<13>(N, K, table, ids, M, out, ldo, flag, stream);
    case 14: return launch_type<14>(N, K, table, ids, M, out, ldo, flag, stream);
    default: return launch_type<30>(N, K, table, ids, M, out, ldo, flag, stream);
  }
}

}  // namespace dq
