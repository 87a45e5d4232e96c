// dq_internal.h -- private to libdq: tile layout, vector types and launchers.
//
// Packed weight layout (written by dq_repack_weights, read by the GEMMs).
// Weights are cut into tiles of 16 weight rows (n) x one 256-wide super-block
// (b); tiles are stored n-tile-major, so the tiles one n-tile needs over the
// whole reduction are contiguous:  tile(nt, b) at ((nt * nb) + b) * TILE_BYTES.
//
// Inside a tile every plane is laid out for the 16x16x64 int8 MFMA: lane l of
// a wave owns weight row n = l % 16 of the tile and the k-quarter kq = l / 16,
// i.e. for each of the 4 MFMA k-chunks c the 16 codes at k = 64kq + 16c + p
// (p = 0..15): lane quarter kq covers k in [64kq, 64kq + 64), so the matching
// activation bytes of one row are a single 64-byte run.  A 16-byte per-lane
// record holds the 4-bit parts of two chunks: dword t (t = 0..3) covers chunk
// 2i + t/2 (record i), half h = t % 2, and its byte e (e = 0..3) carries code
// p = 8h + e in the low nibble and code p = 8h + 4 + e in the high nibble.
// Records are [i][lane][16 B].
//
//   Q4_K tile (2304 B = 16 x 144):
//     [0, 256)     heads: per row n, the 16 GGUF header bytes d, dmin, scales[12]
//     [256, 2304)  codes: 2 records x 64 lanes x 16 B (the layout above)
//   Q6_K tile (3360 B = 16 x 210):
//     [0, 2048)    low 4 bits of the codes: 2 records x 64 lanes x 16 B
//     [2048, 3072) high 2 bits: 1 record x 64 lanes x 16 B; dword t covers
//                  chunk t; its byte e holds the 2-bit parts of codes
//                  p = e, 4+e, 8+e, 12+e at bits 0, 2, 4, 6
//     [3072, 3328) scales: [kq][n] dword, byte c = scale of sub-block 4kq + c
//     [3328, 3360) d: [n] fp16
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dq {

constexpr int QK = 256;
constexpr int TILE_N = 16;
constexpr int Q4K_BLOCK = 144;
constexpr int Q6K_BLOCK = 210;
constexpr int Q4K_TILE = TILE_N * Q4K_BLOCK;  // 2304
constexpr int Q6K_TILE = TILE_N * Q6K_BLOCK;  // 3360
constexpr int Q4K_CODES_OFF = 256;
constexpr int Q6K_QH_OFF = 2048;
constexpr int Q6K_SC_OFF = 3072;
constexpr int Q6K_D_OFF = 3328;

// Quantized-activation records (the layout is part of the C ABI, see dq.h):
// one per (super-block, 16-row block), super-block-major.
constexpr int ACT_ROWS = 16;
constexpr int ACT_RECORD = 5120;
constexpr int ACT_SUMS_OFF = 4096;  // [16 rows][8 groups] binary16 (lo, hi)
constexpr int ACT_DX_OFF = 4608;    // [16 rows] binary32
constexpr int ACT_PAD_OFF = 4672;   // zero up to ACT_RECORD

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// The activation quantization rule of one 256-value block, shared by every
// kernel that quantizes (so their codes agree bit for bit).  A wave holds the
// block with lane l owning values 4l .. 4l+3.

// Cross-lane moves inside a row of 16 lanes (DPP): quad permutations
// [1,0,3,2] and [2,3,0,1], half-row mirror (lane i <-> 7-i of each 8) and
// row mirror (lane i <-> 15-i).  Broadcasts of lane 15 / 31 into the next
// row(s) finish a reduction over the wave in lane 63.
constexpr int DPP_QUAD_1032 = 0xb1, DPP_QUAD_2301 = 0x4e;
constexpr int DPP_ROW_HALF_MIRROR = 0x141, DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;

template <int CTRL, int ROW_MASK = 0xf>
__device__ inline int dpp(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xf, false);
}

// max |x| over the wave (max is exact in any order), the same in every lane
__device__ inline float wave_max(float v) {
  auto step = [](float a, int b) { return fmaxf(a, __builtin_bit_cast(float, b)); };
  v = step(v, dpp<DPP_QUAD_1032>(__builtin_bit_cast(int, v)));
  v = step(v, dpp<DPP_QUAD_2301>(__builtin_bit_cast(int, v)));
  v = step(v, dpp<DPP_ROW_HALF_MIRROR>(__builtin_bit_cast(int, v)));
  v = step(v, dpp<DPP_ROW_MIRROR>(__builtin_bit_cast(int, v)));
  // lanes of rows 1 and 3 take the max with lane 15 of the row before, then
  // rows 2 and 3 with lane 31: lane 63 holds the maximum of all 64 lanes
  v = step(v, dpp<DPP_ROW_BCAST15, 0xa>(__builtin_bit_cast(int, v)));
  v = step(v, dpp<DPP_ROW_BCAST31, 0xc>(__builtin_bit_cast(int, v)));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// The block's max |x| (every lane of the wave takes part).
__device__ inline float block_amax(const float (&v)[4]) {
  return wave_max(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
}

// The lane's 4 codes, packed in k order: inv = 127 / amax (one correctly
// rounded division), q = clamp(rint(x * inv), -127, 127) (one multiply, ties
// to even); all zero when amax is 0.  No step can be contracted.
__device__ inline void quant4(const float (&v)[4], float amax, int (&c)[4]) {
  c[0] = c[1] = c[2] = c[3] = 0;
  if (amax != 0.0f) {
    const float inv = 127.0f / amax;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float t = __builtin_rintf(v[i] * inv);
      t = fminf(fmaxf(t, -127.0f), 127.0f);
      c[i] = (int)t;
    }
  }
}

__device__ inline uint32_t pack4(const int (&c)[4]) {
  return (uint32_t)(c[0] & 255) | ((uint32_t)(c[1] & 255) << 8) |
         ((uint32_t)(c[2] & 255) << 16) | ((uint32_t)(c[3] & 255) << 24);
}

// The block's activation scale d_x.
__device__ inline float block_dx(float amax) { return amax != 0.0f ? amax / 127.0f : 0.0f; }

// exp as the SwiGLU producer defines it: clamp t to [-87, 88]; n = rint(t *
// log2 e); r = (t - n*L1) - n*L2, where L1 + L2 = ln 2 and L1 has few enough
// significant bits that n*L1 is exact (Cody and Waite's reduction); the
// degree-7 Taylor polynomial of e^r (coefficients 1/k! in binary32) by
// Horner; times 2^n, built exactly from its exponent bits.  Every step is
// one binary32 operation, never contracted, so every kernel that includes
// this computes the same bits.
__device__ inline float dq_exp(float t) {
#pragma clang fp contract(off)
  t = fminf(fmaxf(t, -87.0f), 88.0f);
  const float n = __builtin_rintf(t * 1.44269502f);
  const float r = (t - n * 0.693145751953125f) - n * 1.42860677e-06f;
  float p = 1.98412698e-04f;
  p = p * r + 1.38888889e-03f;
  p = p * r + 8.33333377e-03f;
  p = p * r + 4.16666679e-02f;
  p = p * r + 1.66666672e-01f;
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  return p * __builtin_bit_cast(float, (uint32_t)((int)n + 127) << 23);
}

// silu(g) * u = (g / (1 + exp(-g))) * u, the down projection's input
__device__ inline float silu_mul(float g, float u) {
#pragma clang fp contract(off)
  const float den = 1.0f + dq_exp(-g);
  const float s = g / den;
  return s * u;
}

// Compute units and XCDs (each with its own L2) of the current device, queried
// once per device (device.hip); {256, 8} -- a whole MI355X -- if the query
// fails.  The launchers size persistent grids and XCD-aware placements by it.
struct DeviceProps {
  int cus = 256;
  int xcds = 8;
};
DeviceProps device_props();

// Launchers (each returns the hipError_t of its launch).
// Quantize M rows (row m = x[m], or x[idx[m]] when idx is given) into the
// record layout; err[m] flags an index outside [0, L).
hipError_t launch_quantize(int64_t M, int64_t K, const float *x, int64_t ldx, const int32_t *idx,
                           int64_t L, uint8_t *qa, int32_t *err, hipStream_t stream);
hipError_t launch_swiglu_quantize(int64_t M, int64_t F, const float *gu, int64_t ldgu,
                                  uint8_t *qa, hipStream_t stream);
// The RMSNorm producer keeps one sum of squares per 256-block of a row in
// LDS: rows of at most NORM_MAX_BLOCKS blocks (K <= 262144).
constexpr int NORM_MAX_BLOCKS = 1024;
hipError_t launch_rmsnorm_quantize(int64_t M, int64_t K, const float *x, int64_t ldx,
                                   const float *gamma, float eps, uint8_t *qa,
                                   hipStream_t stream);
hipError_t launch_repack(int type, int64_t N, int64_t K, const uint8_t *src, uint8_t *dst,
                         hipStream_t stream);
// mode: 0 canvas GEMM, 1 gathered-row GEMM, 2 debug stores of the exact integers
// (with sub >= 0: every sub-block scale replaced by 1 for sub-block sub and 0
// for the rest, S alone stored as that sub-block's dot, J per super-block),
// 4 canvas GEMM over interleaved gate/up tiles storing silu(gate) * up (y is
// then M x N/2, row stride ldy).
hipError_t launch_qgemm(int type, int mode, int64_t M, int64_t N, int64_t K, const uint8_t *qa,
                        const uint8_t *packed, float *y, int64_t ldy, int32_t *dbg_S,
                        int32_t *dbg_Mn, hipStream_t stream, int sub = -1);

}  // namespace dq
