// quantize.hip -- f32 activations -> int8 codes, one binary32 scale per 256
// values, and code sums per 32 (mojo-dllm "Architecture" page, "Source map":
// activation quantization, int8 with one scale per 256), written in the
// record layout the GEMM loads (documented in dq.h).  The gathered variant
// reads canvas row idx[m] for output row m ("A forward pass", steps 3-4: only
// the requested positions reach the output projection).
//
// One wave64 per (row, 256-block), rows padded to a multiple of 16: each lane
// owns 4 consecutive values.  The block's max |x| is reduced across the wave
// with DPP lane moves (max is exact in any order), then every lane applies
// inv = 127/amax (IEEE division), rint (ties to even) and a clamp to
// [-127, 127]; the 8 lanes of each 32-group sum their codes.  All arithmetic is binary32 with no
// contraction, so codes match any other binary32 implementation of the same
// steps bit for bit.  Padding rows (m >= M) write zeros.
//
// Two fused producers run the same quantizer on what the layer computes just
// before a GEMM ("A forward pass", step 2: RMSNorm, then one quantization for
// Q, K and V; the FFN applies SiLU to gate, multiplies by up and quantizes
// again for down; "Source map": RMSNorm and SwiGLU among the GPU kernels).
// Each is a fixed sequence of binary32 operations, including the order of
// its reduction and its exponential, so the codes are reproducible exactly.
#include "dq_internal.h"

// every step below is one binary32 operation; nothing may be fused
#pragma clang fp contract(off)

namespace dq {
namespace {

constexpr int WAVES_PER_BLOCK = 4;

// sum over each group of 8 lanes (the 32 codes of one group), in every lane
__device__ inline int group8_sum(int s) {
  s += dpp<DPP_QUAD_1032>(s);
  s += dpp<DPP_QUAD_2301>(s);
  s += dpp<DPP_ROW_HALF_MIRROR>(s);
  return s;
}

// The quantizer for one (row, 256-block): lane l holds values 4l .. 4l+3 in
// v; the wave writes row r of the record at rec.  Every lane of the wave
// takes part (the maximum and the group sums are reductions over the wave).
__device__ inline void quantize_lane(const float (&v)[4], uint8_t *__restrict__ rec, int r,
                                     int lane) {
  const float amax = block_amax(v);
  int c[4];
  quant4(v, amax, c);
  // codes: lane owns bytes 4*lane .. 4*lane+3, i.e. unit u = lane/4 of the row
  const uint32_t word = pack4(c);
  const int u = lane >> 2;
  *reinterpret_cast<uint32_t *>(rec + r * QK + 16 * (u ^ r) + 4 * (lane & 3)) = word;

  const int s = group8_sum(c[0] + c[1] + c[2] + c[3]);
  if ((lane & 7) == 0) {
    // (lo, hi) = (s & 63, s - lo): both exact in binary16
    const int lo = s & 63;
    const _Float16 h[2] = {(_Float16)(float)lo, (_Float16)(float)(s - lo)};
    *reinterpret_cast<uint32_t *>(rec + ACT_SUMS_OFF + r * 32 + 4 * (lane >> 3)) =
        __builtin_bit_cast(uint32_t, h);
  }
  if (lane == 0) *reinterpret_cast<float *>(rec + ACT_DX_OFF + 4 * r) = block_dx(amax);
  // the record's zero tail: 448 bytes, 28 per row
  if (lane < 7) *reinterpret_cast<uint32_t *>(rec + ACT_PAD_OFF + 28 * r + 4 * lane) = 0u;
}

template <bool VEC, bool GATHER>
__global__ __launch_bounds__(256) void quantize_kernel(int64_t M, int64_t Mpad, int nb,
                                                       const float *__restrict__ x, int64_t ldx,
                                                       const int32_t *__restrict__ idx,
                                                       int64_t L, uint8_t *__restrict__ qa,
                                                       int32_t *__restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * WAVES_PER_BLOCK + (threadIdx.x >> 6);
  if (item >= Mpad * nb) return;  // whole wave exits together
  const int64_t m = item / nb;
  const int b = (int)(item - m * nb);
  const int64_t mb = m / ACT_ROWS;
  const int r = (int)(m - mb * ACT_ROWS);
  const int64_t nmb = Mpad / ACT_ROWS;
  uint8_t *rec = qa + ((int64_t)b * nmb + mb) * ACT_RECORD;

  int64_t src = m;
  bool valid = m < M;
  if (GATHER && valid) {
    const int32_t s = idx[m];
    const bool in_range = s >= 0 && (int64_t)s < L;
    if (b == 0 && lane == 0) err[m] = in_range ? 0 : 1;
    valid = in_range;
    src = in_range ? s : 0;
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

  quantize_lane(v, rec, r, lane);
}


// Down-projection input: row m of gu holds [gate (F) | up (F)]; one wave per
// (row, 256-block) of silu(gate) * up.
template <bool VEC>
__global__ __launch_bounds__(256) void swiglu_quantize_kernel(int64_t M, int64_t Mpad, int nb,
                                                              const float *__restrict__ gu,
                                                              int64_t ldgu,
                                                              uint8_t *__restrict__ qa) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * WAVES_PER_BLOCK + (threadIdx.x >> 6);
  if (item >= Mpad * nb) return;  // whole wave exits together
  const int64_t m = item / nb;
  const int b = (int)(item - m * nb);
  const int64_t mb = m / ACT_ROWS;
  const int r = (int)(m - mb * ACT_ROWS);
  uint8_t *rec = qa + ((int64_t)b * (Mpad / ACT_ROWS) + mb) * ACT_RECORD;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (m < M) {
    const float *gp = gu + m * ldgu + (int64_t)b * QK + 4 * lane;
    const float *up = gp + (int64_t)nb * QK;
    float g[4], u[4];
    if (VEC) {
      const f32x4 tg = *reinterpret_cast<const f32x4 *>(gp);
      const f32x4 tu = *reinterpret_cast<const f32x4 *>(up);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g[i] = tg[i];
        u[i] = tu[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g[i] = gp[i];
        u[i] = up[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = silu_mul(g[i], u[i]);
  }
  quantize_lane(v, rec, r, lane);
}

// RMSNorm then quantize: one workgroup of 16 waves per (padded) row, wave w
// owning the row's 256-blocks w, w + 16, ...  The sum of squares is formed
// in the order the producer defines: every lane adds its 4 squares in turn,
// the wave adds its 64 lane sums as a pairwise tree (DPP moves pair lanes 2i
// and 2i + 1, then quads, octets, rows of 16, rows 0-1 and 2-3, then the two
// halves), each block's sum goes to LDS, and after one barrier every wave
// adds the block sums in increasing block order.  mean = ss / K, rinv = 1 /
// sqrt(mean + eps), y = (x * rinv) * gamma; each wave then quantizes its
// blocks.
//
// Latency: every wave loads its first block of x and gamma before anything
// waits, so at K <= 4096 the row costs one memory round trip, one barrier
// and no LDS shuffles.
constexpr int NORM_THREADS = 1024;
constexpr int NORM_WAVES = NORM_THREADS / 64;

template <int CTRL, int ROW_MASK = 0xf>
__device__ inline float dpp_or_zero(float v) {
  // lanes of rows outside ROW_MASK read 0
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false));
}

// The pairwise tree over the wave's 64 values; every level adds two values
// the tree pairs (in either order: binary32 addition commutes).  The full
// sum ends in lane 63 and is returned in every lane.
__device__ inline float wave_tree_sum(float v) {
  v = v + dpp_or_zero<DPP_QUAD_1032>(v);
  v = v + dpp_or_zero<DPP_QUAD_2301>(v);
  v = v + dpp_or_zero<DPP_ROW_HALF_MIRROR>(v);
  v = v + dpp_or_zero<DPP_ROW_MIRROR>(v);
  // rows 1 and 3 add the sum of the row before (lane 15 of it), then rows 2
  // and 3 add rows 0 + 1 (lane 31); the other rows add 0
  v = v + dpp_or_zero<DPP_ROW_BCAST15, 0xa>(v);
  v = v + dpp_or_zero<DPP_ROW_BCAST31, 0xc>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

template <bool VEC>
__device__ inline void load4(const float *p, float (&v)[4]) {
  if (VEC) {
    const f32x4 t = *reinterpret_cast<const f32x4 *>(p);
    v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = p[i];
  }
}

template <bool VEC>
__global__ __launch_bounds__(NORM_THREADS) void rmsnorm_quantize_kernel(
    int64_t M, int64_t Mpad, int nb, const float *__restrict__ x, int64_t ldx,
    const float *__restrict__ gamma, float eps, uint8_t *__restrict__ qa) {
  __shared__ float block_ss[NORM_MAX_BLOCKS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m = blockIdx.x;
  const int64_t mb = m / ACT_ROWS;
  const int r = (int)(m - mb * ACT_ROWS);
  const int64_t K = (int64_t)nb * QK;
  const bool valid = m < M;  // uniform across the workgroup
  const float *xr = x + (valid ? m : 0) * ldx;

  // this wave's first block and its weights
  float xv[4] = {0.f, 0.f, 0.f, 0.f}, gv[4] = {0.f, 0.f, 0.f, 0.f};
  if (valid && wave < nb) {
    load4<VEC>(xr + (int64_t)wave * QK + 4 * lane, xv);
    load4<VEC>(gamma + (int64_t)wave * QK + 4 * lane, gv);
  }

  float rinv = 0.0f;
  if (valid) {
    for (int b = wave; b < nb; b += NORM_WAVES) {
      float v[4] = {xv[0], xv[1], xv[2], xv[3]};
      if (b != wave) load4<VEC>(xr + (int64_t)b * QK + 4 * lane, v);
      float t = v[0] * v[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        const float sq = v[i] * v[i];
        t = t + sq;
      }
      t = wave_tree_sum(t);
      if (lane == 0) block_ss[b] = t;
    }
    __syncthreads();
    float ss = block_ss[0];
    for (int b = 1; b < nb; ++b) ss = ss + block_ss[b];
    const float mean = ss / (float)K;
    rinv = 1.0f / __builtin_sqrtf(mean + eps);
  }

  for (int b = wave; b < nb; b += NORM_WAVES) {
    uint8_t *rec = qa + ((int64_t)b * (Mpad / ACT_ROWS) + mb) * ACT_RECORD;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
      if (b != wave) {
        load4<VEC>(xr + (int64_t)b * QK + 4 * lane, xv);
        load4<VEC>(gamma + (int64_t)b * QK + 4 * lane, gv);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float t = xv[i] * rinv;
        v[i] = t * gv[i];
      }
    }
    quantize_lane(v, rec, r, lane);
  }
}

}  // namespace

hipError_t launch_quantize(int64_t M, int64_t K, const float *x, int64_t ldx, const int32_t *idx,
                           int64_t L, uint8_t *qa, int32_t *err, hipStream_t stream) {
  const int nb = (int)(K / QK);
  const int64_t Mpad = (M + ACT_ROWS - 1) / ACT_ROWS * ACT_ROWS;
  const int64_t items = Mpad * nb;
  const int64_t blocks = (items + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  const bool vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (ldx % 4 == 0);
  dim3 grid((unsigned)blocks), block(64 * WAVES_PER_BLOCK);
  if (idx) {
    if (vec)
      hipLaunchKernelGGL((quantize_kernel<true, true>), grid, block, 0, stream, M, Mpad, nb, x,
                         ldx, idx, L, qa, err);
    else
      hipLaunchKernelGGL((quantize_kernel<false, true>), grid, block, 0, stream, M, Mpad, nb, x,
                         ldx, idx, L, qa, err);
  } else {
    if (vec)
      hipLaunchKernelGGL((quantize_kernel<true, false>), grid, block, 0, stream, M, Mpad, nb, x,
                         ldx, idx, L, qa, err);
    else
      hipLaunchKernelGGL((quantize_kernel<false, false>), grid, block, 0, stream, M, Mpad, nb, x,
                         ldx, idx, L, qa, err);
  }
  return hipGetLastError();
}

hipError_t launch_swiglu_quantize(int64_t M, int64_t F, const float *gu, int64_t ldgu,
                                  uint8_t *qa, hipStream_t stream) {
  const int nb = (int)(F / QK);
  const int64_t Mpad = (M + ACT_ROWS - 1) / ACT_ROWS * ACT_ROWS;
  const int64_t blocks = (Mpad * nb + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  const bool vec = (reinterpret_cast<uintptr_t>(gu) % 16 == 0) && (ldgu % 4 == 0);
  dim3 grid((unsigned)blocks), block(64 * WAVES_PER_BLOCK);
  if (vec)
    hipLaunchKernelGGL((swiglu_quantize_kernel<true>), grid, block, 0, stream, M, Mpad, nb, gu,
                       ldgu, qa);
  else
    hipLaunchKernelGGL((swiglu_quantize_kernel<false>), grid, block, 0, stream, M, Mpad, nb, gu,
                       ldgu, qa);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_quantize(int64_t M, int64_t K, const float *x, int64_t ldx,
                                   const float *gamma, float eps, uint8_t *qa,
                                   hipStream_t stream) {
  const int nb = (int)(K / QK);
  const int64_t Mpad = (M + ACT_ROWS - 1) / ACT_ROWS * ACT_ROWS;
  const bool vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (ldx % 4 == 0) &&
                   (reinterpret_cast<uintptr_t>(gamma) % 16 == 0);
  dim3 grid((unsigned)Mpad), block(NORM_THREADS);
  if (vec)
    hipLaunchKernelGGL((rmsnorm_quantize_kernel<true>), grid, block, 0, stream, M, Mpad, nb, x,
                       ldx, gamma, eps, qa);
  else
    hipLaunchKernelGGL((rmsnorm_quantize_kernel<false>), grid, block, 0, stream, M, Mpad, nb, x,
                       ldx, gamma, eps, qa);
  return hipGetLastError();
}

}  // namespace dq
