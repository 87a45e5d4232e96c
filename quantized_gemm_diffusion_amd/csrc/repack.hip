// repack.hip -- load-time permutation of GGUF Q4_K / Q6_K super-blocks into
// the tile layout described in dq_internal.h.  The bits are kept as they are
// (Q4_K stays 4.5 bits per weight, Q6_K stays 6.5625): only their positions
// change, so that each lane of the GEMM reads its codes as aligned 16-byte
// records (mojo-dllm "Architecture" page, "Memory": every projection matrix
// is repacked once at load and stays resident).
//
// GGUF code positions (public ggml K-quant block definitions; the pages name
// the types only):
//   Q4_K weight i: byte 16 + 32*(i/64) + i%32 of the block, low nibble when
//                  i%64 < 32, else high nibble.
//   Q6_K weight i (h = i/128, quarter = (i%128)/32, l = i%32): low 4 bits in
//                  ql byte 64h + l + 32*(quarter odd), low nibble for quarters
//                  0-1, high nibble for 2-3; high 2 bits in qh byte 128 +
//                  32h + l at bit 2*quarter.
//
// One wave per (n-tile, super-block); lane l builds the records it will read
// in the GEMM.  Rows n >= N are written as zeros (d = 0: they add nothing).
#include "dq_internal.h"

namespace dq {
namespace {

__device__ inline uint32_t q4k_code(const uint8_t *blk, int i) {
  const uint8_t byte = blk[16 + 32 * (i >> 6) + (i & 31)];
  return (i & 32) ? (byte >> 4) : (byte & 15);
}

__device__ inline uint32_t q6k_code(const uint8_t *blk, int i) {
  const int h = i >> 7, quarter = (i >> 5) & 3, l = i & 31;
  const uint8_t lo = blk[64 * h + l + ((quarter & 1) ? 32 : 0)];
  const uint32_t low4 = (quarter >= 2) ? (lo >> 4) : (lo & 15);
  const uint32_t high2 = (blk[128 + 32 * h + l] >> (2 * quarter)) & 3;
  return low4 | (high2 << 4);
}

// 16-byte record i of lane quarter kq for one row: two chunks, 4-bit parts.
template <bool Q6>
__device__ inline void nibble_record(const uint8_t *blk, int kq, int i, uint32_t out[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int c = 2 * i + (t >> 1), h = t & 1;
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k_lo = 64 * kq + 16 * c + 8 * h + e;
      const uint32_t lo = Q6 ? (q6k_code(blk, k_lo) & 15) : q4k_code(blk, k_lo);
      const uint32_t hi = Q6 ? (q6k_code(blk, k_lo + 4) & 15) : q4k_code(blk, k_lo + 4);
      w |= (lo | (hi << 4)) << (8 * e);
    }
    out[t] = w;
  }
}

template <int TYPE>
__global__ __launch_bounds__(64) void repack_kernel(int64_t N, int nb, const uint8_t *__restrict__ src,
                                                    uint8_t *__restrict__ dst) {
  constexpr bool Q6 = TYPE == 14;
  constexpr int BB = Q6 ? Q6K_BLOCK : Q4K_BLOCK;
  constexpr int TB = Q6 ? Q6K_TILE : Q4K_TILE;
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  const int64_t nt = blockIdx.y;
  const int r = lane & 15, kq = lane >> 4;
  const int64_t n = nt * TILE_N + r;
  const bool valid = n < N;
  const uint8_t *blk = src + (valid ? (n * nb + b) * BB : 0);
  uint8_t *tile = dst + (nt * nb + b) * TB;

  if (!Q6) {
    if (kq == 0) {
      uint32_t head[4] = {0, 0, 0, 0};
      if (valid)
        for (int t = 0; t < 16; ++t) head[t >> 2] |= (uint32_t)blk[t] << (8 * (t & 3));
      *reinterpret_cast<i32x4 *>(tile + 16 * r) =
          i32x4{(int)head[0], (int)head[1], (int)head[2], (int)head[3]};
    }
    for (int i = 0; i < 2; ++i) {
      uint32_t rec[4] = {0, 0, 0, 0};
      if (valid) nibble_record<false>(blk, kq, i, rec);
      *reinterpret_cast<i32x4 *>(tile + Q4K_CODES_OFF + (i * 64 + lane) * 16) =
          i32x4{(int)rec[0], (int)rec[1], (int)rec[2], (int)rec[3]};
    }
  } else {
    for (int i = 0; i < 2; ++i) {
      uint32_t rec[4] = {0, 0, 0, 0};
      if (valid) nibble_record<true>(blk, kq, i, rec);
      *reinterpret_cast<i32x4 *>(tile + (i * 64 + lane) * 16) =
          i32x4{(int)rec[0], (int)rec[1], (int)rec[2], (int)rec[3]};
    }
    {
      uint32_t rec[4] = {0, 0, 0, 0};
      if (valid) {
        for (int c = 0; c < 4; ++c) {
          uint32_t w = 0;
          for (int e = 0; e < 4; ++e)
            for (int s = 0; s < 4; ++s) {
              const int p = 4 * s + e;
              w |= ((q6k_code(blk, 64 * kq + 16 * c + p) >> 4) & 3) << (8 * e + 2 * s);
            }
          rec[c] = w;
        }
      }
      *reinterpret_cast<i32x4 *>(tile + Q6K_QH_OFF + lane * 16) =
          i32x4{(int)rec[0], (int)rec[1], (int)rec[2], (int)rec[3]};
    }
    // scales: [kq][r] dword, byte c = scale of sub-block 4kq + c
    uint32_t sw = 0;
    if (valid)
      for (int c = 0; c < 4; ++c) sw |= (uint32_t)blk[192 + 4 * kq + c] << (8 * c);
    *reinterpret_cast<uint32_t *>(tile + Q6K_SC_OFF + (kq * 16 + r) * 4) = sw;
    if (kq == 0) {
      const uint16_t dv = valid ? (uint16_t)(blk[208] | (blk[209] << 8)) : 0;
      *reinterpret_cast<uint16_t *>(tile + Q6K_D_OFF + 2 * r) = dv;
    }
  }
}

}  // namespace

hipError_t launch_repack(int type, int64_t N, int64_t K, const uint8_t *src, uint8_t *dst,
                         hipStream_t stream) {
  const int nb = (int)(K / QK);
  const int64_t ntiles = (N + TILE_N - 1) / TILE_N;
  dim3 grid((unsigned)nb, (unsigned)ntiles), block(64);
  if (type == 12)
    hipLaunchKernelGGL(repack_kernel<12>, grid, block, 0, stream, N, nb, src, dst);
  else
    hipLaunchKernelGGL(repack_kernel<14>, grid, block, 0, stream, N, nb, src, dst);
  return hipGetLastError();
}

}  // namespace dq
