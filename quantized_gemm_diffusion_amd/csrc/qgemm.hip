// qgemm.hip -- K-quant weight x int8 activation GEMM on gfx950 matrix cores.
//
// y[m][n] = sum_b d_x[m][b] * (d[n][b] * S[m][n][b] - dmin[n][b] * Mn[m][n][b])
//   S  = sum_j sc_j * dot_j,  dot_j = sum over sub-block j of q_w * q_x
//   Mn = sum_j m_j * bsum_j   (Q4_K only)
// (mojo-dllm "Architecture" page, "Source map": the packed GEMM used for every
// projection and the int8 matrix-core GEMM over Q4_K / Q6_K blocks; "A forward
// pass", step 2: int8 activations quantized once per input.)
//
// How S is formed exactly on int8 MFMA without a per-sub-block VALU fold: the
// sub-block scale is folded into the weight operand as two int8 digits, so
// one int32 MFMA accumulation over the whole 256-wide super-block yields S.
//   Q4_K: sc = 8*sh + sl with sl, sh in [0, 7]; the digits q*sl and q*sh are
//         at most 105, and S = R(q*sl) + 8 * R(q*sh).
//   Q6_K: v = sc * (q - 32) in [-4064, 4096]; lo = v & 127, hi = v >> 7 (in
//         [-32, 32]), and S = R(lo) + 128 * R(hi).
// Every partial sum is an exact int32 (|S| <= 30.7e6 for Q4_K, 1.34e8 for
// Q6_K).  The Q4_K min term is a 16-deep contraction per super-block done on
// the f16 MFMA with operands that are exact in f16: bsum = lo6 + rest
// (lo6 = bsum & 63, rest a multiple of 64 with |rest| <= 4096) against m_j;
// all products and partial sums are integers below 2^24, so Mn is exact.
//
// MFMA operand roles: A = activations (row m = lane % 32 of the m-tile), B =
// weights (column n = lane % 32 of the n-tile); lane half g = lane / 32 owns
// k = 32c + 16g + p of chunk c.  A and B use the same (lane, byte) -> k map,
// which is all the contraction needs.  Accumulator element r of lane l is
// row 8*(r/4) + 4*g + r%4, column l % 32.
#include "dq_internal.h"

namespace dq {
namespace {

__device__ inline float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xffff));
}

// Multiply four packed bytes by the same small factor; every byte product
// stays below 256, so the bytes never carry into each other.
__device__ inline uint32_t mul_bytes(uint32_t u, uint32_t f) {
  const u16x2 a = __builtin_bit_cast(u16x2, u);
  const u16x2 r = a * (u16x2){(unsigned short)f, (unsigned short)f};
  return __builtin_bit_cast(uint32_t, r);
}

// Q4_K 6-bit scale / min of sub-block j from the 12 GGUF scale bytes held as
// three dwords s[0..2] (bytes 0-3, 4-7, 8-11).
__device__ inline uint32_t scale_byte(const uint32_t s[3], int i) {
  return (s[i >> 2] >> (8 * (i & 3))) & 255;
}
__device__ inline uint32_t q4k_sc(const uint32_t s[3], int j) {
  return j < 4 ? (scale_byte(s, j) & 63)
               : ((scale_byte(s, j + 4) & 15) | ((scale_byte(s, j - 4) >> 6) << 4));
}
__device__ inline uint32_t q4k_mn(const uint32_t s[3], int j) {
  return j < 4 ? (scale_byte(s, j + 4) & 63)
               : ((scale_byte(s, j + 4) >> 4) | ((scale_byte(s, j) >> 6) << 4));
}

// Q6_K: 16 codes (one 16-bit lane pair per two codes) -> lo / hi digit bytes.
__device__ inline void q6k_digits(uint32_t codes, int sc, uint32_t &lo, uint32_t &hi) {
  // even codes (bytes 0, 2) and odd codes (bytes 1, 3) in 16-bit lanes
  const uint32_t ev = __builtin_amdgcn_perm(0u, codes, 0x0c020c00u);
  const uint32_t od = __builtin_amdgcn_perm(0u, codes, 0x0c030c01u);
  const s16x2 s2 = {(short)sc, (short)sc};
  const s16x2 o2 = {(short)(-32 * sc), (short)(-32 * sc)};
  const s16x2 ve = __builtin_bit_cast(s16x2, ev) * s2 + o2;  // sc * (q - 32), exact in i16
  const s16x2 vo = __builtin_bit_cast(s16x2, od) * s2 + o2;
  const uint32_t ue = __builtin_bit_cast(uint32_t, ve), uo = __builtin_bit_cast(uint32_t, vo);
  lo = __builtin_amdgcn_perm(uo, ue, 0x06020400u) & 0x7f7f7f7fu;
  // byte 1 of (v << 1) is v >> 7 as a two's-complement byte (|v| < 2^14)
  hi = __builtin_amdgcn_perm(uo << 1, ue << 1, 0x07030501u);
}

template <int TYPE, bool DEBUG>
__global__ __launch_bounds__(64) void qgemm_kernel(int64_t M, int64_t N, int nb,
                                                   const int8_t *__restrict__ q,
                                                   const float *__restrict__ dx,
                                                   const int32_t *__restrict__ bsum,
                                                   const uint8_t *__restrict__ packed,
                                                   float *__restrict__ y, int64_t ldy,
                                                   int32_t *__restrict__ dbg_S,
                                                   int32_t *__restrict__ dbg_Mn) {
  constexpr bool Q6 = TYPE == 14;
  constexpr int TB = Q6 ? Q6K_TILE : Q4K_TILE;
  const int lane = threadIdx.x;
  const int col = lane & 31, g = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * 32;
  const int64_t nt = blockIdx.y;
  const int64_t n = nt * TILE_N + col;
  const int64_t K = (int64_t)nb * QK;

  const int64_t am = m0 + col;  // A-operand row of this lane
  const bool a_ok = am < M;
  const int8_t *qa = q + (a_ok ? am : 0) * K + 16 * g;

  int64_t rows[16];
  bool row_ok[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    rows[r] = m0 + 8 * (r >> 2) + 4 * g + (r & 3);
    row_ok[r] = rows[r] < M;
  }

  f32x16 acc = {};
  const uint8_t *tile = packed + nt * nb * TB;
  for (int b = 0; b < nb; ++b, tile += TB) {
    i32x4 blo[8], bhi[8];
    float dw, dmw = 0.f;
    f16x8 bmin = {};
    if (!Q6) {
      const i32x4 head = *reinterpret_cast<const i32x4 *>(tile + 16 * col);
      dw = half_bits_to_float((uint32_t)head[0]);
      dmw = half_bits_to_float((uint32_t)head[0] >> 16);
      const uint32_t s[3] = {(uint32_t)head[1], (uint32_t)head[2], (uint32_t)head[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x4 rec =
            *reinterpret_cast<const i32x4 *>(tile + Q4K_CODES_OFF + (i * 64 + lane) * 16);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = 2 * i + h;
          const uint32_t sc = q4k_sc(s, c), sl = sc & 7, sh = sc >> 3;
          const uint32_t w0 = (uint32_t)rec[2 * h], w1 = (uint32_t)rec[2 * h + 1];
          const uint32_t u[4] = {w0 & 0x0f0f0f0fu, (w0 >> 4) & 0x0f0f0f0fu, w1 & 0x0f0f0f0fu,
                                 (w1 >> 4) & 0x0f0f0f0fu};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            blo[c][t] = (int)mul_bytes(u[t], sl);
            bhi[c][t] = (int)mul_bytes(u[t], sh);
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const _Float16 mv = (_Float16)(float)q4k_mn(s, 4 * g + jj);
        bmin[2 * jj] = mv;
        bmin[2 * jj + 1] = mv;
      }
    } else {
      dw = half_bits_to_float(*reinterpret_cast<const uint16_t *>(tile + Q6K_D_OFF + 2 * col));
      const uint32_t *sp =
          reinterpret_cast<const uint32_t *>(tile + Q6K_SC_OFF + (g * 32 + col) * 8);
      const uint32_t sw[2] = {sp[0], sp[1]};
      i32x4 qh[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        qh[i] = *reinterpret_cast<const i32x4 *>(tile + Q6K_QH_OFF + (i * 64 + lane) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x4 rec = *reinterpret_cast<const i32x4 *>(tile + (i * 64 + lane) * 16);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = 2 * i + h;
          const int sc = (int)(int8_t)((sw[c >> 2] >> (8 * (c & 3))) & 255);
          const uint32_t u = (uint32_t)qh[c >> 2][c & 3];
          const uint32_t w0 = (uint32_t)rec[2 * h], w1 = (uint32_t)rec[2 * h + 1];
          const uint32_t codes[4] = {
              (w0 & 0x0f0f0f0fu) | ((u << 4) & 0x30303030u),
              ((w0 >> 4) & 0x0f0f0f0fu) | ((u << 2) & 0x30303030u),
              (w1 & 0x0f0f0f0fu) | (u & 0x30303030u),
              ((w1 >> 4) & 0x0f0f0f0fu) | ((u >> 2) & 0x30303030u)};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            uint32_t lo, hi;
            q6k_digits(codes[t], sc, lo, hi);
            blo[c][t] = (int)lo;
            bhi[c][t] = (int)hi;
          }
        }
      }
    }

    i32x16 rl = {}, rh = {};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      i32x4 a = {0, 0, 0, 0};
      if (a_ok) a = *reinterpret_cast<const i32x4 *>(qa + (int64_t)b * QK + 32 * c);
      rl = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, blo[c], rl, 0, 0, 0);
      rh = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bhi[c], rh, 0, 0, 0);
    }
    f32x16 mnf = {};
    if (!Q6) {
      f16x8 amin = {};
      if (a_ok) {
        const i32x4 bs = *reinterpret_cast<const i32x4 *>(bsum + am * (K / 32) + 8 * b + 4 * g);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int v = bs[jj];
          const int lo6 = v & 63;
          amin[2 * jj] = (_Float16)(float)lo6;
          amin[2 * jj + 1] = (_Float16)(float)(v - lo6);
        }
      }
      mnf = __builtin_amdgcn_mfma_f32_32x32x16_f16(amin, bmin, mnf, 0, 0, 0);
    }

#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int s_int = Q6 ? rl[r] + rh[r] * 128 : rl[r] + rh[r] * 8;
      if (DEBUG) {
        if (row_ok[r] && n < N) {
          const int64_t o = (rows[r] * N + n) * nb + b;
          dbg_S[o] = s_int;
          dbg_Mn[o] = Q6 ? 0 : (int32_t)mnf[r];
        }
      } else {
        const float xs = row_ok[r] ? dx[rows[r] * nb + b] : 0.f;
        const float t = Q6 ? dw * (float)s_int : dw * (float)s_int - dmw * mnf[r];
        acc[r] += xs * t;
      }
    }
  }

  if (!DEBUG && n < N) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (row_ok[r]) y[rows[r] * ldy + n] = acc[r];
  }
}

template <int TYPE, bool DEBUG>
hipError_t launch(int64_t M, int64_t N, int nb, const int8_t *q, const float *d,
                  const int32_t *bsum, const uint8_t *packed, float *y, int64_t ldy,
                  int32_t *dbg_S, int32_t *dbg_Mn, hipStream_t stream) {
  dim3 grid((unsigned)((M + 31) / 32), (unsigned)((N + TILE_N - 1) / TILE_N)), block(64);
  hipLaunchKernelGGL((qgemm_kernel<TYPE, DEBUG>), grid, block, 0, stream, M, N, nb, q, d, bsum,
                     packed, y, ldy, dbg_S, dbg_Mn);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qgemm(int type, int64_t M, int64_t N, int64_t K, const int8_t *q,
                        const float *d, const int32_t *bsum, const uint8_t *packed, float *y,
                        int64_t ldy, int32_t *dbg_S, int32_t *dbg_Mn, hipStream_t stream) {
  const int nb = (int)(K / QK);
  const bool dbg = dbg_S != nullptr;
  if (type == 12)
    return dbg ? launch<12, true>(M, N, nb, q, d, bsum, packed, y, ldy, dbg_S, dbg_Mn, stream)
               : launch<12, false>(M, N, nb, q, d, bsum, packed, y, ldy, dbg_S, dbg_Mn, stream);
  return dbg ? launch<14, true>(M, N, nb, q, d, bsum, packed, y, ldy, dbg_S, dbg_Mn, stream)
             : launch<14, false>(M, N, nb, q, d, bsum, packed, y, ldy, dbg_S, dbg_Mn, stream);
}

}  // namespace dq
