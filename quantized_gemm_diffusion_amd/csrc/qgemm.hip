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
// MFMA operand roles (16x16x64): A = activations (row m = lane % 16 of the
// 16-row m-block), B = weights (column n = lane % 16 of the n-tile); lane
// quarter kq = lane / 16 owns k = 64kq + 16c + p of chunk c.  A and B use the
// same (lane, byte) -> k map, which is all the contraction needs.
// Accumulator element i of lane l is row 4*kq + i, column l % 16.
#include <type_traits>

#include "dq_internal.h"

namespace dq {
namespace {

__device__ inline float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xffff));
}

// Multiply four packed bytes by the same small factor held in both 16-bit
// halves of f; every byte product stays below 256, so bytes never carry.
__device__ inline uint32_t mul_bytes(uint32_t u, uint32_t f) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, u) * __builtin_bit_cast(u16x2, f));
}

// Byte i of x copied into the low byte of both 16-bit halves (others zero).
__device__ inline uint32_t byte_pair(uint32_t x, int i) {
  return __builtin_amdgcn_perm(0u, x, 0x0c000c00u | (uint32_t)i | ((uint32_t)i << 16));
}

// Q6_K: 4 codes (bytes) -> lo / hi digit bytes of v = sc * (q - 32).
__device__ inline void q6k_digits(uint32_t codes, uint32_t sc2, uint32_t off2, uint32_t &lo,
                                  uint32_t &hi) {
  // even codes (bytes 0, 2) and odd codes (bytes 1, 3) in 16-bit lanes
  const uint32_t ev = __builtin_amdgcn_perm(0u, codes, 0x0c020c00u);
  const uint32_t od = __builtin_amdgcn_perm(0u, codes, 0x0c030c01u);
  const s16x2 s2 = __builtin_bit_cast(s16x2, sc2), o2 = __builtin_bit_cast(s16x2, off2);
  const uint32_t ue = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, ev) * s2 + o2);
  const uint32_t uo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, od) * s2 + o2);
  lo = __builtin_amdgcn_perm(uo, ue, 0x06020400u) & 0x7f7f7f7fu;
  // byte 1 of (v << 1) is v >> 7 as a two's-complement byte (|v| < 2^14)
  hi = __builtin_amdgcn_perm(uo << 1, ue << 1, 0x07030501u);
}

// All global reads go through buffer resources whose base is advanced with
// scalar arithmetic, so per-lane offsets stay small 32-bit constants and the
// hardware range check (num_records) returns zeros past the end of a buffer:
// activation rows past M read as 0 without any per-lane clamping.
constexpr int RSRC_FLAGS = 0x00020000;

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7fffffff ? 0x7fffffffu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, RSRC_FLAGS);
}
__device__ inline i32x4 ld4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ inline uint2 ld2(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ inline uint32_t ld1(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Raw per-lane weight data of one (n-tile, super-block) tile.
struct RawQ4 {
  i32x4 head;    // d, dmin, scales[12] of this lane's row
  i32x4 rec[2];  // 4-bit codes, records 0..1
};
struct RawQ6 {
  i32x4 rec[2];  // low 4 bits
  i32x4 qh;      // high 2 bits
  uint32_t sw;   // this lane's 4 sub-block scales
  uint32_t d;    // fp16 d of this lane's row in the low half
};

__device__ inline void load_w(const uint8_t *tile, int lane, int col, int kq, RawQ4 &r) {
  const auto R = rsrc(tile, Q4K_TILE);
  r.head = ld4(R, 16 * col);
#pragma unroll
  for (int i = 0; i < 2; ++i) r.rec[i] = ld4(R, Q4K_CODES_OFF + (i * 64 + lane) * 16);
}

__device__ inline void load_w(const uint8_t *tile, int lane, int col, int kq, RawQ6 &r) {
  const auto R = rsrc(tile, Q6K_TILE);
#pragma unroll
  for (int i = 0; i < 2; ++i) r.rec[i] = ld4(R, (i * 64 + lane) * 16);
  r.qh = ld4(R, Q6K_QH_OFF + lane * 16);
  r.sw = ld1(R, Q6K_SC_OFF + (kq * 16 + col) * 4);
  r.d = ld1(R, Q6K_D_OFF + 4 * (col >> 1)) >> (16 * (col & 1));
}

// Per-lane B operands of one super-block: two digit planes, the f16 min
// operand (Q4_K) and the super-block scales.
struct Digits {
  i32x4 lo[4], hi[4];
  f16x4 bmin;
  float dw, dmw;
};

// Q4_K: chunk c of lane quarter kq lies in sub-block 2kq + c/2.  The 6-bit
// scales and mins of sub-blocks 0..3 and 4..7 are formed four at a time from
// the 12 GGUF scale bytes D0 (bytes 0-3), D1 (4-7), D2 (8-11):
//   j < 4 : sc = low 6 bits of byte j, mn = low 6 bits of byte j+4
//   j >= 4: sc = low nibble of byte j+4 | top 2 bits of byte j-4 << 4,
//           mn = high nibble of byte j+4 | top 2 bits of byte j << 4
__device__ inline void make_digits(const RawQ4 &w, int kq, Digits &D) {
  D.dw = half_bits_to_float((uint32_t)w.head[0]);
  D.dmw = half_bits_to_float((uint32_t)w.head[0] >> 16);
  const uint32_t D0 = (uint32_t)w.head[1], D1 = (uint32_t)w.head[2], D2 = (uint32_t)w.head[3];
  const uint32_t sc_lo = D0 & 0x3f3f3f3fu, mn_lo = D1 & 0x3f3f3f3fu;
  const uint32_t sc_hi = (D2 & 0x0f0f0f0fu) | ((D0 >> 2) & 0x30303030u);
  const uint32_t mn_hi = ((D2 >> 4) & 0x0f0f0f0fu) | ((D1 >> 2) & 0x30303030u);
  // bytes 0, 1 of SC / MN: sub-blocks 2kq and 2kq + 1
  const int sh16 = 16 * (kq & 1);
  const uint32_t SC = (kq < 2 ? sc_lo : sc_hi) >> sh16;
  const uint32_t MN = (kq < 2 ? mn_lo : mn_hi) >> sh16;
  const uint32_t SL = SC & 0x07070707u, SH = (SC >> 3) & 0x07070707u;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t fl = byte_pair(SL, i), fh = byte_pair(SH, i);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 2 * i + h;
      const uint32_t w0 = (uint32_t)w.rec[i][2 * h], w1 = (uint32_t)w.rec[i][2 * h + 1];
      const uint32_t u[4] = {w0 & 0x0f0f0f0fu, (w0 >> 4) & 0x0f0f0f0fu, w1 & 0x0f0f0f0fu,
                             (w1 >> 4) & 0x0f0f0f0fu};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        D.lo[c][t] = (int)mul_bytes(u[t], fl);
        D.hi[c][t] = (int)mul_bytes(u[t], fh);
      }
    }
  }
  // (m_j, m_j) as f16 pairs: 0x6400 | m is 1024 + m in f16; subtracting 1024 is exact
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t pr = byte_pair(MN, i) | 0x64006400u;
    const f16x2 v = __builtin_bit_cast(f16x2, pr) - (f16x2){(_Float16)1024.0f, (_Float16)1024.0f};
    D.bmin[2 * i] = v[0];
    D.bmin[2 * i + 1] = v[1];
  }
}

// Q6_K: chunk c of lane quarter kq is sub-block 4kq + c (scale byte c).
__device__ inline void make_digits(const RawQ6 &w, int kq, Digits &D) {
  D.dw = half_bits_to_float(w.d);
  D.dmw = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 2 * i + h;
      const int sc = (int)(int8_t)((w.sw >> (8 * c)) & 255);
      const uint32_t sc2 = ((uint32_t)sc & 0xffffu) * 0x10001u;
      const uint32_t off2 = ((uint32_t)(-32 * sc) & 0xffffu) * 0x10001u;
      const uint32_t u = (uint32_t)w.qh[c];
      const uint32_t w0 = (uint32_t)w.rec[i][2 * h], w1 = (uint32_t)w.rec[i][2 * h + 1];
      const uint32_t codes[4] = {(w0 & 0x0f0f0f0fu) | ((u << 4) & 0x30303030u),
                                 ((w0 >> 4) & 0x0f0f0f0fu) | ((u << 2) & 0x30303030u),
                                 (w1 & 0x0f0f0f0fu) | (u & 0x30303030u),
                                 ((w1 >> 4) & 0x0f0f0f0fu) | ((u >> 2) & 0x30303030u)};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t lo, hi;
        q6k_digits(codes[t], sc2, off2, lo, hi);
        D.lo[c][t] = (int)lo;
        D.hi[c][t] = (int)hi;
      }
    }
  }
}

// Activation staging.  The 16 x 256 code bytes of one (m-block, super-block)
// are read with coalesced loads (each 64-lane load covers 4 whole rows) into
// this wave's LDS slab, rows padded to 272 bytes so that the MFMA fragment
// reads (lane: row l % 16, bytes 64kq .. 64kq+63) are free of bank conflicts.
// The loads for the next step are issued before the current step's MFMAs; the
// slab is rewritten only after the current fragments are in VGPRs.
constexpr int MBLK = 16;  // rows per m-block
constexpr int SLAB_PITCH = 272;
constexpr int SLAB_BYTES = MBLK * SLAB_PITCH + MBLK * 4;  // codes + d_x of the 16 rows

struct ActLoad {
  i32x4 v[4];  // row 4i + lane/16, bytes 16 * (lane % 16) .. +15, for i = 0..3
  float dxv;   // d_x of row (lane % 16)
  uint2 bs;    // code sums of sub-blocks 2kq, 2kq + 1 of row (lane % 16)
};

// Loads of step (m-block starting at row m_base, super-block b).  The
// resource bases start at row m_base, so rows at or past M fall outside
// num_records and read as zeros.
template <bool Q6, bool DEBUG>
__device__ inline void act_issue(const int8_t *q, const float *dx, const int32_t *bsum,
                                 int64_t m_base, int64_t M, int64_t K, int nb, int b, int lane,
                                 ActLoad &L) {
  const int64_t rows_left = M - m_base;
  const auto Rq = rsrc(q + m_base * K + (int64_t)b * QK, rows_left * K - (int64_t)b * QK);
  const int voff = (lane >> 4) * (int)K + 16 * (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) L.v[i] = ld4(Rq, voff + 4 * i * (int)K);
  const int r = lane & 15;
  L.dxv = 0.f;
  if (!DEBUG) {
    const auto Rd = rsrc(dx + m_base * nb + b, (rows_left * nb - b) * 4);
    L.dxv = __builtin_bit_cast(float, ld1(Rd, r * nb * 4));
  }
  L.bs = make_uint2(0u, 0u);
  if (!Q6) {
    const auto Rb = rsrc(bsum + m_base * (K / 32) + 8 * b, (rows_left * (K / 32) - 8 * b) * 4);
    L.bs = ld2(Rb, r * (int)(K / 32) * 4 + 8 * (lane >> 4));
  }
}

__device__ inline void act_store(uint8_t *slab, int lane, const ActLoad &L) {
  const int rsub = lane >> 4, c16 = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<i32x4 *>(slab + (4 * i + rsub) * SLAB_PITCH + 16 * c16) = L.v[i];
  // the four lane quarters hold the same 16 values: every lane writes, so no
  // divergent branch sits between this write and the next step's reads
  reinterpret_cast<float *>(slab + MBLK * SLAB_PITCH)[lane & 15] = L.dxv;
}

// The MFMA part of one step and what its fold needs.
struct StepOut {
  i32x4 rl, rh;
  f32x4 mnf;
  f32x4 x4;
};

template <bool Q6>
__device__ inline void step_mfma(const uint8_t *slab, int col, int kq, const Digits &D,
                                 const uint2 &bs, StepOut &o) {
  i32x4 a[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    a[c] = *reinterpret_cast<const i32x4 *>(slab + col * SLAB_PITCH + 64 * kq + 16 * c);
  o.x4 = *reinterpret_cast<const f32x4 *>(slab + MBLK * SLAB_PITCH + 16 * kq);
  o.rl = i32x4{};
  o.rh = i32x4{};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    o.rl = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[c], D.lo[c], o.rl, 0, 0, 0);
    o.rh = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[c], D.hi[c], o.rh, 0, 0, 0);
  }
  o.mnf = f32x4{};
  if (!Q6) {
    // bsum = lo6 + rest: both exact in f16 (rest is a multiple of 64, |rest| <= 4096)
    f16x4 amin;
    const int v0 = (int)bs.x, v1 = (int)bs.y;
    const int l0 = v0 & 63, l1 = v1 & 63;
    amin[0] = (_Float16)(short)l0;
    amin[1] = (_Float16)(short)(v0 - l0);
    amin[2] = (_Float16)(short)l1;
    amin[3] = (_Float16)(short)(v1 - l1);
    o.mnf = __builtin_amdgcn_mfma_f32_16x16x16f16(amin, D.bmin, o.mnf, 0, 0, 0);
  }
}

template <bool Q6>
__device__ inline void step_fold(const StepOut &o, float dw, float dmw, f32x4 &acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s_int = Q6 ? o.rl[i] + o.rh[i] * 128 : o.rl[i] + o.rh[i] * 8;
    const float tv = Q6 ? dw * (float)s_int : dw * (float)s_int - dmw * o.mnf[i];
    acc[i] += o.x4[i] * tv;
  }
}

template <bool Q6>
__device__ inline void step_debug(const StepOut &o, int64_t row0, int kq, int64_t n, int64_t M,
                                  int64_t N, int nb, int b, int32_t *dbg_S, int32_t *dbg_Mn) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row0 + 4 * kq + i;
    if (row < M && n < N) {
      const int64_t o_ = (row * N + n) * nb + b;
      dbg_S[o_] = Q6 ? o.rl[i] + o.rh[i] * 128 : o.rl[i] + o.rh[i] * 8;
      dbg_Mn[o_] = Q6 ? 0 : (int32_t)o.mnf[i];
    }
  }
}

constexpr int WAVES = 4;
constexpr int MB_MAX = 10;
constexpr int RED_FLOATS = (WAVES / 2) * MB_MAX * 4 * 64;  // reduction buffer

// One workgroup of 4 waves: one 16-column n-tile x MB 16-row m-blocks x the
// whole reduction.  Wave w takes super-blocks b = w, w + 4, ... and builds a
// super-block's weight digits once for all MB m-blocks.  Loads run ahead: the
// next super-block's weights during the current one, the next step's
// activation slab during the current step.  Registers are capped so that at
// least two workgroups share a CU (two waves per SIMD): one wave's MFMAs run
// while another folds or waits.  The 4 f32 partial sums are added in LDS
// (pairwise tree) at the end.
// MODE: 0 = canvas GEMM, 1 = gathered-row GEMM (same code, its own symbol so
// profiles tell the two workloads apart), 2 = debug stores of S and Mn.
template <int TYPE, int MB, int MODE>
__global__ __launch_bounds__(64 * WAVES, 2) void qgemm_kernel(int64_t M, int64_t N, int nb,
                                                              const int8_t *__restrict__ q,
                                                              const float *__restrict__ dx,
                                                              const int32_t *__restrict__ bsum,
                                                              const uint8_t *__restrict__ packed,
                                                              float *__restrict__ y, int64_t ldy,
                                                              int32_t *__restrict__ dbg_S,
                                                              int32_t *__restrict__ dbg_Mn) {
  constexpr bool Q6 = TYPE == 14;
  constexpr bool DEBUG = MODE == 2;
  constexpr int TB = Q6 ? Q6K_TILE : Q4K_TILE;
  constexpr int MR = MB * MBLK;
  constexpr int LDS_BYTES = WAVES * SLAB_BYTES > RED_FLOATS * 4 ? WAVES * SLAB_BYTES : RED_FLOATS * 4;
  static_assert(MB <= MB_MAX, "reduction buffer");
  using Raw = typename std::conditional<Q6, RawQ6, RawQ4>::type;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];

  // the wave index is uniform across the wave; say so, so that every buffer
  // resource built from it stays in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int64_t nt = blockIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * MR;
  const int64_t n = nt * TILE_N + col;
  const int64_t K = (int64_t)nb * QK;
  uint8_t *slab = lds + wave * SLAB_BYTES;

  f32x4 acc[MB];
#pragma unroll
  for (int t = 0; t < MB; ++t) acc[t] = f32x4{};

  const uint8_t *tiles = packed + nt * nb * TB;
  if (wave < nb) {
    int b = wave;
    Raw wcur, wnxt;
    ActLoad al;
    load_w(tiles + (int64_t)b * TB, lane, col, kq, wcur);
    act_issue<Q6, DEBUG>(q, dx, bsum, m0, M, K, nb, b, lane, al);
    load_w(tiles + (int64_t)(b + WAVES < nb ? b + WAVES : b) * TB, lane, col, kq, wnxt);
    act_store(slab, lane, al);
    uint2 bs = al.bs;
    Digits D;
    make_digits(wcur, kq, D);
    for (;;) {
      const bool last_b = b + WAVES >= nb;
      const int bn = last_b ? b : b + WAVES;
#pragma unroll
      for (int t = 0; t < MB; ++t) {
        // next step's activations: (t+1, b), or (0, next super-block)
        if (t + 1 < MB)
          act_issue<Q6, DEBUG>(q, dx, bsum, m0 + MBLK * (t + 1), M, K, nb, b, lane, al);
        else
          act_issue<Q6, DEBUG>(q, dx, bsum, m0, M, K, nb, bn, lane, al);
        StepOut cur;
        step_mfma<Q6>(slab, col, kq, D, bs, cur);
        act_store(slab, lane, al);  // after this step's fragments are in VGPRs
        bs = al.bs;
        if (DEBUG)
          step_debug<Q6>(cur, m0 + MBLK * t, kq, n, M, N, nb, b, dbg_S, dbg_Mn);
        else
          step_fold<Q6>(cur, D.dw, D.dmw, acc[t]);
      }
      if (last_b) break;
      b = bn;
      wcur = wnxt;
      load_w(tiles + (int64_t)(b + WAVES < nb ? b + WAVES : b) * TB, lane, col, kq, wnxt);
      make_digits(wcur, kq, D);
    }
  }
  if (DEBUG) return;

  // cross-wave reduction: pairwise tree through LDS
  float *red = reinterpret_cast<float *>(lds);
  __syncthreads();  // activation slabs no longer needed
#pragma unroll
  for (int half = WAVES / 2; half >= 1; half /= 2) {
    if (wave >= half && wave < 2 * half) {
      float *dst = red + (wave - half) * (MB * 4 * 64);
#pragma unroll
      for (int t = 0; t < MB; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(t * 4 + i) * 64 + lane] = acc[t][i];
    }
    __syncthreads();
    if (wave < half) {
      const float *src = red + wave * (MB * 4 * 64);
#pragma unroll
      for (int t = 0; t < MB; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] += src[(t * 4 + i) * 64 + lane];
    }
    __syncthreads();
  }
  if (wave == 0 && n < N) {
#pragma unroll
    for (int t = 0; t < MB; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + MBLK * t + 4 * kq + i;
        if (row < M) y[row * ldy + n] = acc[t][i];
      }
  }
}

template <int TYPE, int MB>
hipError_t launch2(int mode, int64_t M, int64_t N, int nb, const int8_t *q, const float *d,
                   const int32_t *bsum, const uint8_t *packed, float *y, int64_t ldy,
                   int32_t *dbg_S, int32_t *dbg_Mn, hipStream_t stream) {
  dim3 grid((unsigned)((N + TILE_N - 1) / TILE_N), (unsigned)((M + MBLK * MB - 1) / (MBLK * MB)));
  dim3 block(64 * WAVES);
  if (mode == 2)
    hipLaunchKernelGGL((qgemm_kernel<TYPE, MB, 2>), grid, block, 0, stream, M, N, nb, q, d, bsum,
                       packed, y, ldy, dbg_S, dbg_Mn);
  else if (mode == 1)
    hipLaunchKernelGGL((qgemm_kernel<TYPE, MB, 1>), grid, block, 0, stream, M, N, nb, q, d, bsum,
                       packed, y, ldy, dbg_S, dbg_Mn);
  else
    hipLaunchKernelGGL((qgemm_kernel<TYPE, MB, 0>), grid, block, 0, stream, M, N, nb, q, d, bsum,
                       packed, y, ldy, dbg_S, dbg_Mn);
  return hipGetLastError();
}

// 16-row m-blocks per workgroup, from the compiled set of each type (the
// sets leave out the sizes whose register demand exceeds the two-waves-per-
// SIMD budget).  Prefer the largest MB (the weight digits are built once per
// MB blocks) that still launches two waves per SIMD (n-tiles x m-chunks x 4
// waves >= 2048) with at most one padded m-block per chunk; otherwise the
// choice with the most waves.
constexpr int MB_Q4[] = {8, 5, 4, 3, 2, 1};
constexpr int MB_Q6[] = {10, 5, 4, 3, 2, 1};

template <int TYPE>
constexpr bool has_mb(int mb) {
  for (int v : (TYPE == 14 ? MB_Q6 : MB_Q4))
    if (v == mb) return true;
  return false;
}

template <int TYPE>
int pick_mb(int64_t M, int64_t N) {
  const int64_t mblocks = (M + MBLK - 1) / MBLK, ntiles = (N + TILE_N - 1) / TILE_N;
  int best = 1;
  int64_t best_waves = -1;
  for (int mb : (TYPE == 14 ? MB_Q6 : MB_Q4)) {
    if (mb > mblocks && mb != 1) continue;
    const int64_t chunks = (mblocks + mb - 1) / mb;
    const int64_t waste = chunks * mb - mblocks;
    const int64_t waves = ntiles * chunks * WAVES;
    if (waves >= 2048 && waste <= 1) return mb;
    if (waves > best_waves) {
      best_waves = waves;
      best = mb;
    }
  }
  return best;
}

template <int TYPE>
hipError_t launch_type(int mode, int64_t M, int64_t N, int nb, const int8_t *q, const float *d,
                       const int32_t *bsum, const uint8_t *packed, float *y, int64_t ldy,
                       int32_t *dbg_S, int32_t *dbg_Mn, hipStream_t stream) {
#define DQ_MB(V)                                                                          \
  case V:                                                                                 \
    if constexpr (has_mb<TYPE>(V))                                                        \
      return launch2<TYPE, V>(mode, M, N, nb, q, d, bsum, packed, y, ldy, dbg_S, dbg_Mn, \
                              stream);                                                    \
    break
  switch (pick_mb<TYPE>(M, N)) {
    DQ_MB(10);
    DQ_MB(8);
    DQ_MB(5);
    DQ_MB(4);
    DQ_MB(3);
    DQ_MB(2);
    default: break;
  }
#undef DQ_MB
  return launch2<TYPE, 1>(mode, M, N, nb, q, d, bsum, packed, y, ldy, dbg_S, dbg_Mn, stream);
}

}  // namespace

hipError_t launch_qgemm(int type, int mode, int64_t M, int64_t N, int64_t K, const int8_t *q,
                        const float *d, const int32_t *bsum, const uint8_t *packed, float *y,
                        int64_t ldy, int32_t *dbg_S, int32_t *dbg_Mn, hipStream_t stream) {
  const int nb = (int)(K / QK);
  if (type == 12)
    return launch_type<12>(mode, M, N, nb, q, d, bsum, packed, y, ldy, dbg_S, dbg_Mn, stream);
  return launch_type<14>(mode, M, N, nb, q, d, bsum, packed, y, ldy, dbg_S, dbg_Mn, stream);
}

}  // namespace dq
