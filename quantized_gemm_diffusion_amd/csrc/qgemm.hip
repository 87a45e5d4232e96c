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
//   Q6_K: v = sc * (q - 32) in [-4064, 4096] = 256 * hi + lo with lo in
//         [-128, 127] and hi = (v + 128) >> 8 in [-16, 16] (balanced base-256
//         digits), and S = R(lo) + 256 * R(hi).
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
#include "row_stats.h"

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

// Q6_K: 4 codes (bytes) -> lo / hi digit bytes of v = sc * (q - 32).  off2
// holds 128 - 32 * sc, so each 16-bit lane computes v + 128: its high byte is
// hi, and its low byte with the top bit flipped is the low byte of v, i.e. lo
// as a two's-complement byte.
__device__ inline void q6k_digits(uint32_t codes, uint32_t sc2, uint32_t off2, uint32_t &lo,
                                  uint32_t &hi) {
  // even codes (bytes 0, 2) and odd codes (bytes 1, 3) in 16-bit lanes
  const uint32_t ev = __builtin_amdgcn_perm(0u, codes, 0x0c020c00u);
  const uint32_t od = __builtin_amdgcn_perm(0u, codes, 0x0c030c01u);
  const s16x2 s2 = __builtin_bit_cast(s16x2, sc2), o2 = __builtin_bit_cast(s16x2, off2);
  const uint32_t ue = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, ev) * s2 + o2);
  const uint32_t uo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, od) * s2 + o2);
  lo = __builtin_amdgcn_perm(uo, ue, 0x06020400u) ^ 0x80808080u;
  hi = __builtin_amdgcn_perm(uo, ue, 0x07030501u);
}

// Every global read is a buffer load that writes LDS directly.  One buffer
// descriptor (gfx9 layout: base address, stride 0, size in bytes, flags)
// covers a whole operand; the per-load position is a wave-uniform scalar
// offset plus a per-lane offset that never changes, so issuing a load costs
// no vector instructions.  Every access is inside its operand by
// construction.
constexpr int DESC_FLAGS = 0x00020000;

__device__ inline i32x4 desc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, DESC_FLAGS};
}

// Buffer-to-LDS loads: M0 holds the LDS byte address; lane l writes its
// element at M0 + offset + l * size, and the immediate offset moves the
// global address by the same amount, so consecutive pieces of one copy share
// an M0 value.  A write of M0 needs one wait state before a load that uses
// it (the s_nop).  They are written as inline assembly so that the
// compiler, which cannot tell the LDS slots of the ring apart, does not wait
// for every one of them before each LDS read; all waits on them are explicit
// (wait_vm below).  Descriptor, scalar offset and LDS address are
// wave-uniform.  The copies themselves (dma_record, dma_tile) follow the
// record and tile layouts below.

// Wait until at most N of this wave's vector-memory loads are outstanding
// (they complete in issue order).  The memory clobber keeps every LDS read
// below the wait.
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait for this wave's LDS reads, before a slot they read is refilled.
__device__ inline void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Raw per-lane weight data of one (n-tile, super-block) tile, read from the
// tile's copy in LDS (same byte layout as in global memory).
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

__device__ inline void read_w(const uint8_t *tile, int lane, int col, int kq, RawQ4 &r) {
  r.head = *reinterpret_cast<const i32x4 *>(tile + 16 * col);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    r.rec[i] = *reinterpret_cast<const i32x4 *>(tile + Q4K_CODES_OFF + (i * 64 + lane) * 16);
}

__device__ inline void read_w(const uint8_t *tile, int lane, int col, int kq, RawQ6 &r) {
#pragma unroll
  for (int i = 0; i < 2; ++i) r.rec[i] = *reinterpret_cast<const i32x4 *>(tile + (i * 64 + lane) * 16);
  r.qh = *reinterpret_cast<const i32x4 *>(tile + Q6K_QH_OFF + lane * 16);
  r.sw = *reinterpret_cast<const uint32_t *>(tile + Q6K_SC_OFF + (kq * 16 + col) * 4);
  r.d = *reinterpret_cast<const uint32_t *>(tile + Q6K_D_OFF + 4 * (col >> 1)) >> (16 * (col & 1));
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
//
// With sub >= 0 (the debug hook for per-sub-block dots) every scale is
// replaced by 1 for sub-block sub and 0 for the others, so the digits' exact
// integer sum S is that sub-block's dot.
__device__ inline void make_digits(const RawQ4 &w, int kq, Digits &D, int sub = -1) {
  D.dw = half_bits_to_float((uint32_t)w.head[0]);
  D.dmw = half_bits_to_float((uint32_t)w.head[0] >> 16);
  const uint32_t D0 = (uint32_t)w.head[1], D1 = (uint32_t)w.head[2], D2 = (uint32_t)w.head[3];
  const uint32_t sc_lo = D0 & 0x3f3f3f3fu, mn_lo = D1 & 0x3f3f3f3fu;
  const uint32_t sc_hi = (D2 & 0x0f0f0f0fu) | ((D0 >> 2) & 0x30303030u);
  const uint32_t mn_hi = ((D2 >> 4) & 0x0f0f0f0fu) | ((D1 >> 2) & 0x30303030u);
  // bytes 0, 1 of SC / MN: sub-blocks 2kq and 2kq + 1
  const int sh16 = 16 * (kq & 1);
  uint32_t SC = (kq < 2 ? sc_lo : sc_hi) >> sh16;
  const uint32_t MN = (kq < 2 ? mn_lo : mn_hi) >> sh16;
  if (sub >= 0) SC = (2 * kq == sub ? 1u : 0u) | (2 * kq + 1 == sub ? 0x100u : 0u);
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

// Q6_K: chunk c of lane quarter kq is sub-block 4kq + c (scale byte c);
// sub >= 0 selects one sub-block as above.
__device__ inline void make_digits(const RawQ6 &w, int kq, Digits &D, int sub = -1) {
  D.dw = half_bits_to_float(w.d);
  D.dmw = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 2 * i + h;
      const int sc = sub >= 0 ? (4 * kq + c == sub ? 1 : 0) : (int)(int8_t)((w.sw >> (8 * c)) & 255);
      const uint32_t sc2 = ((uint32_t)sc & 0xffffu) * 0x10001u;
      const uint32_t off2 = ((uint32_t)(128 - 32 * sc) & 0xffffu) * 0x10001u;
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

// ---------------------------------------------------------------------------
// Staging.  A step is one (16-row block, super-block) pair; its activation
// record (codes, code sums, d_x: one quantized-activation record) is copied
// verbatim into an LDS slab of the wave's own ring of R slabs, D = R - 1
// steps ahead of its use, by five 1 KB loads.  The codes arrive already
// swizzled (16-byte unit u of row r at unit u ^ r), so the fragment reads (16
// lanes = 16 rows at one column unit) fall in 16 distinct bank groups.
// Weight tiles go the same way into W slots, W super-blocks ahead.
typedef __attribute__((address_space(3))) void *lds_ptr_t;

constexpr int MBLK = ACT_ROWS;  // rows per m-block
constexpr int SLAB = ACT_RECORD;
constexpr int GA = ACT_RECORD / 1024;  // loads per step

// A record: 1 KB pieces at offsets 0 .. 3072 from one M0, the last from a
// second (the immediate offset stops at 4095).
__device__ inline void dma_record(const i32x4 &d, uint32_t slab, int soff, int lane) {
  static_assert(GA == 5, "record copy is five 1 KB pieces");
  asm volatile(
      "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %2, %4, %5 offen lds\n\t"
      "buffer_load_dwordx4 %2, %4, %5 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %2, %4, %5 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %2, %4, %5 offen offset:3072 lds\n\t"
      "s_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %3, %4, %5 offen lds"
      :
      : "s"(slab), "s"(slab + 4096), "v"(16 * lane), "v"(4096 + 16 * lane), "s"(d), "s"(soff)
      : "memory");
}

// Weight tile of one (n-tile, super-block) into an LDS slot: 1 KB loads for
// the records, 256 B loads for the tail.  Q6_K's 288-byte tail (scales and
// d) is brought by two overlapping 256 B loads (bytes 3072.. and 3104..);
// where they overlap they write the same bytes.
template <bool Q6>
constexpr int wslot_bytes() {
  return Q6 ? 3376 : Q4K_TILE;
}
template <bool Q6>
constexpr int dma_per_tile() {
  return Q6 ? 5 : 3;
}

template <bool Q6>
__device__ inline void dma_tile(const i32x4 &d, uint32_t slot, int soff, int lane) {
  static_assert(Q6K_SC_OFF == 3072 && Q6K_TILE - 256 == 3104, "Q6_K tile tail offsets");
  if (!Q6) {
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %3, %4 offen lds\n\t"
        "buffer_load_dwordx4 %1, %3, %4 offen offset:1024 lds\n\t"
        "buffer_load_dword %2, %3, %4 offen offset:2048 lds"
        :
        : "s"(slot), "v"(16 * lane), "v"(4 * lane), "s"(d), "s"(soff)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %3, %4 offen lds\n\t"
        "buffer_load_dwordx4 %1, %3, %4 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %1, %3, %4 offen offset:2048 lds\n\t"
        "buffer_load_dword %2, %3, %4 offen offset:3072 lds\n\t"
        "buffer_load_dword %2, %3, %4 offen offset:3104 lds"
        :
        : "s"(slot), "v"(16 * lane), "v"(4 * lane), "s"(d), "s"(soff)
        : "memory");
  }
}

// One step's activation operands, read from the slab once and used against
// every weight tile the wave owns.
struct Frag {
  i32x4 a[4];   // codes of row `col`, chunks 0..3 of this lane's k-quarter
  f32x4 x4;     // d_x of rows 4kq .. 4kq+3
  f16x4 amin;   // (Q4_K) code sums of groups 2kq, 2kq+1 of row `col`
};

template <bool Q6>
__device__ inline void read_frag(const uint8_t *slab, const int (&frag)[4], int col, int kq,
                                 Frag &f) {
#pragma unroll
  for (int c = 0; c < 4; ++c) f.a[c] = *reinterpret_cast<const i32x4 *>(slab + frag[c]);
  f.x4 = *reinterpret_cast<const f32x4 *>(slab + ACT_DX_OFF + 16 * kq);
  f.amin = f16x4{};
  if (!Q6) f.amin = *reinterpret_cast<const f16x4 *>(slab + ACT_SUMS_OFF + 32 * col + 8 * kq);
  // issue every read of this slab here, a step before the slab is refilled,
  // so the refill's wait for outstanding LDS reads finds them done
  asm volatile("" ::: "memory");
}

// The MFMA part of one step for one weight tile.
struct StepOut {
  i32x4 rl, rh;
  f32x4 mnf;
};

template <bool Q6>
__device__ inline void step_mfma(const Frag &f, const Digits &D, StepOut &o) {
  o.rl = i32x4{};
  o.rh = i32x4{};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    o.rl = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.a[c], D.lo[c], o.rl, 0, 0, 0);
    o.rh = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.a[c], D.hi[c], o.rh, 0, 0, 0);
  }
  o.mnf = f32x4{};
  if (!Q6) {
    // the code sums of groups 2kq, 2kq+1 of row `col`, each as the exact
    // binary16 pair (lo, hi), against (m, m) of the same groups
    o.mnf = __builtin_amdgcn_mfma_f32_16x16x16f16(f.amin, D.bmin, o.mnf, 0, 0, 0);
  }
}

template <bool Q6>
__device__ inline void step_fold(const StepOut &o, const f32x4 &x4, float dw, float dmw,
                                 f32x4 &acc) {
  // d and dmin enter as binary32 registers: folded back into mixed-precision
  // FMAs (v_fma_mix_f32) they would cost a wait state before each
  // accumulation that reads the result
  asm("" : "+v"(dw), "+v"(dmw));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s_int = Q6 ? o.rl[i] + o.rh[i] * 256 : o.rl[i] + o.rh[i] * 8;
    const float tv = Q6 ? dw * (float)s_int : dw * (float)s_int - dmw * o.mnf[i];
    acc[i] += x4[i] * tv;
  }
}

// Debug stores: S and Mn of (row, n, super-block b) at (row * N + n) * nb + b;
// with sub >= 0 (one-hot scales) S alone, the dot of sub-block sub, at
// ((row * N + n) * nb + b) * J + sub, J sub-blocks per super-block.
template <bool Q6>
__device__ inline void step_debug(const StepOut &o, int64_t row0, int kq, int64_t n, int64_t M,
                                  int64_t N, int nb, int b, int32_t *dbg_S, int32_t *dbg_Mn,
                                  int sub) {
  constexpr int J = Q6 ? 16 : 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row0 + 4 * kq + i;
    if (row < M && n < N) {
      const int64_t o_ = (row * N + n) * nb + b;
      const int32_t S = Q6 ? o.rl[i] + o.rh[i] * 256 : o.rl[i] + o.rh[i] * 8;
      if (sub >= 0) {
        dbg_S[o_ * J + sub] = S;
      } else {
        dbg_S[o_] = S;
        dbg_Mn[o_] = Q6 ? 0 : (int32_t)o.mnf[i];
      }
    }
  }
}


// Launch shape of one GEMM variant: MB 16-row m-blocks per workgroup, NT
// 16-column weight tiles per wave (every activation record and fragment read
// feeds NT tiles), R activation slabs per wave (prefetch distance R - 1
// steps), WAVES waves splitting the reduction, and OCC workgroups per CU
// (LDS and registers are sized for it).
template <int MB_, int NT_, int R_, int WAVES_, int OCC_>
struct Shape {
  static constexpr int MB = MB_, NT = NT_, R = R_, WAVES = WAVES_, OCC = OCC_;
};

template <bool Q6, class SH>
constexpr int wave_lds() {
  return SH::R * SLAB + SH::NT * wslot_bytes<Q6>();
}
template <bool Q6, class SH>
constexpr int lds_bytes() {
  constexpr int ring = SH::WAVES * wave_lds<Q6, SH>();
  constexpr int red = SH::WAVES * SH::MB * SH::NT * 4 * 64 * 4;
  return ring > red ? ring : red;
}
constexpr int cap63(int v) { return v > 63 ? 63 : v; }

// Workgroups are dealt to the device's xcds XCDs in turn (workgroup i to XCD
// i mod xcds), and each XCD has its own L2.  The nrg row groups of one column
// group read the same weight tiles, so they are placed xcds apart in launch
// order: they run on one XCD at about the same time, and the tiles come from
// HBM once.  Column groups past the last complete set of xcds are numbered in
// order.
__device__ inline void place(int id, int ncg, int nrg, int xcds, int &cg, int &rg) {
  const int full = ncg / xcds * xcds;
  if (id < full * nrg) {
    const int slot = id / xcds, xcd = id - slot * xcds;
    cg = slot / nrg * xcds + xcd;
    rg = slot % nrg;
  } else {
    const int t = id - full * nrg;
    cg = full + t / nrg;
    rg = t % nrg;
  }
}

// One workgroup of WAVES waves: NT 16-column n-tiles x MB 16-row m-blocks x
// the whole reduction.  Wave w takes super-blocks b = w, w + WAVES, ...; it builds a
// super-block's weight digits once per tile and runs the MB steps of that
// super-block against them, each step reading its activation operands once
// for all NT tiles.  The WAVES f32 partial sums are added through LDS at the
// end, one after another in wave order.  MODE: 0 = canvas GEMM, 1 = gathered-row GEMM (same code, its
// own symbol so profiles tell the two workloads apart), 2 = debug stores of
// S and Mn, 3 = gathered-row GEMM whose output rows are folded into sampler
// states (one per row per workgroup, at part[row * npart + column group])
// instead of being stored, 4 = canvas GEMM over an interleaved gate/up
// matrix (n-tiles 2i and 2i + 1 are gate and up tile i) that stores
// silu(gate) * up, M x N/2, instead of the two tiles.
//
// Load schedule of one wave (every load is a buffer-to-LDS load, and loads
// complete in issue order, so a wait for one load also waits for every older
// one):
//   prologue      : tiles of super-block 0, slabs of steps 0 .. D-1
//   super-block i : wait for its tiles; digits
//     step s      : refill the slab read by step s - 1 with step s + D;
//                   at step TW = max(0, MB - D - 1) of the super-block, also
//                   refill the tile slots with super-block i + 1;
//                   wait for step s; MFMAs; fold
// The tile loads are issued as late as their latency allows: the first wait
// that covers them is the one for the next super-block's tiles, D + 1 steps
// later.  Loads past the wave's last tile or step repeat the last one (valid
// memory into a slot nobody reads again), so the number of loads issued after
// any given load is fixed, and each wait is a constant vmcnt: at most that
// many loads may still be outstanding when the awaited one must have landed.
template <int TYPE, class SH, int MODE>
__global__ __launch_bounds__(64 * SH::WAVES, SH::OCC) void qgemm_kernel(int M, int64_t N, int nb,
                                                                   const uint8_t *__restrict__ qa,
                                                                   uint32_t qa_bytes,
                                                                   const uint8_t *__restrict__ packed,
                                                                   float *__restrict__ y, int64_t ldy,
                                                                   int y_vec,
                                                                   int32_t *__restrict__ dbg_S,
                                                                   int32_t *__restrict__ dbg_Mn,
                                                                   float beta,
                                                                   float4 *__restrict__ part,
                                                                   int npart, int xcds, int sub) {
  constexpr bool Q6 = TYPE == 14;
  constexpr bool DEBUG = MODE == 2;
  constexpr int MB = SH::MB, NT = SH::NT, R = SH::R, D = R - 1, WAVES = SH::WAVES;
  constexpr int TB = Q6 ? Q6K_TILE : Q4K_TILE;
  constexpr int WSLOT = wslot_bytes<Q6>();
  constexpr int GW = NT * dma_per_tile<Q6>();
  constexpr int TW = MB - D - 1 > 0 ? MB - D - 1 : 0;  // step that refills the tile slots
  // loads issued after the awaited one: the next tiles (D + 1 steps after their
  // refill, or fewer when MB is small; the prologue issues D slabs after them)
  constexpr int WAIT_W = cap63((MB - 1 - TW < D ? MB - 1 - TW : D) * GA);
  static_assert(R >= 2 && (D * GA + GW) < 64, "pipeline shape");
  static_assert(lds_bytes<Q6, SH>() * SH::OCC <= 160 * 1024, "workgroups per CU");
  using Raw = typename std::conditional<Q6, RawQ6, RawQ4>::type;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[lds_bytes<Q6, SH>()];

  // the wave index is uniform across the wave; say so, so that every scalar
  // offset and LDS address derived from it stays in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int64_t ntiles = (N + TILE_N - 1) / TILE_N;
  const int nmb = (M + MBLK - 1) / MBLK;
  int cg, rg;  // column group (NT n-tiles) and row group (MB m-blocks) of this workgroup
  place((int)blockIdx.x, (int)((ntiles + NT - 1) / NT), (nmb + MB - 1) / MB, xcds, cg, rg);
  const int64_t nt0 = (int64_t)cg * NT;
  const int mb0 = rg * MB;  // first 16-row block of this workgroup
  // this wave's LDS: R activation slabs, then NT tile slots
  uint8_t *ring = lds + wave * wave_lds<Q6, SH>();
  uint8_t *wslot = ring + R * SLAB;
  const uint32_t ring_a = (uint32_t)(uintptr_t)(lds_ptr_t)ring;
  const uint32_t wslot_a = ring_a + R * SLAB;

  f32x4 acc[MB][NT];
#pragma unroll
  for (int t = 0; t < MB; ++t)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[t][j] = f32x4{};

  const int nbw = wave < nb ? (nb - wave + WAVES - 1) / WAVES : 0;  // this wave's super-blocks
  const int S = nbw * MB;                                           // and steps
  if (S > 0) {
    const i32x4 dqa = desc(qa, qa_bytes);
    // a tile index past the last n-tile repeats the last one (its columns are
    // not stored)
    i32x4 dw[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int64_t tj = nt0 + j < ntiles ? nt0 + j : ntiles - 1;
      dw[j] = desc(packed + tj * nb * TB, (uint32_t)(nb * TB));
    }
    int frag[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) frag[c] = col * QK + 16 * ((4 * kq + c) ^ col);

    // step s -> record of (super-block wave + WAVES * (s / MB), block mb0 + s % MB);
    // blocks past the last one re-load the last (their rows are never stored)
    auto issue_a = [&](int s, int slot) {
      s = s < S ? s : S - 1;
      const int bi = s / MB, t = s - bi * MB;
      const int mb = mb0 + t < nmb ? mb0 + t : nmb - 1;
      dma_record(dqa, ring_a + slot * SLAB, ((wave + WAVES * bi) * nmb + mb) * ACT_RECORD, lane);
    };
    auto issue_w = [&](int bi) {
      bi = bi < nbw ? bi : nbw - 1;
#pragma unroll
      for (int j = 0; j < NT; ++j)
        dma_tile<Q6>(dw[j], wslot_a + j * WSLOT, (wave + WAVES * bi) * TB, lane);
    };
    issue_w(0);
#pragma unroll
    for (int p = 0; p < D; ++p) issue_a(p, p);

    int s_next = D;     // next step to load
    int slot_next = D;  // its slab
    int slot_use = 0;   // slab of the current step
    for (int bi = 0; bi < nbw; ++bi) {
      const int b = wave + WAVES * bi;
      wait_vm<WAIT_W>();
      Digits Dg[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        Raw w;
        read_w(wslot + j * WSLOT, lane, col, kq, w);
        make_digits(w, kq, Dg[j], DEBUG ? sub : -1);
      }
#pragma unroll
      for (int t = 0; t < MB; ++t) {
        // the slab about to be refilled was read by the previous step, and
        // at step TW the tile slots were read by this super-block's digits
        wait_lds();
        issue_a(s_next, slot_next);
        ++s_next;
        slot_next = slot_next + 1 == R ? 0 : slot_next + 1;
        if (t == TW) issue_w(bi + 1);
        // loads issued after this step's slab: D slabs, and the tiles when
        // they were issued at or after the slab (steps TW .. TW + D of the
        // tiles' super-block, all of which lie in this super-block)
        if (t >= TW)
          wait_vm<D * GA + GW>();
        else
          wait_vm<D * GA>();
        Frag f;
        read_frag<Q6>(ring + slot_use * SLAB, frag, col, kq, f);
        slot_use = slot_use + 1 == R ? 0 : slot_use + 1;
        // tile j's MFMAs are issued before tile j - 1 is folded, so the fold
        // reads results that are already complete while the matrix core
        // works on the next tile
        StepOut out[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          step_mfma<Q6>(f, Dg[j], out[j]);
          if (DEBUG)
            step_debug<Q6>(out[j], (int64_t)(mb0 + t) * MBLK, kq, (nt0 + j) * TILE_N + col, M,
                           nt0 + j < ntiles ? N : 0, nb, b, dbg_S, dbg_Mn, sub);
          else if (j > 0)
            step_fold<Q6>(out[j - 1], f.x4, Dg[j - 1].dw, Dg[j - 1].dmw, acc[t][j - 1]);
        }
        if (!DEBUG) step_fold<Q6>(out[NT - 1], f.x4, Dg[NT - 1].dw, Dg[NT - 1].dmw, acc[t][NT - 1]);
      }
    }
    wait_vm<0>();  // no LDS write may land after this point
  }
  if (DEBUG) return;

  // Cross-wave reduction.  Every wave stores its partial sums to LDS; then
  // wave w owns output tiles (t, j) = w, w + WAVES, ... and adds the WAVES
  // partials of each element in wave order (the same order on every run).
  // Lane L of the owning wave takes row r = 4 * ((L >> 2) & 3) + (L >> 4) and
  // the 4 columns 4 * (L & 3) .. +3 of the tile: a 16-byte store per row
  // segment, and each 16-lane group of the LDS reads hits 16 distinct bank
  // groups.  Partial (t, j, i) of lane l sits at ((t * NT + j) * 4 + i) * 64 + l.
  constexpr int PER = MB * NT * 4;  // partial sums per lane
  float *red = reinterpret_cast<float *>(lds);
  __syncthreads();  // every wave is done with its ring
  {
    float *dst = red + wave * (PER * 64);
#pragma unroll
    for (int t = 0; t < MB; ++t)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[((t * NT + j) * 4 + i) * 64 + lane] = acc[t][j][i];
  }
  __syncthreads();
  const int ri = lane >> 4, rq = (lane >> 2) & 3, c0 = 4 * (lane & 3);
  const int r = 4 * rq + ri;
  if (MODE == 3) {
    // wave w takes the m-blocks t = w, w + WAVES, ...: each lane folds its
    // row's 4 columns of every n-tile, the 4 lanes of a row merge (lanes
    // 4g .. 4g+3 share row r), and one of them stores the row's state
    for (int t = wave; t < MB; t += WAVES) {
      RowStat st = stat_empty();
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int p = t * NT + j;
        const float *src = red + (p * 4 + ri) * 64 + 16 * rq + c0;
        f32x4 v = *reinterpret_cast<const f32x4 *>(src);
#pragma unroll
        for (int w = 1; w < WAVES; ++w) v += *reinterpret_cast<const f32x4 *>(src + w * (PER * 64));
        const int64_t n0 = (nt0 + j) * TILE_N + c0;
        const int64_t left = nt0 + j < ntiles ? N - n0 : 0;
        const float z[4] = {beta * v[0], beta * v[1], beta * v[2], beta * v[3]};
        stat_push4(st, z, (int)n0, left < 0 ? 0 : left > 4 ? 4 : (int)left);
      }
      st = stat_merge(st, stat_shfl_xor(st, 1));
      st = stat_merge(st, stat_shfl_xor(st, 2));
      const int row = (mb0 + t) * MBLK + r;
      if ((lane & 3) == 0 && row < M) part[(int64_t)row * npart + cg] = stat_pack(st);
    }
    return;
  }
  if constexpr (MODE == 4) {
    // the workgroup's two n-tiles are gate tile cg and up tile cg of an
    // interleaved gate/up matrix: wave w takes m-blocks t = w, w + WAVES, ...,
    // adds each tile's partials exactly as the plain store does, and stores
    // silu(gate) * up at columns 16 cg + c0 .. +3 of the M x N/2 output
    static_assert(NT == 2, "one gate/up tile pair per workgroup");
    for (int t = wave; t < MB; t += WAVES) {
      const int row = (mb0 + t) * MBLK + r;
      const float *sg = red + ((t * NT) * 4 + ri) * 64 + 16 * rq + c0;
      const float *su = red + ((t * NT + 1) * 4 + ri) * 64 + 16 * rq + c0;
      f32x4 g = *reinterpret_cast<const f32x4 *>(sg);
      f32x4 u = *reinterpret_cast<const f32x4 *>(su);
#pragma unroll
      for (int w = 1; w < WAVES; ++w) {
        g += *reinterpret_cast<const f32x4 *>(sg + w * (PER * 64));
        u += *reinterpret_cast<const f32x4 *>(su + w * (PER * 64));
      }
      if (nt0 + 1 >= ntiles || row >= M) continue;
      const f32x4 h = {silu_mul(g[0], u[0]), silu_mul(g[1], u[1]), silu_mul(g[2], u[2]),
                       silu_mul(g[3], u[3])};
      float *yp = y + (int64_t)row * ldy + (int64_t)cg * TILE_N + c0;
      if (y_vec) {
        *reinterpret_cast<f32x4 *>(yp) = h;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) yp[c] = h[c];
      }
    }
    return;
  }
  for (int p = wave; p < MB * NT; p += WAVES) {
    const int t = p / NT, j = p - t * NT;
    const int64_t n0 = (nt0 + j) * TILE_N + c0;
    const int row = (mb0 + t) * MBLK + r;
    const float *src = red + (p * 4 + ri) * 64 + 16 * rq + c0;
    f32x4 v = *reinterpret_cast<const f32x4 *>(src);
#pragma unroll
    for (int w = 1; w < WAVES; ++w) v += *reinterpret_cast<const f32x4 *>(src + w * (PER * 64));
    if (nt0 + j >= ntiles || row >= M || n0 >= N) continue;
    float *yp = y + (int64_t)row * ldy + n0;
    if (y_vec && n0 + 3 < N) {
      *reinterpret_cast<f32x4 *>(yp) = v;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (n0 + c < N) yp[c] = v[c];
    }
  }
}

// ---------------------------------------------------------------------------
// Canvas GEMM with one n-tile per wave and shared activation records.
//
// Every wave of a workgroup owns one 16-column n-tile and a contiguous range of
// super-blocks (its K-part), and runs all MB m-blocks of the workgroup's row
// group against that tile: acc[MB] f32x4, one digit set and one fragment keep
// a wave within 168 registers, so three waves share each SIMD where the
// canvas kernel has two (more waves to cover the waits; matrix and vector
// instructions of different waves overlap little on this part).  The NTW waves of a
// K-part read the same activation records, so each record is copied into LDS
// once for all of them: the K-part's ring holds two phases of P steps, and
// the workgroup crosses one barrier per phase.
//   step s of a K-part: record (super-block sb0 + s / MB, m-block mb0 + s % MB)
//   phase ph          : steps ph*P .. ph*P + P - 1, read from ring half ph & 1
// At the start of phase ph (just after the barrier that ends phase ph - 1)
// the records of phase ph + 1 are copied into the other half, which every
// wave finished reading in phase ph - 1; P of the K-part's waves each copy
// one record (five 1 KB buffer-to-LDS loads).  Each wave's weight tile goes
// into its own LDS slot the same way: the next super-block's tile is copied
// in the super-block's first phase, once this super-block's digits have
// read the slot, and only the phase that ends the super-block waits for it.
// Each phase ends with every wave waiting for its own loads and the barrier,
// so the records of phase ph + 1 are complete before any wave reads them.
// Column groups visit their K-parts' super-blocks in rotated order, so the
// workgroups running at once copy different records.  K-parts are balanced
// to within one super-block; every wave crosses the same barriers, whether
// or not its K-part has steps left.  At the end the KS partial sums of each
// output are added in K-part order through LDS and stored with 16-byte row
// segments.  MODE: 0 = canvas GEMM, 2 = debug stores of S and Mn (or of one
// sub-block's dots), 4 = SiLU(gate) * up of an interleaved gate/up matrix
// (pairs of n-tiles 2i, 2i + 1 inside one workgroup: NTW even).
template <int MB_, int NTW_, int KS_, int P_>
struct RingShape {
  static constexpr int MB = MB_, NTW = NTW_, KS = KS_, P = P_, WAVES = NTW_ * KS_;
};

template <bool Q6, class RS>
constexpr int ring_bytes() {
  return RS::KS * 2 * RS::P * SLAB + RS::WAVES * wslot_bytes<Q6>();
}
template <class RS>
constexpr int ring_red_bytes() {
  return RS::WAVES * RS::MB * 4 * 64 * 4;
}
template <bool Q6, class RS>
constexpr int ring_lds_bytes() {
  return ring_bytes<Q6, RS>() > ring_red_bytes<RS>() ? ring_bytes<Q6, RS>() : ring_red_bytes<RS>();
}

// End of a phase: this wave's loads other than the newest N have landed and
// its LDS reads are done; then every wave of the workgroup meets.
template <int N>
__device__ inline void phase_barrier() {
  wait_vm<N>();
  wait_lds();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int TYPE, class RS, int MODE>
__global__ __launch_bounds__(64 * RS::WAVES, 12 / RS::WAVES) void qgemm_ring_kernel(
    int M, int64_t N, int nb, const uint8_t *__restrict__ qa, uint32_t qa_bytes,
    const uint8_t *__restrict__ packed, float *__restrict__ y, int64_t ldy, int y_vec,
    int32_t *__restrict__ dbg_S, int32_t *__restrict__ dbg_Mn, int xcds, int sub) {
  constexpr bool Q6 = TYPE == 14;
  constexpr bool DEBUG = MODE == 2;
  constexpr int MB = RS::MB, NTW = RS::NTW, KS = RS::KS, P = RS::P, HP = MB / P;
  constexpr int TB = Q6 ? Q6K_TILE : Q4K_TILE;
  constexpr int GW = dma_per_tile<Q6>();
  static_assert(MB % P == 0 && P <= NTW, "phases split super-blocks; one record per wave");
  static_assert(ring_lds_bytes<Q6, RS>() * (12 / RS::WAVES) <= 160 * 1024, "LDS per CU");
  using Raw = typename std::conditional<Q6, RawQ6, RawQ4>::type;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[ring_lds_bytes<Q6, RS>()];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int kp = wave / NTW, tw = wave - kp * NTW;  // K-part and tile of this wave
  const int64_t ntiles = (N + TILE_N - 1) / TILE_N;
  const int nmb = (M + MBLK - 1) / MBLK;
  int cg, rg;
  place((int)blockIdx.x, (int)((ntiles + NTW - 1) / NTW), (nmb + MB - 1) / MB, xcds, cg, rg);
  const int64_t tile = (int64_t)cg * NTW + tw;
  const int64_t tile_c = tile < ntiles ? tile : ntiles - 1;  // past the last: repeat it, store nothing
  const int mb0 = rg * MB;
  const int sb0 = kp * nb / KS, nsb = (kp + 1) * nb / KS - sb0;  // this K-part's super-blocks
  const int nsb_max = (nb + KS - 1) / KS;                           // the longest K-part's
  const int steps = nsb * MB;
  // Column groups start their K-parts at different super-blocks, so the
  // workgroups running at the same time copy different records.
  const int rot = nsb > 0 ? cg % nsb : 0;
  auto sb_of = [&](int sbi) { return sb0 + (sbi + rot < nsb ? sbi + rot : sbi + rot - nsb); };

  uint8_t *ring = lds + kp * (2 * P * SLAB);
  uint8_t *wslot = lds + KS * 2 * P * SLAB + wave * wslot_bytes<Q6>();
  const uint32_t ring_a = (uint32_t)(uintptr_t)(lds_ptr_t)ring;
  const uint32_t wslot_a = (uint32_t)(uintptr_t)(lds_ptr_t)wslot;
  const i32x4 dqa = desc(qa, qa_bytes);
  const i32x4 dw = desc(packed + tile_c * nb * TB, (uint32_t)(nb * TB));
  int frag[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) frag[c] = col * QK + 16 * ((4 * kq + c) ^ col);

  // records of phase ph of this K-part (ring half ph & 1): wave tw copies
  // step ph * P + tw
  auto issue_phase = [&](int ph) {
    const int s = ph * P + tw;
    if (tw < P && s < steps) {
      const int sbi = s / MB, t = s - sbi * MB;
      const int mb = mb0 + t < nmb ? mb0 + t : nmb - 1;  // past the last m-block: repeat it
      dma_record(dqa, ring_a + ((ph & 1) * P + tw) * SLAB, (sb_of(sbi) * nmb + mb) * ACT_RECORD,
                 lane);
    }
  };

  f32x4 acc[MB];
#pragma unroll
  for (int t = 0; t < MB; ++t) acc[t] = f32x4{};
  Digits Dg;
  if (steps > 0) dma_tile<Q6>(dw, wslot_a, sb_of(0) * TB, lane);
  issue_phase(0);
  phase_barrier<0>();

  for (int sbi = 0; sbi < nsb_max; ++sbi) {
    const bool active = sbi < nsb;
    const bool wnext = sbi + 1 < nsb;
#pragma unroll
    for (int h = 0; h < HP; ++h) {
      const int ph = sbi * HP + h;
      if (h == 0 && active) {
        Raw w;
        read_w(wslot, lane, col, kq, w);
        make_digits(w, kq, Dg, DEBUG ? sub : -1);
      }
      // the other ring half was read in phase ph - 1, which every wave has
      // finished; the weight slot is refilled with the next super-block's
      // tile once its reads above are done, and only the phase that ends
      // the super-block waits for it
      issue_phase(ph + 1);
      if (h == 0 && wnext) {
        wait_lds();
        dma_tile<Q6>(dw, wslot_a, sb_of(sbi + 1) * TB, lane);
      }
      if (active) {
        const uint8_t *half = ring + (ph & 1) * (P * SLAB);
#pragma unroll
        for (int i = 0; i < P; ++i) {
          const int t = h * P + i;
          Frag f;
          read_frag<Q6>(half + i * SLAB, frag, col, kq, f);
          StepOut o;
          step_mfma<Q6>(f, Dg, o);
          if (DEBUG)
            step_debug<Q6>(o, (int64_t)(mb0 + t) * MBLK, kq, tile * TILE_N + col, M,
                           tile < ntiles ? N : 0, nb, sb_of(sbi), dbg_S, dbg_Mn, sub);
          else
            step_fold<Q6>(o, f.x4, Dg.dw, Dg.dmw, acc[t]);
        }
      }
      // the records of phase ph + 1 have landed once at most the loads
      // issued after them are outstanding: in a super-block's first phase,
      // the next tile's copies (unless this phase also ends the super-block,
      // whose end must find the tile in place); in any later phase, none
      if (h == 0 && HP > 1 && wnext)
        phase_barrier<GW>();
      else
        phase_barrier<0>();
    }
  }
  if (DEBUG) return;

  // Every wave stores its partial sums (the ring is no longer read: the last
  // phase ended with a barrier); wave (kp, tw) then adds the KS partials of
  // tile tw, in K-part order, for m-blocks t = kp, kp + KS, ..., and stores
  // them.  Lane L takes row r = 4 * ((L >> 2) & 3) + (L >> 4) and columns
  // 4 * (L & 3) .. +3 of the tile.
  float *red = reinterpret_cast<float *>(lds);
  {
    float *dst = red + wave * (MB * 4 * 64);
#pragma unroll
    for (int t = 0; t < MB; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(t * 4 + i) * 64 + lane] = acc[t][i];
  }
  __syncthreads();
  const int ri = lane >> 4, rq = (lane >> 2) & 3, c0 = 4 * (lane & 3);
  const int r = 4 * rq + ri;
  if constexpr (MODE == 4) {
    // tiles 2p and 2p + 1 of the workgroup are gate and up tile cg * NTW / 2
    // + p of an interleaved gate/up matrix: the (pair, m-block) items are
    // dealt to the waves in turn; each tile's KS partials are added exactly
    // as the plain store adds them, then silu(gate) * up is stored
    static_assert(NTW % 2 == 0, "whole gate/up tile pairs per workgroup");
    constexpr int PAIRS = NTW / 2;
    for (int item = wave; item < PAIRS * MB; item += RS::WAVES) {
      const int pr = item / MB, t = item - pr * MB;
      const int64_t tg = (int64_t)cg * NTW + 2 * pr;  // the pair's gate tile
      const int row = (mb0 + t) * MBLK + r;
      const float *sg = red + (2 * pr) * (MB * 4 * 64) + (t * 4 + ri) * 64 + 16 * rq + c0;
      const float *su = sg + MB * 4 * 64;
      f32x4 g = *reinterpret_cast<const f32x4 *>(sg);
      f32x4 u = *reinterpret_cast<const f32x4 *>(su);
#pragma unroll
      for (int k = 1; k < KS; ++k) {
        g += *reinterpret_cast<const f32x4 *>(sg + k * NTW * (MB * 4 * 64));
        u += *reinterpret_cast<const f32x4 *>(su + k * NTW * (MB * 4 * 64));
      }
      if (tg + 1 >= ntiles || row >= M) continue;
      const f32x4 h = {silu_mul(g[0], u[0]), silu_mul(g[1], u[1]), silu_mul(g[2], u[2]),
                       silu_mul(g[3], u[3])};
      float *yp = y + (int64_t)row * ldy + (tg / 2) * TILE_N + c0;
      if (y_vec) {
        *reinterpret_cast<f32x4 *>(yp) = h;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) yp[c] = h[c];
      }
    }
    return;
  }
  const int64_t n0 = tile * TILE_N + c0;
  for (int t = kp; t < MB; t += KS) {
    const int row = (mb0 + t) * MBLK + r;
    const float *src = red + tw * (MB * 4 * 64) + (t * 4 + ri) * 64 + 16 * rq + c0;
    f32x4 v = *reinterpret_cast<const f32x4 *>(src);
#pragma unroll
    for (int k = 1; k < KS; ++k) v += *reinterpret_cast<const f32x4 *>(src + k * NTW * (MB * 4 * 64));
    if (tile >= ntiles || row >= M || n0 >= N) continue;
    float *yp = y + (int64_t)row * ldy + n0;
    if (y_vec && n0 + 3 < N) {
      *reinterpret_cast<f32x4 *>(yp) = v;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (n0 + c < N) yp[c] = v[c];
    }
  }
}

template <int TYPE, class RS>
hipError_t launch_ring(int mode, int64_t M, int64_t N, int nb, const uint8_t *qa,
                       const uint8_t *packed, float *y, int64_t ldy, int32_t *dbg_S,
                       int32_t *dbg_Mn, hipStream_t stream, int sub = -1) {
  const int64_t nmb = (M + MBLK - 1) / MBLK;
  const int64_t ntiles = (N + TILE_N - 1) / TILE_N;
  dim3 grid((unsigned)(((ntiles + RS::NTW - 1) / RS::NTW) * ((nmb + RS::MB - 1) / RS::MB)));
  dim3 block(64 * RS::WAVES);
  const uint32_t qa_bytes = (uint32_t)(nmb * nb * ACT_RECORD);
  const int y_vec = (reinterpret_cast<uintptr_t>(y) % 16 == 0) && (ldy % 4 == 0);
  if (mode == 2)
    hipLaunchKernelGGL((qgemm_ring_kernel<TYPE, RS, 2>), grid, block, 0, stream, (int)M, N, nb,
                       qa, qa_bytes, packed, y, ldy, y_vec, dbg_S, dbg_Mn, device_props().xcds, sub);
  else if (mode == 4) {
    if constexpr (RS::NTW % 2 == 0)
      hipLaunchKernelGGL((qgemm_ring_kernel<TYPE, RS, 4>), grid, block, 0, stream, (int)M, N, nb,
                         qa, qa_bytes, packed, y, ldy, y_vec, dbg_S, dbg_Mn, device_props().xcds,
                         sub);
    else
      return hipErrorInvalidValue;  // gate/up pairs need an even number of tiles
  } else
    hipLaunchKernelGGL((qgemm_ring_kernel<TYPE, RS, 0>), grid, block, 0, stream, (int)M, N, nb,
                       qa, qa_bytes, packed, y, ldy, y_vec, dbg_S, dbg_Mn, device_props().xcds, sub);
  return hipGetLastError();
}

// Shapes of the shared-record kernel: 160 rows (10 m-blocks) in two K-parts,
// 128 rows (8 m-blocks) in two K-parts, 80 rows (5 m-blocks) in two K-parts;
// six n-tiles per K-part, twelve waves per workgroup.
using RingA = RingShape<10, 6, 2, 5>;
using RingB = RingShape<8, 6, 2, 4>;
using RingC = RingShape<5, 6, 2, 5>;

// The shared-record kernel runs one workgroup per CU for the whole launch,
// so it is taken where its grid makes one round that fills at least 70% of
// the CUs (more rounds measured slower than the two-workgroup-per-CU canvas
// kernel), with at most one padded m-block per row group and at least four
// super-blocks per K-part pair.  Measured on MI355X against the canvas
// kernel on the same device: LLaDA-8B's stacked gate/up (160 x 24576 x 4096,
// 256 workgroups of RingA) 2% and stacked Q/K/V (160 x 12288 x 4096, 256 of
// RingC) 4% faster, Dream-7B's stacked Q/K/V (512 x 4608 x 3584, 192 of
// RingB) 12% faster.  Returns 0 (none), 1 (RingA), 2 (RingB) or 3 (RingC).
inline int ring_pick(int64_t M, int64_t N, int nb) {
  if (nb < 4) return 0;
  const int64_t nmb = (M + MBLK - 1) / MBLK, ntiles = (N + TILE_N - 1) / TILE_N;
  const int64_t cus = device_props().cus;
  const int mbs[3] = {RingA::MB, RingB::MB, RingC::MB};
  for (int i = 0; i < 3; ++i) {
    const int mb = mbs[i];
    if (nmb < mb) continue;
    const int64_t rgs = (nmb + mb - 1) / mb;
    if (rgs * mb - nmb > 1) continue;
    const int64_t wgs = (ntiles + 5) / 6 * rgs;
    if (wgs <= cus && 10 * wgs >= 7 * cus) return i + 1;
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Narrow M (at most 32 rows, K of 8 to 16 super-blocks in pairs): the weight
// stream is the whole cost (the output projection on the requested rows moves
// 425 MB of weights for 32 rows), so the operands switch roles.  One
// persistent workgroup per CU, of K/512 waves, walks n-tiles blockIdx.x,
// blockIdx.x + grid, ...; wave w owns super-blocks w and w + K/512 and holds
// their activation fragments in registers for the whole launch.  The loop
// then only streams weight tiles: buffer-to-LDS loads into S slots per wave,
// explicit waits as in the canvas kernel.  A slot is refilled as soon as its
// tile has been read into registers, so S n-tiles are in flight while one is
// being computed.  The waves'
// partial sums of each tile meet in LDS (double buffered: one barrier per
// tile) and waves 0 .. MB-1 add them in wave order and store.  With STATS the
// storing lanes fold their outputs into a running sampler state instead (no
// stores in the loop), and each row's state of the workgroup goes to
// part[row * npart + blockIdx.x] at the end.
constexpr int NW_WAVES = 8;  // most waves per narrow workgroup
constexpr int NW_KB = 2;     // super-blocks per wave

// Output stores of the narrow kernel, through a buffer resource over the
// wave's 16-row block of y: a lane whose element is not stored passes an
// offset past the resource's size, which the hardware drops.  Every call is
// one store instruction whatever the lanes hold, so the explicit weight-load
// waits can count them.  The trailing s_nop covers the one wait state a VALU
// write to the data registers of a wider-than-8-byte store needs.
__device__ inline void bstore4(const i32x4 &d, uint32_t off, const f32x4 &v) {
  asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen\n\ts_nop 1" ::"v"(v), "v"(off), "s"(d)
               : "memory");
}
__device__ inline void bstore1(const i32x4 &d, uint32_t off, float v) {
  asm volatile("buffer_store_dword %0, %1, %2, 0 offen" ::"v"(v), "v"(off), "s"(d) : "memory");
}
constexpr uint32_t NW_DROP = 0x80000000u;  // offset past every narrow store resource

template <bool Q6, int MB, int S>
constexpr int narrow_lds() {
  return 2 * NW_WAVES * MB * 4 * 64 * 4 + NW_WAVES * S * NW_KB * wslot_bytes<Q6>();
}

template <int TYPE, int MB, int S, bool VEC, bool STATS>
__global__ __launch_bounds__(64 * NW_WAVES, 1) void qgemm_narrow_kernel(
    int M, int64_t N, int nb, const uint8_t *__restrict__ qa, const uint8_t *__restrict__ packed,
    float *__restrict__ y, int64_t ldy, float beta, float4 *__restrict__ part, int npart) {
  constexpr bool Q6 = TYPE == 14;
  constexpr int TB = Q6 ? Q6K_TILE : Q4K_TILE;
  constexpr int WSLOT = wslot_bytes<Q6>();
  constexpr int SET = NW_KB * WSLOT;                      // one n-tile of one wave
  constexpr int DPS = NW_KB * dma_per_tile<Q6>();         // loads per set
  constexpr int SC = STATS ? 0 : VEC ? 1 : 4;            // stores per tile (storing waves)
  constexpr int PER = MB * 4 * 64;                        // partial sums per wave per tile
  static_assert(S >= 2 && (S - 1) * DPS + S * SC < 64, "pipeline shape");
  static_assert(narrow_lds<Q6, MB, S>() <= 160 * 1024, "LDS");
  using Raw = typename std::conditional<Q6, RawQ6, RawQ4>::type;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[narrow_lds<Q6, MB, S>()];
  float *red = reinterpret_cast<float *>(lds);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int64_t ntiles = (N + TILE_N - 1) / TILE_N;
  const int nmb = (M + MBLK - 1) / MBLK;  // == MB
  const int nw = nb / NW_KB;              // waves in this workgroup
  const int64_t G = gridDim.x;

  // this wave's activation operands, for the whole launch
  Frag act[NW_KB][MB];
#pragma unroll
  for (int i = 0; i < NW_KB; ++i) {
    const int b = wave + nw * i;
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      const uint8_t *rec = qa + ((int64_t)b * nmb + t) * ACT_RECORD;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        act[i][t].a[c] = *reinterpret_cast<const i32x4 *>(rec + col * QK + 16 * ((4 * kq + c) ^ col));
      act[i][t].x4 = *reinterpret_cast<const f32x4 *>(rec + ACT_DX_OFF + 16 * kq);
      act[i][t].amin = f16x4{};
      if (!Q6) act[i][t].amin = *reinterpret_cast<const f16x4 *>(rec + ACT_SUMS_OFF + 32 * col + 8 * kq);
    }
  }
  // all of them in before the first weight load: from here on the only
  // memory loads in flight are this wave's weight tiles
  __builtin_amdgcn_s_waitcnt(0);

  uint8_t *slots = lds + 2 * NW_WAVES * PER * 4 + wave * S * SET;
  const uint32_t slots_a = (uint32_t)(uintptr_t)(lds_ptr_t)slots;
  // tiles of n-tile blockIdx.x + kk * grid (past the end: the last n-tile,
  // whose slot is never read) into slot `slot`
  auto issue = [&](int64_t kk, int slot) {
    int64_t nt = blockIdx.x + kk * G;
    nt = nt < ntiles ? nt : ntiles - 1;
    const i32x4 d = desc(packed + nt * nb * TB, (uint32_t)(nb * TB));
#pragma unroll
    for (int i = 0; i < NW_KB; ++i)
      dma_tile<Q6>(d, slots_a + slot * SET + i * WSLOT, (wave + nw * i) * TB, lane);
  };

  // the storing wave's resource: rows 16 t .. 16 t + 15 of y
  const bool storer = wave < MB;
  const int t_st = storer ? wave : 0;
  const int rows_st = M - MBLK * t_st < MBLK ? M - MBLK * t_st : MBLK;
  const i32x4 dy = STATS ? i32x4{} : desc(y + (int64_t)t_st * MBLK * ldy,
                                          (uint32_t)(((int64_t)(rows_st - 1) * ldy + N) * 4));
  const int ri = lane >> 4, rq = (lane >> 2) & 3, c0 = 4 * (lane & 3);
  const int r_st = 4 * rq + ri;  // this lane's row and first column in the tile
  RowStat st = stat_empty();      // STATS: this lane's row over its columns so far

#pragma unroll
  for (int p = 0; p < S; ++p) issue(p, p);

  int slot = 0;
  for (int64_t k = 0;; ++k) {
    const int64_t nt = blockIdx.x + k * G;
    if (nt >= ntiles) break;
    // younger than this tile's loads: the next S - 1 sets, and the stores of
    // the last S tiles (fewer in the first tiles: then the wait only waits
    // longer)
    if (SC > 0 && storer && k >= S)
      wait_vm<(S - 1) * DPS + S * SC>();
    else
      wait_vm<(S - 1) * DPS>();
    Raw w[NW_KB];
#pragma unroll
    for (int i = 0; i < NW_KB; ++i) read_w(slots + slot * SET + i * WSLOT, lane, col, kq, w[i]);
    // the slot is free once its reads are in: refill it with the tile S ahead
    wait_lds();
    issue(k + S, slot);
    slot = slot + 1 == S ? 0 : slot + 1;

    f32x4 acc[MB];
#pragma unroll
    for (int t = 0; t < MB; ++t) acc[t] = f32x4{};
#pragma unroll
    for (int i = 0; i < NW_KB; ++i) {
      Digits Dg;
      make_digits(w[i], kq, Dg);
#pragma unroll
      for (int t = 0; t < MB; ++t) {
        StepOut o;
        step_mfma<Q6>(act[i][t], Dg, o);
        step_fold<Q6>(o, act[i][t].x4, Dg.dw, Dg.dmw, acc[t]);
      }
    }

    // partial sums into this tile's buffer; the buffer alternates, so the one
    // written here was last read before the previous tile's barrier
    float *dst = red + (int)(k & 1) * NW_WAVES * PER + wave * PER;
#pragma unroll
    for (int t = 0; t < MB; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(t * 4 + i) * 64 + lane] = acc[t][i];
    wait_lds();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (storer) {
      const float *src = red + (int)(k & 1) * NW_WAVES * PER + (t_st * 4 + ri) * 64 + 16 * rq + c0;
      f32x4 v = *reinterpret_cast<const f32x4 *>(src);
      for (int ww = 1; ww < nw; ++ww) v += *reinterpret_cast<const f32x4 *>(src + ww * PER);
      const int64_t n0 = nt * TILE_N + c0;
      const uint32_t off = (uint32_t)(((int64_t)r_st * ldy + n0) * 4);
      const bool row_ok = r_st < rows_st;
      if (STATS) {
        const int64_t left = row_ok ? N - n0 : 0;
        const float z[4] = {beta * v[0], beta * v[1], beta * v[2], beta * v[3]};
        stat_push4(st, z, (int)n0, left < 0 ? 0 : left > 4 ? 4 : (int)left);
      } else if (VEC) {
        bstore4(dy, row_ok && n0 < N ? off : NW_DROP, v);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) bstore1(dy, row_ok && n0 + c < N ? off + 4 * c : NW_DROP, v[c]);
      }
    }
  }
  wait_vm<0>();  // no LDS write may land after the workgroup ends
  if (STATS && storer) {
    st = stat_merge(st, stat_shfl_xor(st, 1));
    st = stat_merge(st, stat_shfl_xor(st, 2));
    if ((lane & 3) == 0 && r_st < rows_st)
      part[(int64_t)(t_st * MBLK + r_st) * npart + blockIdx.x] = stat_pack(st);
  }
}

// Single-row Q6_K projection (M = 1, e.g. the logits of one committed
// position).  With one row, 15 of the 16 rows of the MFMA's activation
// operand would be padding; here they carry the row's 16 sub-blocks instead.
// Operand row j holds the row's codes where k lies in sub-block j and zeros
// elsewhere (the lane of row j and k-quarter kq has them in chunk j - 4kq),
// so one int32 accumulation over the super-block's four chunks against the
// raw 6-bit codes q (0..63, no digit split) leaves dot_j(q) = sum over
// sub-block j of q * x in accumulator row j: every per-sub-block dot of the
// super-block at once, for a quarter of the MFMAs and none of the digit
// work.  The Q6_K offset enters as dot_j(q - 32) = dot_j(q) - 32 * xs_j (xs_j
// the sum of the row's codes over sub-block j, formed once per launch), and
// the lane of column n and k-quarter kq holds sub-blocks 4kq .. 4kq + 3 --
// the four scale bytes its tile dword already carries -- so it forms
// sum_j sc_j * dot_j(q - 32) over them in exact integers (|dot_j| < 2^18,
// |sc_j * dot_j| < 2^25), scales it by d_x * d in binary32, and the four
// k-quarters of a column are added by two lane exchanges in a fixed order.
// Streaming, slots, waits and the cross-wave sum are those of the narrow
// kernel above, with one float per column and wave.
//
// With GATHER the row is canvas row idx[0], read and quantized here (every
// wave its own two blocks, by the quantization rule every quantizer shares)
// instead of by a separate gather-quantize launch; flags[0] reports an index
// outside [0, L) (the row is then taken as zeros).
struct Gather {
  const float *canvas = nullptr;
  int64_t ldc = 0, L = 0;
  const int32_t *idx = nullptr;
  int32_t *flags = nullptr;
  int vec = 0;  // rows 16-byte aligned
};

template <int S, bool VEC, bool STATS, bool GATHER>
__global__ __launch_bounds__(64 * NW_WAVES, 1) void qgemm_row1_kernel(
    int64_t N, int nb, const uint8_t *__restrict__ qa, const uint8_t *__restrict__ packed,
    float *__restrict__ y, float beta, float4 *__restrict__ part, int npart, Gather gx) {
  constexpr int TB = Q6K_TILE;
  constexpr int WSLOT = wslot_bytes<true>();
  constexpr int SET = NW_KB * WSLOT;
  constexpr int DPS = NW_KB * dma_per_tile<true>();
  constexpr int SC = STATS ? 0 : VEC ? 1 : 4;
  static_assert(S >= 2 && (S - 1) * DPS + S * SC < 64, "pipeline shape");
  constexpr int RED = 2 * NW_WAVES * 64 * 4;  // column sums per wave, double buffered
  static_assert(RED + NW_WAVES * S * SET <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[RED + NW_WAVES * S * SET];
  float *red = reinterpret_cast<float *>(lds);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int64_t ntiles = (N + TILE_N - 1) / TILE_N;
  const int nw = nb / NW_KB;
  const int64_t G = gridDim.x;

  // activation operands of super-blocks wave and wave + nw (one record each,
  // one 16-row block of which only row 0 is real)
  i32x4 act[NW_KB][4];
  int xs32[NW_KB][4];  // 32 * xs_j for the lane's sub-blocks j = 4kq + t
  float dx[NW_KB];
  const int cs = col - 4 * kq;  // the chunk holding sub-block `col` in this lane's k-quarter
  if (GATHER) {
    const int32_t src = gx.idx[0];
    const bool valid = src >= 0 && (int64_t)src < gx.L;
    if (blockIdx.x == 0 && threadIdx.x == 0) gx.flags[0] = valid ? 0 : 1;
    const float *xr = gx.canvas + (valid ? (int64_t)src : 0) * gx.ldc;
#pragma unroll
    for (int i = 0; i < NW_KB; ++i) {
      // lane l holds values 4l .. 4l+3 of the block, i.e. a quarter of unit l / 4
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (valid) {
        const float *p = xr + (int64_t)(wave + nw * i) * QK + 4 * lane;
        if (gx.vec) {
          const f32x4 t = *reinterpret_cast<const f32x4 *>(p);
          v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = p[e];
        }
      }
      const float amax = block_amax(v);
      int c4[4];
      quant4(v, amax, c4);
      const int word = (int)pack4(c4);
      dx[i] = block_dx(amax);
      // the unit (16 codes) of sub-block `col`: the words of lanes 4 col .. 4 col + 3
      i32x4 unit;
#pragma unroll
      for (int e = 0; e < 4; ++e) unit[e] = __shfl(word, 4 * col + e, 64);
#pragma unroll
      for (int c = 0; c < 4; ++c) act[i][c] = c == cs ? unit : i32x4{};
      // code sums of units 4kq + t: each lane's 4 codes, summed over the quad
      // of lanes that holds a unit, then fetched from the quad's first lane
      int q4 = __builtin_amdgcn_sdot4(word, 0x01010101, 0, false);
      q4 += dpp<DPP_QUAD_1032>(q4);
      q4 += dpp<DPP_QUAD_2301>(q4);
#pragma unroll
      for (int t = 0; t < 4; ++t) xs32[i][t] = 32 * __shfl(q4, 4 * (4 * kq + t), 64);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NW_KB; ++i) {
      const uint8_t *rec = qa + (int64_t)(wave + nw * i) * ACT_RECORD;  // row 0: unit u at 16 u
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const i32x4 v = *reinterpret_cast<const i32x4 *>(rec + 16 * (4 * kq + c));
        act[i][c] = c == cs ? v : i32x4{};
        int sum = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) sum = __builtin_amdgcn_sdot4(v[e], 0x01010101, sum, false);
        xs32[i][c] = 32 * sum;
      }
      dx[i] = *reinterpret_cast<const float *>(rec + ACT_DX_OFF);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  uint8_t *slots = lds + RED + wave * S * SET;
  const uint32_t slots_a = (uint32_t)(uintptr_t)(lds_ptr_t)slots;
  auto issue = [&](int64_t kk, int slot) {
    int64_t nt = blockIdx.x + kk * G;
    nt = nt < ntiles ? nt : ntiles - 1;
    const i32x4 d = desc(packed + nt * nb * TB, (uint32_t)(nb * TB));
#pragma unroll
    for (int i = 0; i < NW_KB; ++i)
      dma_tile<true>(d, slots_a + slot * SET + i * WSLOT, (wave + nw * i) * TB, lane);
  };

  // wave 0 stores: lanes 0..3 carry columns 4 * lane .. 4 * lane + 3 of the tile
  const bool storer = wave == 0;
  const int c0 = 4 * (lane & 3);
  const i32x4 dy = STATS ? i32x4{} : desc(y, (uint32_t)(N * 4));
  RowStat st = stat_empty();

#pragma unroll
  for (int p = 0; p < S; ++p) issue(p, p);

  int slot = 0;
  for (int64_t k = 0;; ++k) {
    const int64_t nt = blockIdx.x + k * G;
    if (nt >= ntiles) break;
    if (SC > 0 && storer && k >= S)
      wait_vm<(S - 1) * DPS + S * SC>();
    else
      wait_vm<(S - 1) * DPS>();
    RawQ6 w[NW_KB];
#pragma unroll
    for (int i = 0; i < NW_KB; ++i) read_w(slots + slot * SET + i * WSLOT, lane, col, kq, w[i]);
    wait_lds();
    issue(k + S, slot);
    slot = slot + 1 == S ? 0 : slot + 1;

    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < NW_KB; ++i) {
      i32x4 dot = i32x4{};
#pragma unroll
      for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = 2 * r + h;
          const uint32_t u = (uint32_t)w[i].qh[c];
          const uint32_t w0 = (uint32_t)w[i].rec[r][2 * h], w1 = (uint32_t)w[i].rec[r][2 * h + 1];
          const i32x4 q = {(int)((w0 & 0x0f0f0f0fu) | ((u << 4) & 0x30303030u)),
                           (int)(((w0 >> 4) & 0x0f0f0f0fu) | ((u << 2) & 0x30303030u)),
                           (int)((w1 & 0x0f0f0f0fu) | (u & 0x30303030u)),
                           (int)(((w1 >> 4) & 0x0f0f0f0fu) | ((u >> 2) & 0x30303030u))};
          dot = __builtin_amdgcn_mfma_i32_16x16x64_i8(act[i][c], q, dot, 0, 0, 0);
        }
      }
      // accumulator element t: sub-block 4kq + t of column `col`
      int sacc = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int sc = (int)(int8_t)((w[i].sw >> (8 * t)) & 255u);
        sacc += sc * (dot[t] - xs32[i][t]);
      }
      const float dd = dx[i] * half_bits_to_float(w[i].d);
      acc += dd * (float)sacc;
    }
    // the column's four k-quarters, in a fixed order
    acc += __shfl_xor(acc, 16, 64);
    acc += __shfl_xor(acc, 32, 64);

    float *buf = red + (int)(k & 1) * NW_WAVES * 64;
    if (lane < 16) buf[wave * 64 + lane] = acc;
    wait_lds();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (storer) {
      const float *src = buf + c0;
      f32x4 v = *reinterpret_cast<const f32x4 *>(src);
      for (int ww = 1; ww < nw; ++ww) v += *reinterpret_cast<const f32x4 *>(src + ww * 64);
      const int64_t n0 = nt * TILE_N + c0;
      const bool ok = lane < 4;
      const uint32_t off = (uint32_t)(n0 * 4);
      if (STATS) {
        const int64_t left = ok ? N - n0 : 0;
        const float z[4] = {beta * v[0], beta * v[1], beta * v[2], beta * v[3]};
        stat_push4(st, z, (int)n0, left < 0 ? 0 : left > 4 ? 4 : (int)left);
      } else if (VEC) {
        bstore4(dy, ok && n0 < N ? off : NW_DROP, v);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) bstore1(dy, ok && n0 + c < N ? off + 4 * c : NW_DROP, v[c]);
      }
    }
  }
  wait_vm<0>();  // no LDS write may land after the workgroup ends
  if (STATS && storer) {
    st = stat_merge(st, stat_shfl_xor(st, 1));
    st = stat_merge(st, stat_shfl_xor(st, 2));
    if (lane == 0) part[blockIdx.x] = stat_pack(st);
  }
}

// Q6_K projection of 2 to 4 rows (R = 1; the template also takes R = 2 for 8
// rows), the same idea for more than one row.  In row group g (rows 4g ..
// 4g + 3) operand row 4m + p holds row 4g + m's codes
// where k lies in k-quarter p of the chunk and zeros elsewhere, so one MFMA
// per chunk c separates the chunk's four sub-blocks: accumulator element i
// of the lane of column n and k-quarter kq is the dot of row 4g + kq over
// k-quarter i of chunk c, i.e. sub-block 4i + c.  Over the four chunks a
// lane thus sees all 16 sub-blocks of its own row and forms S = sum_j sc_j *
// dot_j in exact integers (|dot_j| < 2^16), the weight operand being q - 32
// as a byte (no digit split); the rows need no exchange between lanes.
// Streaming, slots and waits follow the narrow kernel; wave g < R stores row
// group g, one element per lane and tile.
template <int R, int S, bool STATS>
__global__ __launch_bounds__(64 * NW_WAVES, 1) void qgemm_rows4_kernel(
    int M, int64_t N, int nb, const uint8_t *__restrict__ qa, const uint8_t *__restrict__ packed,
    float *__restrict__ y, int64_t ldy, float beta, float4 *__restrict__ part, int npart) {
  constexpr int TB = Q6K_TILE;
  constexpr int WSLOT = wslot_bytes<true>();
  constexpr int SET = NW_KB * WSLOT;
  constexpr int DPS = NW_KB * dma_per_tile<true>();
  constexpr int SC = STATS ? 0 : 1;
  static_assert(R >= 1 && R <= 2, "at most 8 rows");
  static_assert(S >= 2 && (S - 1) * DPS + S * SC < 64, "pipeline shape");
  constexpr int RED = 2 * NW_WAVES * R * 64 * 4;  // per wave and row group, double buffered
  static_assert(RED + NW_WAVES * S * SET <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[RED + NW_WAVES * S * SET];
  float *red = reinterpret_cast<float *>(lds);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int64_t ntiles = (N + TILE_N - 1) / TILE_N;
  const int nw = nb / NW_KB;
  const int64_t G = gridDim.x;

  // operand rows: this lane supplies row 4g + col / 4 in k-quarter kq when
  // col % 4 == kq, zeros otherwise; dx of the lane's output row 4g + kq
  i32x4 act[NW_KB][R][4];
  float dx[NW_KB][R];
  const bool mine = (col & 3) == kq;
#pragma unroll
  for (int i = 0; i < NW_KB; ++i) {
    const uint8_t *rec = qa + (int64_t)(wave + nw * i) * ACT_RECORD;  // one 16-row block
#pragma unroll
    for (int g = 0; g < R; ++g) {
      const int r = 4 * g + (col >> 2);  // the operand row's row of the record
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const i32x4 v = *reinterpret_cast<const i32x4 *>(rec + r * QK + 16 * ((4 * kq + c) ^ r));
        act[i][g][c] = mine ? v : i32x4{};
      }
      dx[i][g] = *reinterpret_cast<const float *>(rec + ACT_DX_OFF + 4 * (4 * g + kq));
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  uint8_t *slots = lds + RED + wave * S * SET;
  const uint32_t slots_a = (uint32_t)(uintptr_t)(lds_ptr_t)slots;
  auto issue = [&](int64_t kk, int slot) {
    int64_t nt = blockIdx.x + kk * G;
    nt = nt < ntiles ? nt : ntiles - 1;
    const i32x4 d = desc(packed + nt * nb * TB, (uint32_t)(nb * TB));
#pragma unroll
    for (int i = 0; i < NW_KB; ++i)
      dma_tile<true>(d, slots_a + slot * SET + i * WSLOT, (wave + nw * i) * TB, lane);
  };

  // storing wave g: row 4g + kq, column `col` of each tile
  const bool storer = wave < R;
  const int row_st = 4 * (storer ? wave : 0) + kq;
  const bool row_ok = row_st < M;
  const i32x4 dy = STATS ? i32x4{} : desc(y, (uint32_t)(((int64_t)(M - 1) * ldy + N) * 4));
  RowStat st = stat_empty();

#pragma unroll
  for (int p = 0; p < S; ++p) issue(p, p);

  int slot = 0;
  for (int64_t k = 0;; ++k) {
    const int64_t nt = blockIdx.x + k * G;
    if (nt >= ntiles) break;
    if (SC > 0 && storer && k >= S)
      wait_vm<(S - 1) * DPS + S * SC>();
    else
      wait_vm<(S - 1) * DPS>();
    RawQ6 w[NW_KB];
    uint32_t scw[NW_KB][4];  // scale dword of k-quarter i: byte c = sub-block 4i + c
#pragma unroll
    for (int i = 0; i < NW_KB; ++i) {
      const uint8_t *tile = slots + slot * SET + i * WSLOT;
      read_w(tile, lane, col, kq, w[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        scw[i][q] = *reinterpret_cast<const uint32_t *>(tile + Q6K_SC_OFF + (q * 16 + col) * 4);
    }
    wait_lds();
    issue(k + S, slot);
    slot = slot + 1 == S ? 0 : slot + 1;

    float acc[R];
#pragma unroll
    for (int g = 0; g < R; ++g) acc[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < NW_KB; ++i) {
      int sacc[R];
#pragma unroll
      for (int g = 0; g < R; ++g) sacc[g] = 0;
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = 2 * r2 + h;
          const uint32_t u = (uint32_t)w[i].qh[c];
          const uint32_t w0 = (uint32_t)w[i].rec[r2][2 * h], w1 = (uint32_t)w[i].rec[r2][2 * h + 1];
          const uint32_t code[4] = {(w0 & 0x0f0f0f0fu) | ((u << 4) & 0x30303030u),
                                    ((w0 >> 4) & 0x0f0f0f0fu) | ((u << 2) & 0x30303030u),
                                    (w1 & 0x0f0f0f0fu) | (u & 0x30303030u),
                                    ((w1 >> 4) & 0x0f0f0f0fu) | ((u >> 2) & 0x30303030u)};
          // q - 32 as a two's-complement byte: (q + 128 - 32) with bit 7 flipped,
          // no borrow between bytes
          i32x4 qm;
#pragma unroll
          for (int t = 0; t < 4; ++t) qm[t] = (int)(((code[t] | 0x80808080u) - 0x20202020u) ^ 0x80808080u);
#pragma unroll
          for (int g = 0; g < R; ++g) {
            const i32x4 dot = __builtin_amdgcn_mfma_i32_16x16x64_i8(act[i][g][c], qm, i32x4{}, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int sc = (int)(int8_t)((scw[i][q] >> (8 * c)) & 255u);  // sub-block 4q + c
              sacc[g] += sc * dot[q];
            }
          }
        }
      }
      const float dw = half_bits_to_float(w[i].d);
#pragma unroll
      for (int g = 0; g < R; ++g) acc[g] += (dx[i][g] * dw) * (float)sacc[g];
    }

    float *buf = red + (int)(k & 1) * NW_WAVES * R * 64;
#pragma unroll
    for (int g = 0; g < R; ++g) buf[(wave * R + g) * 64 + lane] = acc[g];
    wait_lds();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (storer) {
      const float *src = buf + wave * 64 + lane;  // row group `wave` of wave 0
      float v = src[0];
      for (int ww = 1; ww < nw; ++ww) v += src[ww * R * 64];
      const int64_t n = nt * TILE_N + col;
      if (STATS) {
        const float z[4] = {beta * v, 0.f, 0.f, 0.f};
        stat_push4(st, z, (int)n, row_ok && n < N ? 1 : 0);
      } else {
        const uint32_t off = (uint32_t)(((int64_t)row_st * ldy + n) * 4);
        bstore1(dy, row_ok && n < N ? off : NW_DROP, v);
      }
    }
  }
  wait_vm<0>();  // no LDS write may land after the workgroup ends
  if (STATS && storer) {
#pragma unroll
    for (int x = 1; x < 16; x <<= 1) st = stat_merge(st, stat_shfl_xor(st, x));
    if (col == 0 && row_ok) part[(int64_t)row_st * npart + blockIdx.x] = stat_pack(st);
  }
}

// Narrow launches: one workgroup per CU (fewer if there are fewer tiles).
inline int64_t narrow_grid(int64_t N) {
  const int64_t ntiles = (N + TILE_N - 1) / TILE_N;
  const int64_t cus = device_props().cus;
  return ntiles < cus ? ntiles : cus;
}

// part == nullptr: store y; otherwise fold the rows into part (npart =
// narrow_grid(N) states per row).
template <int TYPE, int MB>
hipError_t launch_narrow(int64_t M, int64_t N, int nb, const uint8_t *qa, const uint8_t *packed,
                         float *y, int64_t ldy, float beta, float4 *part, hipStream_t stream) {
  dim3 grid((unsigned)narrow_grid(N)), block(64 * (nb / NW_KB));
  const int npart = (int)grid.x;
  const bool vec = (reinterpret_cast<uintptr_t>(y) % 16 == 0) && (ldy % 4 == 0) && (N % 4 == 0);
  // Q6_K tiles are larger: two slots per wave fit beside the sums, Q4_K three
  constexpr int S = TYPE == 14 ? 2 : 3;
  const int m = (int)M;
  if (part)
    hipLaunchKernelGGL((qgemm_narrow_kernel<TYPE, MB, S, true, true>), grid, block, 0, stream, m,
                       N, nb, qa, packed, nullptr, (int64_t)0, beta, part, npart);
  else if (vec)
    hipLaunchKernelGGL((qgemm_narrow_kernel<TYPE, MB, S, true, false>), grid, block, 0, stream, m,
                       N, nb, qa, packed, y, ldy, 0.0f, nullptr, 0);
  else
    hipLaunchKernelGGL((qgemm_narrow_kernel<TYPE, MB, S, false, false>), grid, block, 0, stream, m,
                       N, nb, qa, packed, y, ldy, 0.0f, nullptr, 0);
  return hipGetLastError();
}

// Single-row Q6_K launches (the same grid and eligibility as the narrow kernel);
// with gx.idx set the kernel gathers and quantizes the row itself.
hipError_t launch_row1(int64_t N, int nb, const uint8_t *qa, const uint8_t *packed, float *y,
                       float beta, float4 *part, const Gather &gx, hipStream_t stream) {
  dim3 grid((unsigned)narrow_grid(N)), block(64 * (nb / NW_KB));
  const bool vec = (reinterpret_cast<uintptr_t>(y) % 16 == 0) && (N % 4 == 0);
#define DQ_ROW1(VEC, STATS, GATHER)                                                           \
  hipLaunchKernelGGL((qgemm_row1_kernel<2, VEC, STATS, GATHER>), grid, block, 0, stream, N, nb, \
                     qa, packed, y, beta, part, (int)grid.x, gx)
  if (gx.idx) {
    if (part) DQ_ROW1(true, true, true);
    else if (vec) DQ_ROW1(true, false, true);
    else DQ_ROW1(false, false, true);
  } else {
    if (part) DQ_ROW1(true, true, false);
    else if (vec) DQ_ROW1(true, false, false);
    else DQ_ROW1(false, false, false);
  }
#undef DQ_ROW1
  return hipGetLastError();
}

// Q6_K launches for 2 to 4 rows (the same grid and eligibility as the narrow
// kernel).  One row group only: at 5 to 8 rows the two-group variant measured
// no faster than the narrow kernel (both stream at about 5.3 TB/s there).
hipError_t launch_rows4(int64_t M, int64_t N, int nb, const uint8_t *qa, const uint8_t *packed,
                        float *y, int64_t ldy, float beta, float4 *part, hipStream_t stream) {
  dim3 grid((unsigned)narrow_grid(N)), block(64 * (nb / NW_KB));
  const int m = (int)M, np = (int)grid.x;
  if (part)
    hipLaunchKernelGGL((qgemm_rows4_kernel<1, 2, true>), grid, block, 0, stream, m, N, nb, qa,
                       packed, nullptr, (int64_t)0, beta, part, np);
  else
    hipLaunchKernelGGL((qgemm_rows4_kernel<1, 2, false>), grid, block, 0, stream, m, N, nb, qa,
                       packed, y, ldy, 0.0f, nullptr, 0);
  return hipGetLastError();
}

// The narrow kernel serves up to 2 blocks of 16 rows, K of 8 to 16 super-blocks
// in pairs (2 per wave, at least 4 waves), enough n-tiles to give every CU a
// stream, a row stride that keeps a 16-row block of y under 2 GB (its store
// offsets are 32-bit, with the top bit marking a dropped store), and not the
// debug or gate/up mode.
inline bool use_narrow(int mode, int64_t M, int64_t N, int nb, int64_t ldy) {
  const int64_t ntiles = (N + TILE_N - 1) / TILE_N;
  return mode != 2 && mode != 4 && M <= 2 * MBLK && nb % NW_KB == 0 && nb >= 4 * NW_KB &&
         nb <= NW_WAVES * NW_KB && ntiles >= 4 * device_props().cus && ldy <= (int64_t(1) << 25);
}

struct Extra {  // arguments of the debug and sampler-state modes
  int32_t *dbg_S = nullptr, *dbg_Mn = nullptr;
  int sub = -1;  // debug: the one sub-block whose dot S becomes, or -1
  float beta = 0.0f;
  float4 *part = nullptr;
  int npart = 0;
};

template <int TYPE, class SH>
hipError_t launch2(int mode, int64_t M, int64_t N, int nb, const uint8_t *qa,
                   const uint8_t *packed, float *y, int64_t ldy, const Extra &x,
                   hipStream_t stream) {
  const int64_t nmb = (M + MBLK - 1) / MBLK;
  const int64_t ntiles = (N + TILE_N - 1) / TILE_N;
  dim3 grid((unsigned)(((ntiles + SH::NT - 1) / SH::NT) * ((nmb + SH::MB - 1) / SH::MB)));
  dim3 block(64 * SH::WAVES);
  const int m = (int)M;
  const uint32_t qa_bytes = (uint32_t)(nmb * nb * ACT_RECORD);
  // rows of y can take 16-byte stores
  const int y_vec = (reinterpret_cast<uintptr_t>(y) % 16 == 0) && (ldy % 4 == 0);
#define DQ_LAUNCH(MODE)                                                                        \
  hipLaunchKernelGGL((qgemm_kernel<TYPE, SH, MODE>), grid, block, 0, stream, m, N, nb, qa,        \
                     qa_bytes, packed, y, ldy, y_vec, x.dbg_S, x.dbg_Mn, x.beta, x.part, x.npart, \
                     device_props().xcds, x.sub)
  switch (mode) {
    case 1: DQ_LAUNCH(1); break;
    case 2: DQ_LAUNCH(2); break;
    case 3: DQ_LAUNCH(3); break;
    case 4:
      if constexpr (SH::NT == 2) {
        DQ_LAUNCH(4);
        break;
      } else {
        return hipErrorInvalidValue;  // the launcher gives mode 4 two tiles per wave
      }
    default: DQ_LAUNCH(0); break;
  }
#undef DQ_LAUNCH
  return hipGetLastError();
}

// Compiled variants, indexed by the number of 16-row m-blocks per workgroup:
// two n-tiles per wave, and as many activation slabs (3 for Q4_K at 4 waves,
// else 2) as keep the workgroups' LDS within the CU's 160 KB; a third slab
// measured no faster at 8 waves or for Q6_K.  WAVES = 8 (one workgroup per
// CU) splits the reduction twice as finely as WAVES = 4 (two workgroups per
// CU) over the same tile grid, and WAVES = 2 (four workgroups per CU, the
// same 8 waves) splits it half as finely: each wave's pipeline is twice as
// long and the cross-wave sum has two partials.  Two variants take three n-tiles per wave
// (four waves, two slabs; five m-blocks for Q4_K, four for the larger Q6_K
// tiles): every activation fragment read then feeds three tiles, and the
// rings (68.6 KB and 81.5 KB) still leave room for two workgroups per CU.
template <int TYPE, int MB, int WAVES, int NT = 2>
struct ShapeOf {
  using type = Shape<MB, NT, (TYPE == 14 || NT == 3 || WAVES != 4) ? 2 : 3, WAVES,
                     WAVES == 8 ? 1 : WAVES == 2 ? 4 : 2>;
};
constexpr int MB_SET[] = {8, 5, 4, 3, 2, 1};
constexpr int NT_STATS = 2;  // n-tiles per wave of the sampler-state launches (mode 3)

struct Pick {
  int mb, waves, nt;
};

// Fraction of workgroup slots used over a launch of wgs workgroups with
// per_cu workgroups resident per CU.
inline double fill(int64_t wgs, int64_t per_cu) {
  const int64_t slots = device_props().cus * per_cu;
  const int64_t rounds = (wgs + slots - 1) / slots;
  return (double)wgs / (double)(rounds * slots);
}

// Prefer the largest MB (weight digits are built once per MB steps) with at
// most one padded m-block per m-chunk that gives at least one wave per SIMD
// (1024 waves at 4 waves per workgroup).  Take three n-tiles per wave (Q4_K
// with MB = 5, Q6_K with MB = 4) when that makes at least a full round of two
// workgroups per CU and fills the workgroup slots at least as well, or runs
// four or more rounds (LLaDA-8B's stacked Q/K/V and gate/up at L = 160: 512
// and 1024 workgroups instead of 768 and 1536, 8-11% faster on MI355X;
// Dream-7B's logits on 64 gathered rows: 3168 workgroups, 8% faster).  With
// 1024 or more workgroups, the three-tile shapes and Q4_K at MB = 8 take
// 2-wave workgroups, four per CU (LLaDA's gate/up 7% and Dream's gate/up 4%
// faster; below 1024 workgroups four per CU cannot fill the CUs).  Use
// 8 waves per workgroup when the reduction has at least 16 super-blocks
// (each wave still gets 2 or more) and that fills the CUs in whole rounds
// better than 4 (one 8-wave or two 4-wave workgroups per CU).
inline Pick pick_shape(int type, int mode, int64_t M, int64_t N, int64_t nb) {
  const int64_t mblocks = (M + MBLK - 1) / MBLK;
  const int64_t ntiles = (N + TILE_N - 1) / TILE_N;
  const int64_t tiles = (ntiles + 1) / 2;
  int mb = 1;
  int64_t best_waves = -1;
  for (int cand : MB_SET) {
    if (cand > mblocks && cand != 1) continue;
    const int64_t chunks = (mblocks + cand - 1) / cand;
    const int64_t waste = chunks * cand - mblocks;
    const int64_t waves = tiles * chunks * 4;
    if (waves >= 1024 && waste <= 1) {
      mb = cand;
      break;
    }
    if (waves > best_waves) {
      best_waves = waves;
      mb = cand;
    }
  }
  const int64_t chunks = (mblocks + mb - 1) / mb;
  const int64_t wgs = tiles * chunks;
  Pick pk{mb, 4, 2};
  const int64_t wgs3 = (ntiles + 2) / 3 * chunks;
  const int64_t CUS = device_props().cus;
  if (((type == 12 && mb == 5) || (type == 14 && mb == 4)) && wgs3 >= 2 * CUS &&
      (fill(wgs3, 2) >= fill(wgs, 2) || wgs3 >= 8 * CUS))
    pk = Pick{mb, wgs3 >= 4 * CUS ? 2 : 4, 3};
  else if (type == 12 && mb == 8 && wgs >= 4 * CUS)
    pk = Pick{8, 2, 2};
  else if (nb >= 16 && fill(wgs, 1) > fill(wgs, 2) + 0.05)
    pk = Pick{mb, 8, 2};
  // The sampler-state launch keeps two tiles per wave (one state per row per
  // 32-column group) but the same waves: each output element is then summed
  // in the same order as the plain launch stores it, bit for bit.  So does
  // the gate/up launch with silu(gate) * up in its epilogue (one gate/up tile
  // pair per workgroup).
  if (mode == 3 || mode == 4) pk.nt = 2;
  return pk;
}

template <int TYPE>
hipError_t launch_type(int mode, int64_t M, int64_t N, int nb, const uint8_t *qa,
                       const uint8_t *packed, float *y, int64_t ldy, const Extra &x,
                       hipStream_t stream) {
  const Pick pk = pick_shape(TYPE, mode, M, N, nb);
  if (pk.nt == 3) {
    constexpr int MB3 = TYPE == 12 ? 5 : 4;
    if (pk.waves == 2)
      return launch2<TYPE, typename ShapeOf<TYPE, MB3, 2, 3>::type>(mode, M, N, nb, qa, packed, y,
                                                                    ldy, x, stream);
    return launch2<TYPE, typename ShapeOf<TYPE, MB3, 4, 3>::type>(mode, M, N, nb, qa, packed, y,
                                                                  ldy, x, stream);
  }
  if (pk.waves == 2) {  // (Q4_K, MB 5 or 8) or (Q6_K, MB 4), two tiles per wave
    if constexpr (TYPE == 12) {
      if (pk.mb == 8)
        return launch2<TYPE, typename ShapeOf<TYPE, 8, 2>::type>(mode, M, N, nb, qa, packed, y,
                                                                 ldy, x, stream);
      return launch2<TYPE, typename ShapeOf<TYPE, 5, 2>::type>(mode, M, N, nb, qa, packed, y, ldy,
                                                               x, stream);
    } else {
      return launch2<TYPE, typename ShapeOf<TYPE, 4, 2>::type>(mode, M, N, nb, qa, packed, y, ldy,
                                                               x, stream);
    }
  }
#define DQ_MB(X)                                                                               \
  case X:                                                                                      \
    if (pk.waves == 8)                                                                         \
      return launch2<TYPE, typename ShapeOf<TYPE, X, 8>::type>(mode, M, N, nb, qa, packed, y,  \
                                                               ldy, x, stream);                \
    return launch2<TYPE, typename ShapeOf<TYPE, X, 4>::type>(mode, M, N, nb, qa, packed, y,    \
                                                             ldy, x, stream)
  switch (pk.mb) {
    DQ_MB(8);
    DQ_MB(5);
    DQ_MB(4);
    DQ_MB(3);
    DQ_MB(2);
    default: break;
  }
#undef DQ_MB
  if (pk.waves == 8)
    return launch2<TYPE, typename ShapeOf<TYPE, 1, 8>::type>(mode, M, N, nb, qa, packed, y, ldy,
                                                             x, stream);
  return launch2<TYPE, typename ShapeOf<TYPE, 1, 4>::type>(mode, M, N, nb, qa, packed, y, ldy, x,
                                                           stream);
}

}  // namespace

hipError_t launch_qgemm(int type, int mode, int64_t M, int64_t N, int64_t K, const uint8_t *qa,
                        const uint8_t *packed, float *y, int64_t ldy, int32_t *dbg_S,
                        int32_t *dbg_Mn, hipStream_t stream, int sub) {
  const int nb = (int)(K / QK);
  if (use_narrow(mode, M, N, nb, ldy)) {
    const bool two = M > MBLK;
    if (type == 14 && M == 1) return launch_row1(N, nb, qa, packed, y, 0.0f, nullptr, Gather{}, stream);
    if (type == 14 && M <= 4) return launch_rows4(M, N, nb, qa, packed, y, ldy, 0.0f, nullptr, stream);
    if (type == 12)
      return two ? launch_narrow<12, 2>(M, N, nb, qa, packed, y, ldy, 0.0f, nullptr, stream)
                 : launch_narrow<12, 1>(M, N, nb, qa, packed, y, ldy, 0.0f, nullptr, stream);
    return two ? launch_narrow<14, 2>(M, N, nb, qa, packed, y, ldy, 0.0f, nullptr, stream)
               : launch_narrow<14, 1>(M, N, nb, qa, packed, y, ldy, 0.0f, nullptr, stream);
  }
  switch (mode == 0 || mode == 2 || mode == 4 ? ring_pick(M, N, nb) : 0) {
    case 1:
      return type == 12 ? launch_ring<12, RingA>(mode, M, N, nb, qa, packed, y, ldy, dbg_S, dbg_Mn, stream, sub)
                        : launch_ring<14, RingA>(mode, M, N, nb, qa, packed, y, ldy, dbg_S, dbg_Mn, stream, sub);
    case 2:
      return type == 12 ? launch_ring<12, RingB>(mode, M, N, nb, qa, packed, y, ldy, dbg_S, dbg_Mn, stream, sub)
                        : launch_ring<14, RingB>(mode, M, N, nb, qa, packed, y, ldy, dbg_S, dbg_Mn, stream, sub);
    case 3:
      return type == 12 ? launch_ring<12, RingC>(mode, M, N, nb, qa, packed, y, ldy, dbg_S, dbg_Mn, stream, sub)
                        : launch_ring<14, RingC>(mode, M, N, nb, qa, packed, y, ldy, dbg_S, dbg_Mn, stream, sub);
    default: break;
  }
  Extra x;
  x.dbg_S = dbg_S;
  x.dbg_Mn = dbg_Mn;
  x.sub = sub;
  if (type == 12) return launch_type<12>(mode, M, N, nb, qa, packed, y, ldy, x, stream);
  return launch_type<14>(mode, M, N, nb, qa, packed, y, ldy, x, stream);
}

// The sampler-state GEMM takes the narrow kernel where the plain one would
// (its row-stride condition does not apply: nothing is stored per column),
// else the canvas kernel with one state per row per column group.
// The single-row output projection with the gather and quantization folded
// into the GEMM launch (Q6_K, one row, where the narrow kernel would run):
// part == nullptr stores y (row stride irrelevant for one row), else folds
// sampler states.  Returns false, launching nothing, where it does not apply.
bool launch_rows_gather_row1(int type, int64_t M, int64_t N, int64_t K, const float *canvas,
                             int64_t ldc, const int32_t *idx, int64_t L, int32_t *flags,
                             const uint8_t *packed, float *y, float beta, float4 *part,
                             hipStream_t stream, hipError_t &err) {
  const int nb = (int)(K / QK);
  if (type != 14 || M != 1 || !use_narrow(part ? 3 : 1, M, N, nb, part ? 0 : N)) return false;
  Gather gx;
  gx.canvas = canvas;
  gx.ldc = ldc;
  gx.L = L;
  gx.idx = idx;
  gx.flags = flags;
  gx.vec = reinterpret_cast<uintptr_t>(canvas) % 16 == 0 && ldc % 4 == 0;
  err = launch_row1(N, nb, nullptr, packed, y, beta, part, gx, stream);
  return true;
}

int qgemm_stats_parts(int64_t M, int64_t N, int64_t K) {
  const int nb = (int)(K / QK);
  if (use_narrow(3, M, N, nb, 0)) return (int)narrow_grid(N);
  const int64_t ntiles = (N + TILE_N - 1) / TILE_N;
  return (int)((ntiles + NT_STATS - 1) / NT_STATS);
}

hipError_t launch_qgemm_stats(int type, int64_t M, int64_t N, int64_t K, const uint8_t *qa,
                              const uint8_t *packed, float beta, float4 *part, int npart,
                              hipStream_t stream) {
  const int nb = (int)(K / QK);
  if (use_narrow(3, M, N, nb, 0)) {
    const bool two = M > MBLK;
    if (type == 14 && M == 1)
      return launch_row1(N, nb, qa, packed, nullptr, beta, part, Gather{}, stream);
    if (type == 14 && M <= 4)
      return launch_rows4(M, N, nb, qa, packed, nullptr, 0, beta, part, stream);
    if (type == 12)
      return two ? launch_narrow<12, 2>(M, N, nb, qa, packed, nullptr, 0, beta, part, stream)
                 : launch_narrow<12, 1>(M, N, nb, qa, packed, nullptr, 0, beta, part, stream);
    return two ? launch_narrow<14, 2>(M, N, nb, qa, packed, nullptr, 0, beta, part, stream)
               : launch_narrow<14, 1>(M, N, nb, qa, packed, nullptr, 0, beta, part, stream);
  }
  Extra x;
  x.beta = beta;
  x.part = part;
  x.npart = npart;
  if (type == 12) return launch_type<12>(3, M, N, nb, qa, packed, nullptr, 0, x, stream);
  return launch_type<14>(3, M, N, nb, qa, packed, nullptr, 0, x, stream);
}

}  // namespace dq
