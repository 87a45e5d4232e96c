// attention.hip -- bidirectional attention of every canvas position over all
// L positions, on the f16 matrix cores of gfx950 (mojo-dllm "Architecture"
// page, "A forward pass", step 2: RoPE rotates Q and K, attention runs over all
// L positions with no mask; "Source map": NORM and NEOX RoPE; aiboss88 news
// page, capability list: attention on f16 tensor cores, 16 queries per warp,
// keys streamed through shared memory with an online softmax).
//
// out[l][h*128 + d] = sum_j p_j v_j[d] / sum_j p_j,
//   p_j = exp(q_l . k_j / sqrt(128) - max),  over the L keys j of kv head
//   h / (H / Hkv); q and k rotated (RoPE, binary32, fixed operation order), then
//   q, k, v rounded to binary16; products accumulated in binary32.
//
// Two kernels.  The pack kernel rotates K (RoPE), rounds K and V to f16 and
// writes, per kv head and block of 32 keys, the exact LDS image the attention
// kernel contracts against (K row-major, V transposed), so every key block is
// converted once per kv head, not once per query workgroup.  The attention
// kernel gives each wave 16 queries of one head; a workgroup of QW waves takes
// 16 QW consecutive queries of that head and copies the head's block images
// into a ring of 4 LDS slots by buffer-to-LDS loads (no registers; up to 3
// blocks in flight; one barrier per block).  Per block a wave runs
//   S^T (32 keys x 16 queries) = K Q^T : 2 tiles x 4 v_mfma_f32_16x16x32_f16
//   O^T (128 d x 16 queries) += V^T P^T : 8 tiles x 1 v_mfma_f32_16x16x32_f16
// Transposing both products puts one query in each lane (column l % 16 of
// every accumulator), so the softmax state of a query (running max, the
// rescale factor) is a per-lane value shared by the 4 lanes l % 16 + 16g: the
// block maximum takes two cross-lane steps and the output rescale none.
// P^T leaves the S^T accumulators in exactly the B-operand layout of the
// second product once the keys of its contraction are ordered as the lanes
// hold them (key 16t + 4g + i at contraction slot 8g + 4t + i); the V^T image
// is written in that key order.
#include "attention.h"

#include "dq_internal.h"

namespace dq {
namespace {

constexpr int AD = 128;          // head dimension
constexpr int KB = 32;           // keys per block
constexpr int K_LD = AD + 8;     // K image rows, halves (272 B: conflict-free 16-B reads)
constexpr int VT_LD = KB + 8;    // V^T image rows, halves (80 B)
constexpr int K_BYTES = KB * K_LD * 2;           // 8704
constexpr int VT_BYTES = AD * VT_LD * 2;         // 10240
constexpr int IMG_BYTES = 20 * 1024;             // one block's image, in 1 KB pieces
static_assert(K_BYTES + VT_BYTES <= IMG_BYTES, "block image");
// LDS slots per workgroup: 4 (80 KB, two workgroups per CU; deeper rings at
// one workgroup per CU measured slower).  A wave keeps at most 4 * 20 / QW
// loads in flight, within the hardware's count of 63.
constexpr int ring_slots(int) { return 4; }

// RoPE of one pair (a, b) by (c, s): a' = fma(a, c, -(b*s)), b' = fma(b, c, a*s),
// every step rounded in binary32.  The empty asm pins each result as a binary32
// value in a register: otherwise the compiler may fuse an fma with the
// following conversion to f16 (v_fma_mix*_f16), which rounds once, straight to
// f16, instead of to binary32 and then to f16.
__device__ inline void rope_pair(float a, float b, float c, float s, float &ra, float &rb) {
  float bs = __fmul_rn(b, s);
  float as = __fmul_rn(a, s);
  asm volatile("" : "+v"(bs), "+v"(as));
  float x = __fmaf_rn(a, c, -bs);
  float y = __fmaf_rn(b, c, as);
  asm volatile("" : "+v"(x), "+v"(y));
  ra = x;
  rb = y;
}

// The key held at contraction slot j (0..31) of a block in the second product:
// slot 8g + 4t + i holds key 16t + 4g + i.
__device__ inline int slot_key(int j) { return 16 * ((j >> 2) & 1) + 4 * (j >> 3) + (j & 3); }

// This lane's Q^T operand (d = 32c + 8g + e, e = 0..7) of one query: the row
// (128 f32) rotated in registers and rounded to f16; rrow is the query's
// RoPE table row (64 x (cos, sin)).
template <int MODE>
__device__ inline void load_q(const float *__restrict__ row, const float *__restrict__ rrow, int g,
                              f16x8 (&qf)[4]) {
  float x[4][8];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float4 lo = *reinterpret_cast<const float4 *>(row + 32 * c + 8 * g);
    const float4 hi = *reinterpret_cast<const float4 *>(row + 32 * c + 8 * g + 4);
    x[c][0] = lo.x, x[c][1] = lo.y, x[c][2] = lo.z, x[c][3] = lo.w;
    x[c][4] = hi.x, x[c][5] = hi.y, x[c][6] = hi.z, x[c][7] = hi.w;
  }
  if (MODE == 1) {  // NORM: pairs (2i, 2i+1), i = 16c + 4g + e/2
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int i = 16 * c + 4 * g + e / 2;
        const float2 cs = *reinterpret_cast<const float2 *>(rrow + 2 * i);
        rope_pair(x[c][e], x[c][e + 1], cs.x, cs.y, x[c][e], x[c][e + 1]);
      }
  } else if (MODE == 2) {  // NEOX: pairs (i, i + 64): chunk c with chunk c + 2
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 32 * c + 8 * g + e;
        const float2 cs = *reinterpret_cast<const float2 *>(rrow + 2 * i);
        rope_pair(x[c][e], x[c + 2][e], cs.x, cs.y, x[c][e], x[c + 2][e]);
      }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[c][e] = (_Float16)x[c][e];
}

// One block of 32 keys (K image kl, V^T image vt; keys kb0 .. kb0 + 31, those
// past L masked) into this wave's online softmax state (m, lsum) and O^T.
__device__ inline void attend_block(const _Float16 *kl, const _Float16 *vt, const f16x8 (&qf)[4],
                                    int kb0, int L, int col, int g, float &m, float &lsum,
                                    f32x4 (&o)[8]) {
  // log2(e) / sqrt(128): scores go straight to exp2
  const float sc = 1.4426950408889634f * 0.08838834764831845f;
  // S^T: lane holds query col, keys 16t + 4g + e
  f32x4 s[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    s[t] = f32x4{};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f16x8 ka = *reinterpret_cast<const f16x8 *>(kl + (16 * t + col) * K_LD + 32 * c + 8 * g);
      s[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qf[c], s[t], 0, 0, 0);
    }
  }
  float bm = -INFINITY;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = s[t][e] * sc;
      if (kb0 + 16 * t + 4 * g + e >= L) v = -INFINITY;
      s[t][e] = v;
      bm = fmaxf(bm, v);
    }
  bm = fmaxf(bm, __shfl_xor(bm, 16));
  bm = fmaxf(bm, __shfl_xor(bm, 32));
  const float mn = fmaxf(m, bm);
  const float alpha = __builtin_amdgcn_exp2f(m - mn);  // 0 on the first block
  m = mn;
  f16x8 pf;
  float ps = 0.0f;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = __builtin_amdgcn_exp2f(s[t][e] - mn);
      ps += p;
      pf[4 * t + e] = (_Float16)p;
    }
  lsum = lsum * alpha + ps;
  // O^T += V^T P^T
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    o[dt] *= alpha;
    const f16x8 va = *reinterpret_cast<const f16x8 *>(vt + (16 * dt + col) * VT_LD + 8 * g);
    o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pf, o[dt], 0, 0, 0);
  }
}

// The 4 lanes of a query hold partial sums over their keys; store O = O^T / lsum.
__device__ inline void store_out(float lsum, const f32x4 (&o)[8], float *orow, int out_vec) {
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  const float inv = 1.0f / lsum;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const f32x4 v = o[dt] * inv;
    if (out_vec) {
      *reinterpret_cast<f32x4 *>(orow + 16 * dt) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) orow[16 * dt + e] = v[e];
    }
  }
}

// Workgroups are dealt to the device's XCDS XCDs in turn, and each XCD has
// its own L2: number the workgroups of one kv head XCDS apart (while whole
// groups of XCDS kv heads remain) so that they run on one XCD and fetch that
// head's images into one L2.
// With fewer kv heads than XCDs (dividing XCDS), each kv head's workgroups go
// to XCDS / nkv XCDs instead (all of them stay busy).
__device__ inline void place_kv(int id, int nkv, int per, int XCDS, int &kv, int &item) {
  if (nkv < XCDS && XCDS % nkv == 0 && per % (XCDS / nkv) == 0) {
    const int slot = id / XCDS, xcd = id - slot * XCDS;
    kv = xcd % nkv;
    item = slot * (XCDS / nkv) + xcd / nkv;
    return;
  }
  const int full = nkv / XCDS * XCDS;
  if (id < full * per) {
    const int slot = id / XCDS, xcd = id - slot * XCDS;
    kv = slot / per * XCDS + xcd;
    item = slot % per;
  } else {
    const int t = id - full * per;
    kv = full + t / per;
    item = t % per;
  }
}

// ---------------------------------------------------------------------------
// Pack: image (hk, b) of kv head hk and block b is 1280 16-byte chunks, one per
// thread of the 5 workgroups of items 5b .. 5b + 4 of kv head hk:
//   chunks 0 .. 543     K rows: row k = c / 17; chunk c % 17 of the row (16:
//                       the pad) holds d = 8 (c % 17) .. + 7
//   chunks 544 .. 1183  V^T rows: row d = c' / 5; chunk c' % 5 (4: the pad)
//                       holds slots 8 (c' % 5) .. + 7
//   chunks 1184 ..      zeros up to the last 1 KB piece
// Keys past L are zeros.
template <int MODE>
__global__ __launch_bounds__(256) void attention_pack_kernel(int L, int H, int Hkv,
                                                             const float *__restrict__ qkv,
                                                             int64_t ldqkv,
                                                             const float *__restrict__ rope,
                                                             uint8_t *__restrict__ img,
                                                             int xcds) {
  const int nblk = (L + KB - 1) / KB;
  int hk, item;  // the kv head's workgroups on the XCD its attention workgroups use
  place_kv(blockIdx.x, Hkv, nblk * 5, xcds, hk, item);
  const int b = item / 5;
  const int im = hk * nblk + b;  // image hk * nblk + b
  const int kcol = (H + hk) * AD, vcol = (H + Hkv + hk) * AD;
  const int c = threadIdx.x + 256 * (item - 5 * b);
  _Float16 hv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) hv[e] = (_Float16)0.0f;
  if (c < 544) {
    const int k = c / 17, part = c - 17 * (c / 17), key = b * KB + k;
    if (part < 16 && key < L) {
      const float *row = qkv + (int64_t)key * ldqkv + kcol;
      const int d0 = 8 * part;
      float x[8];
      {
        const float4 lo = *reinterpret_cast<const float4 *>(row + d0);
        const float4 hi = *reinterpret_cast<const float4 *>(row + d0 + 4);
        x[0] = lo.x, x[1] = lo.y, x[2] = lo.z, x[3] = lo.w;
        x[4] = hi.x, x[5] = hi.y, x[6] = hi.z, x[7] = hi.w;
      }
      if (MODE == 1) {  // NORM: pairs (2i, 2i+1) inside the chunk
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float2 cs =
              *reinterpret_cast<const float2 *>(rope + ((int64_t)key * 64 + (d0 + e) / 2) * 2);
          rope_pair(x[e], x[e + 1], cs.x, cs.y, x[e], x[e + 1]);
        }
      } else if (MODE == 2) {  // NEOX: pairs (i, i + 64), the partner from the other half
        const bool low = d0 < 64;
        const int i0 = low ? d0 : d0 - 64;
        const float *prow = row + (low ? d0 + 64 : d0 - 64);
        const float4 plo = *reinterpret_cast<const float4 *>(prow);
        const float4 phi = *reinterpret_cast<const float4 *>(prow + 4);
        const float other[8] = {plo.x, plo.y, plo.z, plo.w, phi.x, phi.y, phi.z, phi.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 cs = *reinterpret_cast<const float2 *>(rope + ((int64_t)key * 64 + i0 + e) * 2);
          float ra, rb;
          if (low)
            rope_pair(x[e], other[e], cs.x, cs.y, ra, rb);
          else
            rope_pair(other[e], x[e], cs.x, cs.y, rb, ra);
          x[e] = ra;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = (_Float16)x[e];
    }
  } else if (c < 1184) {
    const int cv = c - 544, d = cv / 5, part = cv - 5 * (cv / 5);
    if (part < 4) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = b * KB + slot_key(8 * part + e);
        if (key < L) hv[e] = (_Float16)qkv[(int64_t)key * ldqkv + vcol + d];
      }
    }
  }
  *reinterpret_cast<f16x8 *>(img + (int64_t)im * IMG_BYTES + 16 * c) =
      f16x8{hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]};
}

// ---------------------------------------------------------------------------
// Buffer-to-LDS copies: M0 holds the LDS byte address, lane l writes its 16
// bytes at M0 + offset + 16 l, and the immediate offset moves the global
// address too; a write of M0 needs one wait state before a load that uses it.
// The loads are inline assembly with explicit waits, since the compiler
// cannot tell the ring's slots apart.
constexpr int DESC_FLAGS = 0x00020000;
typedef __attribute__((address_space(3))) void *lds_ptr_t;

__device__ inline i32x4 desc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, DESC_FLAGS};
}

template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// N (1, 2 or 4) consecutive 1 KB pieces: global soff + vo + 1024 p to LDS
// lds + 1024 p (+ 16 lane on both sides), p = 0 .. N-1.
template <int N>
__device__ inline void dma_pieces(const i32x4 &d, uint32_t lds, int soff, uint32_t vo) {
  static_assert(N == 1 || N == 2 || N == 4, "pieces per M0 value");
  if (N == 4)
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:3072 lds" ::"s"(lds),
        "v"(vo), "s"(d), "s"(soff)
        : "memory");
  else if (N == 2)
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:1024 lds" ::"s"(lds),
        "v"(vo), "s"(d), "s"(soff)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds),
        "v"(vo), "s"(d), "s"(soff)
        : "memory");
}

// This wave's share (20 / QW pieces of 1 KB) of one block image into a slot.
template <int QW>
__device__ inline void dma_share(const i32x4 &d, uint32_t slot, int img_off, int wave, int lane) {
  constexpr int P = IMG_BYTES / 1024 / QW;
  static_assert(P * QW * 1024 == IMG_BYTES, "image split");
  static_assert(P == 10 || P == 5, "piece groups");
  const int base = wave * P * 1024;
  const uint32_t vo = (uint32_t)(16 * lane + base);
  dma_pieces<4>(d, slot + base, img_off, vo);
  if (P == 10) {
    dma_pieces<4>(d, slot + base + 4096, img_off, vo + 4096);
    dma_pieces<2>(d, slot + base + 8192, img_off, vo + 8192);
  } else {
    dma_pieces<1>(d, slot + base + 4096, img_off, vo + 4096);
  }
}

template <int MODE, int QW>
__global__ __launch_bounds__(64 * QW) void attention_kernel(int L, int H, int Hkv,
                                                            const float *__restrict__ qkv,
                                                            int64_t ldqkv,
                                                            const float *__restrict__ rope,
                                                            const uint8_t *__restrict__ img,
                                                            float *__restrict__ out, int64_t ldo,
                                                            int out_vec, int xcds) {
  constexpr int LPW = IMG_BYTES / 1024 / QW;  // loads per wave per block
  constexpr int RING = ring_slots(QW);
  // the first RING - 1 copies, then Q's 8 + 16 loads (rows and RoPE table)
  static_assert((RING - 1) * LPW + 24 < 64, "loads in flight");
  static_assert(RING * IMG_BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[RING * IMG_BYTES];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, g = lane >> 4;
  const int qblocks = (L + 16 * QW - 1) / (16 * QW);
  const int G = H / Hkv;
  int hk, item;  // kv head, and (query head in its group, query block)
  place_kv(blockIdx.x, Hkv, G * qblocks, xcds, hk, item);
  const int h = hk * G + item / qblocks;
  const int q0 = (item % qblocks) * 16 * QW + 16 * wave;
  const int nblk = (L + KB - 1) / KB;

  // the kv head's images, block b at b * IMG_BYTES (blocks past the last
  // repeat it: those slots are never read)
  const i32x4 dimg = desc(img + (int64_t)hk * nblk * IMG_BYTES, (uint32_t)(nblk * IMG_BYTES));
  const uint32_t ring = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
  auto issue = [&](int blk, int slot) {
    blk = blk < nblk ? blk : nblk - 1;
    dma_share<QW>(dimg, ring + slot * IMG_BYTES, blk * IMG_BYTES, wave, lane);
  };

#pragma unroll
  for (int s = 0; s < RING - 1; ++s) issue(s, s);

  // this lane's query (rows past L repeat the last one; they are not stored)
  const int q = q0 + col < L ? q0 + col : L - 1;
  // Q^T operand: d = 32c + 8g + e (e = 0..7), rotated in registers
  f16x8 qf[4];
  load_q<MODE>(qkv + (int64_t)q * ldqkv + h * AD, MODE ? rope + (int64_t)q * 128 : rope, g, qf);

  // the last slot's copy once Q is in registers (the copies of the first
  // RING - 1 blocks were issued before Q's loads, so both latencies overlap
  // and at most (RING - 1) * LPW + 24 loads are ever in flight)
  wait_vm<0>();
  issue(RING - 1, RING - 1);

  float m = -INFINITY, lsum = 0.0f;
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{};

  for (int b = 0; b < nblk; ++b) {
    // loads issued after block b's: blocks b + 1 .. b + RING - 2 (at b = 0 up
    // to b + RING - 1, so the first wait only waits longer)
    wait_vm<(RING - 2) * LPW>();
    __syncthreads();  // every wave's share of block b has landed
    // every wave is past block b - 1: refill its slot
    if (b > 0) issue(b - 1 + RING, (b - 1) % RING);
    const uint8_t *buf = lds + (b % RING) * IMG_BYTES;
    const _Float16 *kl = reinterpret_cast<const _Float16 *>(buf);
    const _Float16 *vt = reinterpret_cast<const _Float16 *>(buf + K_BYTES);
    attend_block(kl, vt, qf, b * KB, L, col, g, m, lsum, o);
  }
  wait_vm<0>();  // no LDS write may land after the workgroup ends
  if (q0 + col < L) store_out(lsum, o, out + (int64_t)(q0 + col) * ldo + h * AD + 4 * g, out_vec);
}

template <int MODE>
hipError_t launch_mode(int64_t L, int64_t H, int64_t Hkv, const float *qkv, int64_t ldqkv,
                       const float *rope, uint8_t *img, float *out, int64_t ldo,
                       hipStream_t stream) {
  const int64_t nblk = (L + KB - 1) / KB;
  const int xcds = device_props().xcds;
  hipLaunchKernelGGL((attention_pack_kernel<MODE>), dim3((unsigned)(Hkv * nblk * 5)), dim3(256),
                     0, stream, (int)L, (int)H, (int)Hkv, qkv, ldqkv, rope, img, xcds);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int out_vec = (reinterpret_cast<uintptr_t>(out) % 16 == 0) && (ldo % 4 == 0);
  // 32 queries per workgroup; 64 once that still gives a workgroup to half the
  // CUs (measured: Dream-7B's 224 four-wave workgroups beat its 448 two-wave
  // ones by 6%, LLaDA-8B's 96 would lose to its 160)
  if (H * ((L + 63) / 64) >= device_props().cus / 2) {
    hipLaunchKernelGGL((attention_kernel<MODE, 4>), dim3((unsigned)(H * ((L + 63) / 64))),
                       dim3(256), 0, stream, (int)L, (int)H, (int)Hkv, qkv, ldqkv, rope, img, out,
                       ldo, out_vec, xcds);
  } else {
    hipLaunchKernelGGL((attention_kernel<MODE, 2>), dim3((unsigned)(H * ((L + 31) / 32))),
                       dim3(128), 0, stream, (int)L, (int)H, (int)Hkv, qkv, ldqkv, rope, img, out,
                       ldo, out_vec, xcds);
  }
  return hipGetLastError();
}

}  // namespace

int64_t attention_workspace_bytes(int64_t L, int64_t Hkv) {
  return Hkv * ((L + KB - 1) / KB) * (int64_t)IMG_BYTES;
}

hipError_t launch_attention(int64_t L, int64_t H, int64_t Hkv, const float *qkv, int64_t ldqkv,
                            const float *rope, int rope_mode, uint8_t *ws, float *out,
                            int64_t ldo, hipStream_t stream) {
  if (rope_mode == 1) return launch_mode<1>(L, H, Hkv, qkv, ldqkv, rope, ws, out, ldo, stream);
  if (rope_mode == 2) return launch_mode<2>(L, H, Hkv, qkv, ldqkv, rope, ws, out, ldo, stream);
  return launch_mode<0>(L, H, Hkv, qkv, ldqkv, rope, ws, out, ldo, stream);
}

}  // namespace dq
