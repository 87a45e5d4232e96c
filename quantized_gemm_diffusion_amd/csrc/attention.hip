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
// One wave takes 16 queries of one head; a workgroup of QW waves takes 16 QW
// consecutive queries of that head and streams the head's keys in blocks of
// 32 through LDS (double buffered, one barrier per block): the workgroup's
// threads load a block's K and V rows (f32), rotate K, round both to f16 and
// write K row-major and V transposed.  Per block a wave runs
//   S^T (32 keys x 16 queries) = K Q^T : 2 tiles x 4 v_mfma_f32_16x16x32_f16
//   O^T (128 d x 16 queries) += V^T P^T : 8 tiles x 1 v_mfma_f32_16x16x32_f16
// Transposing both products puts one query in each lane (column l % 16 of
// every accumulator), so the softmax state of a query (running max, the
// rescale factor) is a per-lane value shared by the 4 lanes l % 16 + 16g: the
// block maximum takes two cross-lane steps and the output rescale none.
// P^T leaves the S^T accumulators in exactly the B-operand layout of the
// second product once the keys of its contraction are ordered as the lanes
// hold them (key 16t + 4g + i at contraction slot 8g + 4t + i); V^T is written
// to LDS in that key order.
#include "attention.h"

#include "dq_internal.h"

namespace dq {
namespace {

constexpr int AD = 128;          // head dimension
constexpr int KB = 32;           // keys per block
constexpr int K_LD = AD + 8;     // K rows in LDS, halves (272 B: conflict-free 16-B reads)
constexpr int VT_LD = KB + 8;    // V^T rows in LDS, halves (80 B)
constexpr int K_BYTES = KB * K_LD * 2;
constexpr int VT_BYTES = AD * VT_LD * 2;
constexpr int BUF_BYTES = K_BYTES + VT_BYTES;

// RoPE of one pair (a, b) by (c, s): a' = fma(a, c, -(b*s)), b' = fma(b, c, a*s),
// every step rounded in binary32 (no further contraction).
__device__ inline void rope_pair(float a, float b, float c, float s, float &ra, float &rb) {
  const float bs = __fmul_rn(b, s);
  const float as = __fmul_rn(a, s);
  ra = __fmaf_rn(a, c, -bs);
  rb = __fmaf_rn(b, c, as);
}

// Contraction slot of key k (0..31) of a block in the second product.
__device__ inline int key_slot(int k) { return 8 * ((k & 15) >> 2) + 4 * (k >> 4) + (k & 3); }

// The workgroup's share of one key block: 32 keys x 64 pairs of K and 32 x 64
// pairs of V per thread group.  Items per thread: 2048 / threads of each.
template <int MODE, int T>
struct BlockRegs {
  static constexpr int N = KB * (AD / 2) / T;  // pairs of K (and of V) per thread
  float ka[N], kb[N], va[N], vb[N];
};

// Item u of the block (u = thread + T * n): key u / 64, pair u % 64.  K pair:
// NORM (2p, 2p+1), NEOX (p, p+64), none (2p, 2p+1); V pair (2p, 2p+1).  Keys
// past L load row L - 1 (valid memory) and keep zeros.
template <int MODE, int T>
__device__ inline void load_block(BlockRegs<MODE, T> &r, const float *__restrict__ qkv,
                                  int64_t ldqkv, int L, int kcol, int vcol,
                                  const float *__restrict__ rope, int kb0) {
#pragma unroll
  for (int n = 0; n < BlockRegs<MODE, T>::N; ++n) {
    const int u = threadIdx.x + T * n;
    const int key = kb0 + (u >> 6), p = u & 63;
    const bool ok = key < L;
    const int kc = ok ? key : L - 1;
    const float *row = qkv + (int64_t)kc * ldqkv;
    const int ia = MODE == 2 ? p : 2 * p, ib = MODE == 2 ? p + 64 : 2 * p + 1;
    float a = row[kcol + ia], b = row[kcol + ib];
    if (MODE != 0) {
      const float2 cs = *reinterpret_cast<const float2 *>(rope + ((int64_t)kc * 64 + p) * 2);
      rope_pair(a, b, cs.x, cs.y, a, b);
    }
    const float2 v = *reinterpret_cast<const float2 *>(row + vcol + 2 * p);
    r.ka[n] = ok ? a : 0.0f;
    r.kb[n] = ok ? b : 0.0f;
    r.va[n] = ok ? v.x : 0.0f;
    r.vb[n] = ok ? v.y : 0.0f;
  }
}

template <int MODE, int T>
__device__ inline void store_block(const BlockRegs<MODE, T> &r, uint8_t *buf) {
  _Float16 *kl = reinterpret_cast<_Float16 *>(buf);
  _Float16 *vt = reinterpret_cast<_Float16 *>(buf + K_BYTES);
#pragma unroll
  for (int n = 0; n < BlockRegs<MODE, T>::N; ++n) {
    const int u = threadIdx.x + T * n;
    const int k = u >> 6, p = u & 63;
    const int ia = MODE == 2 ? p : 2 * p, ib = MODE == 2 ? p + 64 : 2 * p + 1;
    kl[k * K_LD + ia] = (_Float16)r.ka[n];
    kl[k * K_LD + ib] = (_Float16)r.kb[n];
    const int slot = key_slot(k);
    vt[(2 * p) * VT_LD + slot] = (_Float16)r.va[n];
    vt[(2 * p + 1) * VT_LD + slot] = (_Float16)r.vb[n];
  }
}

template <int MODE, int QW>
__global__ __launch_bounds__(64 * QW) void attention_kernel(int L, int H, int Hkv,
                                                            const float *__restrict__ qkv,
                                                            int64_t ldqkv,
                                                            const float *__restrict__ rope,
                                                            float *__restrict__ out, int64_t ldo,
                                                            int out_vec) {
  constexpr int T = 64 * QW;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BUF_BYTES];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, g = lane >> 4;
  const int qblocks = (L + 16 * QW - 1) / (16 * QW);
  const int h = blockIdx.x / qblocks;
  const int q0 = (blockIdx.x - h * qblocks) * 16 * QW + 16 * wave;
  const int hk = h / (H / Hkv);
  const int kcol = (H + hk) * AD, vcol = (H + Hkv + hk) * AD;

  // this lane's query (rows past L repeat the last one; they are not stored)
  const int q = q0 + col < L ? q0 + col : L - 1;
  // Q^T operand: d = 32c + 8g + e (e = 0..7), rotated in registers
  f16x8 qf[4];
  {
    const float *row = qkv + (int64_t)q * ldqkv + h * AD;
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
          const float2 cs = *reinterpret_cast<const float2 *>(rope + ((int64_t)q * 64 + i) * 2);
          rope_pair(x[c][e], x[c][e + 1], cs.x, cs.y, x[c][e], x[c][e + 1]);
        }
    } else if (MODE == 2) {  // NEOX: pairs (i, i + 64): chunk c with chunk c + 2
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 32 * c + 8 * g + e;
          const float2 cs = *reinterpret_cast<const float2 *>(rope + ((int64_t)q * 64 + i) * 2);
          rope_pair(x[c][e], x[c + 2][e], cs.x, cs.y, x[c][e], x[c + 2][e]);
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[c][e] = (_Float16)x[c][e];
  }

  // log2(e) / sqrt(128): scores go straight to exp2
  const float sc = 1.4426950408889634f * 0.08838834764831845f;
  float m = -INFINITY, lsum = 0.0f;
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{};

  const int nblk = (L + KB - 1) / KB;
  BlockRegs<MODE, T> r;
  load_block<MODE, T>(r, qkv, ldqkv, L, kcol, vcol, rope, 0);
  store_block<MODE, T>(r, lds);
  for (int b = 0; b < nblk; ++b) {
    __syncthreads();  // block b is in its buffer; the other buffer is free
    const bool more = b + 1 < nblk;
    if (more) load_block<MODE, T>(r, qkv, ldqkv, L, kcol, vcol, rope, (b + 1) * KB);
    const uint8_t *buf = lds + (b & 1) * BUF_BYTES;
    const _Float16 *kl = reinterpret_cast<const _Float16 *>(buf);
    const _Float16 *vt = reinterpret_cast<const _Float16 *>(buf + K_BYTES);

    // S^T: lane holds query col, keys 16t + 4g + i
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
    // online softmax over the block
    const int kb0 = b * KB;
    float bm = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = s[t][i] * sc;
        if (kb0 + 16 * t + 4 * g + i >= L) v = -INFINITY;
        s[t][i] = v;
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
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[t][i] - mn);
        ps += p;
        pf[4 * t + i] = (_Float16)p;
      }
    lsum = lsum * alpha + ps;
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      o[dt] *= alpha;
      const f16x8 va = *reinterpret_cast<const f16x8 *>(vt + (16 * dt + col) * VT_LD + 8 * g);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pf, o[dt], 0, 0, 0);
    }
    if (more) store_block<MODE, T>(r, lds + ((b + 1) & 1) * BUF_BYTES);
  }

  // the 4 lanes of a query hold partial sums over their keys
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  const float inv = 1.0f / lsum;
  if (q0 + col >= L) return;
  float *orow = out + (int64_t)(q0 + col) * ldo + h * AD + 4 * g;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const f32x4 v = o[dt] * inv;
    if (out_vec) {
      *reinterpret_cast<f32x4 *>(orow + 16 * dt) = v;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) orow[16 * dt + i] = v[i];
    }
  }
}

template <int MODE>
hipError_t launch_mode(int64_t L, int64_t H, int64_t Hkv, const float *qkv, int64_t ldqkv,
                       const float *rope, float *out, int64_t ldo, hipStream_t stream) {
  const int out_vec = (reinterpret_cast<uintptr_t>(out) % 16 == 0) && (ldo % 4 == 0);
  // 4 waves (64 queries) per workgroup once that still gives a workgroup per CU
  const bool wide = H * ((L + 63) / 64) >= 256;
  if (wide) {
    const unsigned grid = (unsigned)(H * ((L + 63) / 64));
    hipLaunchKernelGGL((attention_kernel<MODE, 4>), dim3(grid), dim3(256), 0, stream, (int)L,
                       (int)H, (int)Hkv, qkv, ldqkv, rope, out, ldo, out_vec);
  } else {
    const unsigned grid = (unsigned)(H * ((L + 31) / 32));
    hipLaunchKernelGGL((attention_kernel<MODE, 2>), dim3(grid), dim3(128), 0, stream, (int)L,
                       (int)H, (int)Hkv, qkv, ldqkv, rope, out, ldo, out_vec);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(int64_t L, int64_t H, int64_t Hkv, const float *qkv, int64_t ldqkv,
                            const float *rope, int rope_mode, float *out, int64_t ldo,
                            hipStream_t stream) {
  if (rope_mode == 1) return launch_mode<1>(L, H, Hkv, qkv, ldqkv, rope, out, ldo, stream);
  if (rope_mode == 2) return launch_mode<2>(L, H, Hkv, qkv, ldqkv, rope, out, ldo, stream);
  return launch_mode<0>(L, H, Hkv, qkv, ldqkv, rope, out, ldo, stream);
}

}  // namespace dq
