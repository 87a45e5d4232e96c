// row_stats.h -- private to libdq: the per-row reduction of logits that the
// samplers read (greedy token, maximum, log-partition, entropy), kept as a
// running state that any set of columns can be folded into, in any grouping.
//
// A state over a set of columns with values z (z = beta * logit, binary32):
//   m = max z, i = smallest column attaining m,
//   s = sum exp(z - m)             (s >= 1 once a column is in; 0 = empty),
//   a = sum exp(z - m) * (z - m)   (<= 0).
// Two states merge exactly as the sums over the union (the one with the
// smaller maximum is rescaled by exp(m_lo - m_hi)); from the final state
//   log-partition = m + log s,  entropy = log s - a / s,  top probability = 1 / s.
// Partial states travel through memory as a float4 {m, bits of i, s, a}.
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

namespace dq {

struct RowStat {
  float m;
  int i;
  float s;
  float a;
};

__device__ inline RowStat stat_empty() { return RowStat{-INFINITY, INT_MAX, 0.0f, 0.0f}; }

// Fold up to 4 consecutive columns n0 .. n0 + cnt - 1 with values z[0 .. cnt-1]
// into st; columns must arrive in increasing order across calls on one state
// (a later column never displaces an equal maximum).
__device__ inline void stat_push4(RowStat &st, const float z[4], int n0, int cnt) {
  float lm = -INFINITY;
  int li = INT_MAX;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (c < cnt && z[c] > lm) {
      lm = z[c];
      li = n0 + c;
    }
  if (lm > st.m) {
    // the sums so far were taken relative to the old maximum
    if (st.s > 0.0f) {
      const float d = st.m - lm;
      const float r = __expf(d);
      st.a = r * (st.a + d * st.s);
      st.s = r * st.s;
    }
    st.m = lm;
    st.i = li;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (c < cnt) {
      const float t = z[c] - st.m;
      const float e = __expf(t);
      st.s += e;
      st.a += e * t;
    }
}

// Union of two states.  The result does not depend on the argument order.
// (Field-wise selects, no branches: both states stay in registers.)
__device__ inline RowStat stat_merge(const RowStat &x, const RowStat &y) {
  // an empty state never becomes the high one, and its rescaled sums are 0
  const bool y_hi = x.s == 0.0f || (y.s != 0.0f && (y.m > x.m || (y.m == x.m && y.i < x.i)));
  const float hm = y_hi ? y.m : x.m, hs = y_hi ? y.s : x.s, ha = y_hi ? y.a : x.a;
  const float lm = y_hi ? x.m : y.m, ls = y_hi ? x.s : y.s, la = y_hi ? x.a : y.a;
  const int hi = y_hi ? y.i : x.i;
  if (ls == 0.0f) return RowStat{hm, hi, hs, ha};
  const float d = lm - hm;
  const float r = __expf(d);
  return RowStat{hm, hi, hs + r * ls, ha + r * (la + d * ls)};
}

__device__ inline RowStat stat_shfl_xor(const RowStat &x, int mask) {
  return RowStat{__shfl_xor(x.m, mask), __shfl_xor(x.i, mask), __shfl_xor(x.s, mask),
                 __shfl_xor(x.a, mask)};
}

__device__ inline float4 stat_pack(const RowStat &x) {
  return make_float4(x.m, __int_as_float(x.i), x.s, x.a);
}

__device__ inline RowStat stat_unpack(const float4 &v) {
  return RowStat{v.x, __float_as_int(v.y), v.z, v.w};
}

// Launchers (each returns the hipError_t of its last launch).
// Partial states of M rows of an f32 logits matrix, npart per row (row r's
// partials at part[r * npart ...]), columns cut into npart equal chunks.
int logits_stats_parts(int64_t N);
hipError_t launch_logits_stats_partial(int64_t M, int64_t N, const float *y, int64_t ldy,
                                       float beta, int npart, float4 *part, hipStream_t stream);
// Merge the npart partials of each row in a fixed order and write token[r]
// and stats[4r .. 4r+3] = {max, log-partition, entropy, top probability}.
hipError_t launch_row_stats_finish(int64_t M, int npart, const float4 *part, int32_t *token,
                                   float *stats, hipStream_t stream);
// The gathered-row GEMM whose epilogue folds each output row into partial
// states instead of storing it; qgemm_stats_parts gives their count per row.
int qgemm_stats_parts(int64_t M, int64_t N, int64_t K);
// Single-row Q6_K projection with the gather-quantize in the GEMM launch (see
// qgemm.hip); false (nothing launched) where it does not apply.
bool launch_rows_gather_row1(int type, int64_t M, int64_t N, int64_t K, const float *canvas,
                             int64_t ldc, const int32_t *idx, int64_t L, int32_t *flags,
                             const uint8_t *packed, float *y, float beta, float4 *part,
                             hipStream_t stream, hipError_t &err);
hipError_t launch_qgemm_stats(int type, int64_t M, int64_t N, int64_t K, const uint8_t *qa,
                              const uint8_t *packed, float beta, float4 *part, int npart,
                              hipStream_t stream);

}  // namespace dq
