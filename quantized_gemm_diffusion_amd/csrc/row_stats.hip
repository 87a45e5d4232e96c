// row_stats.hip -- what the samplers read from each requested row of logits:
// the greedy token, the maximum, the log-partition, the entropy and the top
// probability of softmax(beta * logits) (heatdrop.ai card, "The interesting
// bit": logits are computed only for the positions the sampler can commit;
// aiboss88 news page, capability list: LLaDA remasks its lowest-confidence
// predictions, Dream orders positions by entropy).
//
// Both kernels are bound by what they read: the partial kernel streams the
// logits once (4 bytes per logit), the finish kernel reads 16 bytes per
// partial state.  The state algebra is in row_stats.h.
#include "dq_internal.h"
#include "row_stats.h"

namespace dq {
namespace {

constexpr int RS_THREADS = 256;
constexpr int RS_CHUNK = 4096;  // columns per partial of the standalone reduction

// Reduce the block's states into thread 0's: an xor tree inside each wave,
// then wave 0 .. 3's results merged in order.  Every thread must call it.
__device__ inline RowStat block_merge(RowStat st, float4 *lds) {
  for (int mask = 32; mask >= 1; mask >>= 1) st = stat_merge(st, stat_shfl_xor(st, mask));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) lds[wave] = stat_pack(st);
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < RS_THREADS / 64; ++w) st = stat_merge(st, stat_unpack(lds[w]));
  return st;
}

// Workgroup r * npart + c computes partial c of row r, over the columns
// c * RS_CHUNK .. min(N, (c + 1) * RS_CHUNK) - 1; thread t takes the RS_G groups
// of 4 columns that start 4 * (t + 256 g) columns into the chunk, all loaded
// before any is folded (RS_G loads in flight per thread).
constexpr int RS_G = RS_CHUNK / (4 * RS_THREADS);

template <bool VEC>
__global__ __launch_bounds__(RS_THREADS) void logits_stats_partial_kernel(
    int64_t N, const float *__restrict__ y, int64_t ldy, float beta, int npart,
    float4 *__restrict__ part) {
  __shared__ float4 lds[RS_THREADS / 64];
  const int64_t r = blockIdx.x / npart;
  const int c = (int)(blockIdx.x - r * npart);
  const float *yr = y + r * ldy;
  const int64_t lo = (int64_t)c * RS_CHUNK;
  const int64_t hi = lo + RS_CHUNK < N ? lo + RS_CHUNK : N;
  float v[RS_G][4];
  int cnt[RS_G];
#pragma unroll
  for (int g = 0; g < RS_G; ++g) {
    const int64_t n0 = lo + 4 * (threadIdx.x + RS_THREADS * g);
    const int64_t left = hi - n0;
    cnt[g] = left <= 0 ? 0 : left > 4 ? 4 : (int)left;
    if (VEC && cnt[g] == 4) {
      const float4 q = *reinterpret_cast<const float4 *>(yr + n0);
      v[g][0] = q.x, v[g][1] = q.y, v[g][2] = q.z, v[g][3] = q.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[g][i] = i < cnt[g] ? yr[n0 + i] : 0.0f;
    }
  }
  RowStat st = stat_empty();
#pragma unroll
  for (int g = 0; g < RS_G; ++g) {
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = beta * v[g][i];
    stat_push4(st, z, (int)(lo + 4 * (threadIdx.x + RS_THREADS * g)), cnt[g]);
  }
  st = block_merge(st, lds);
  if (threadIdx.x == 0) part[r * npart + c] = stat_pack(st);
}

// One workgroup per row: thread t merges partials t, t + 256, ... in order,
// then the block merge.
__global__ __launch_bounds__(RS_THREADS) void row_stats_finish_kernel(
    int npart, const float4 *__restrict__ part, int32_t *__restrict__ token,
    float *__restrict__ stats) {
  __shared__ float4 lds[RS_THREADS / 64];
  const int64_t r = blockIdx.x;
  RowStat st = stat_empty();
  for (int p = threadIdx.x; p < npart; p += RS_THREADS)
    st = stat_merge(st, stat_unpack(part[r * npart + p]));
  st = block_merge(st, lds);
  if (threadIdx.x == 0) {
    const float ls = logf(st.s);
    token[r] = st.i;
    stats[4 * r + 0] = st.m;
    stats[4 * r + 1] = st.m + ls;
    stats[4 * r + 2] = ls - st.a / st.s;
    stats[4 * r + 3] = 1.0f / st.s;
  }
}

}  // namespace

int logits_stats_parts(int64_t N) { return (int)((N + RS_CHUNK - 1) / RS_CHUNK); }

hipError_t launch_logits_stats_partial(int64_t M, int64_t N, const float *y, int64_t ldy,
                                       float beta, int npart, float4 *part, hipStream_t stream) {
  dim3 grid((unsigned)(npart * M)), block(RS_THREADS);
  const bool vec = reinterpret_cast<uintptr_t>(y) % 16 == 0 && ldy % 4 == 0;
  if (vec)
    hipLaunchKernelGGL(logits_stats_partial_kernel<true>, grid, block, 0, stream, N, y, ldy, beta,
                       npart, part);
  else
    hipLaunchKernelGGL(logits_stats_partial_kernel<false>, grid, block, 0, stream, N, y, ldy,
                       beta, npart, part);
  return hipGetLastError();
}

hipError_t launch_row_stats_finish(int64_t M, int npart, const float4 *part, int32_t *token,
                                   float *stats, hipStream_t stream) {
  hipLaunchKernelGGL(row_stats_finish_kernel, dim3((unsigned)M), dim3(RS_THREADS), 0, stream,
                     npart, part, token, stats);
  return hipGetLastError();
}

}  // namespace dq
