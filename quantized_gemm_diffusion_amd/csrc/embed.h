// embed.h -- private to libdq: the embedding-row decoder's launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dq {

// Bytes of one row of K values of a GGUF type (F32 0, F16 1, Q8_0 8, Q4_K 12,
// Q5_K 13, Q6_K 14, BF16 30); 0 for another type or K not a positive multiple
// of 256.
int64_t embed_row_bytes(int type, int64_t K);

// out[i] (row stride ldo) = row ids[i] of the N x K table decoded to f32;
// flag[i] (if flag) = 1 where ids[i] is outside [0, N) (then the row is 0).
hipError_t launch_embed_rows(int type, int64_t N, int64_t K, const uint8_t *table,
                             const int32_t *ids, int64_t M, float *out, int64_t ldo,
                             int32_t *flag, hipStream_t stream);

}  // namespace dq
