// attention.h -- private to libdq: the launcher of the canvas attention kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dq {

constexpr int ATTN_HEAD_DIM = 128;  // the one head dimension the kernel is built for

// Bytes of the f16 key/value block images (the workspace).
int64_t attention_workspace_bytes(int64_t L, int64_t Hkv);

// qkv: L rows [Q (H*128) | K (Hkv*128) | V (Hkv*128)] f32, row stride ldqkv;
// rope: L x 64 x (cos, sin) f32 for rope_mode 1 (NORM) and 2 (NEOX), unused for 0;
// ws: attention_workspace_bytes(L, Hkv) bytes, 16-byte aligned;
// out: L rows of H*128 f32, row stride ldo.
hipError_t launch_attention(int64_t L, int64_t H, int64_t Hkv, const float *qkv, int64_t ldqkv,
                            const float *rope, int rope_mode, uint8_t *ws, float *out,
                            int64_t ldo, hipStream_t stream);

}  // namespace dq
