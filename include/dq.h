/*
 * dq.h -- C ABI of libdq: GGUF K-quant weight x int8 activation GEMM on
 * AMD Instinct MI355X (gfx950).
 *
 * The workload: a diffusion LLM (LLaDA, Dream) run from GGUF files reruns
 * every Q/K/V/O, gate/up and down projection over the whole canvas of L
 * tokens on each denoising step, and runs the output projection only on the
 * canvas rows the sampler may commit (heatdrop.ai "vladimirrott/mojo-dllm"
 * card, "What it does" and "The interesting bit"; mojo-dllm "Architecture"
 * page, "A forward pass").  This library is that GEMM and nothing else.
 *
 * Conventions shared by every entry point
 *   - Every data pointer is DEVICE memory owned by the caller.  The library
 *     allocates nothing and is safe to call from several host threads.  Its
 *     only state: a per-device cache of the compute-unit and XCD counts the
 *     launchers size their grids by (queried on the first call on a device),
 *     and the device address of dq_qgemm_rows_noalloc's built-in array.
 *   - Every call only validates its arguments on the host and enqueues work on
 *     `stream`; it returns before the work runs.  Results are visible after
 *     the caller synchronizes the stream.
 *   - Shapes: K is the reduction length and must be a positive multiple of
 *     256 (one K-quant super-block).  M (activation rows) and N (weight rows)
 *     may be any value >= 0; M == 0 or N == 0 is a valid no-op.
 *   - Return value: DQ_OK or one of the DQ_E* codes below.  A call that
 *     returns DQ_EINVAL, DQ_EUNSUPPORTED or DQ_EWORKSPACE has enqueued
 *     nothing (every argument is checked before the first launch).  DQ_EHIP
 *     means the HIP runtime refused a launch; in a call that makes several
 *     launches (dq_qgemm_rows, dq_qgemm_rows_sample, dq_logits_stats,
 *     dq_attention, dq_debug_subdots) the launches before the refused one may already be
 *     enqueued and may have written the workspace, the flags or the output.
 *     dq_last_error() gives a message for the last error raised on the
 *     calling host thread.
 *   - Types: weights are GGUF tensors of type DQ_Q4_K or DQ_Q6_K (the GGUF
 *     type ids).  A 2-D GGUF weight of shape N x K is N rows, each of K/256
 *     consecutive super-blocks (144 bytes for Q4_K, 210 bytes for Q6_K).
 */
#ifndef DQ_H
#define DQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* GGUF tensor type ids of the supported weight blocks. */
enum { DQ_Q4_K = 12, DQ_Q6_K = 14 };

/* Status codes. */
enum {
  DQ_OK = 0,
  DQ_EINVAL = 1,       /* bad shape, leading dimension, alignment or NULL pointer */
  DQ_EUNSUPPORTED = 2, /* unknown weight type */
  DQ_EWORKSPACE = 3,   /* workspace pointer NULL or smaller than required */
  DQ_EHIP = 4          /* the HIP runtime refused a launch */
};

/* Human-readable name of a status code (static string). */
const char *dq_status_string(int status);

/* Message describing the last error returned on this host thread ("" if none). */
const char *dq_last_error(void);

/* --------------------------------------------------------------------------
 * dq_packed_size -- bytes of the repacked matrix (host-only, no GPU work).
 *
 * Source (of this and the other size queries, dq_act_size and the
 * *_workspace calls): Architecture page, "A forward pass" (the forward pass
 * allocates nothing; every buffer is sized once, up front, for the longest
 * canvas) and the aiboss88 news page, licence and limits (when free VRAM is
 * short the program reports the VRAM it needs and exits): the caller learns
 * every size before it allocates, and the library never allocates.
 *
 * The repacked layout holds the same bits as the GGUF blocks (4.5 bits per
 * Q4_K weight, 6.5625 bits per Q6_K weight), permuted into tiles of 16 weight
 * rows x one super-block; N is rounded up to a multiple of 16 with zero rows.
 * bytes = ceil(N/16) * 16 * (K/256) * block_bytes.
 * Errors: DQ_EUNSUPPORTED (type), DQ_EINVAL (K, N < 0, bytes NULL).
 * ------------------------------------------------------------------------ */
int dq_packed_size(int type, int64_t N, int64_t K, size_t *bytes);

/* --------------------------------------------------------------------------
 * dq_repack_weights -- load-time permutation of GGUF K-quant blocks into the
 * gfx950 tile layout used by dq_qgemm / dq_qgemm_rows.
 *
 * Source: the pages' load-time repack (heatdrop.ai card, "The interesting
 * bit"; Architecture page, "Memory": every projection matrix is repacked once
 * at load and stays resident; Q4_K stays 4-bit).  Here it is a lossless
 * permutation at the same bit-width (Q6_K is not expanded).
 *
 *   gguf   : device, N*(K/256) blocks, row-major as in the GGUF file; read only.
 *   packed : device, dq_packed_size() bytes, 16-byte aligned; written fully
 *            (padding rows are zero).  Must not overlap gguf.
 * Errors: DQ_EUNSUPPORTED, DQ_EINVAL (shape, NULL, alignment), DQ_EHIP.
 * ------------------------------------------------------------------------ */
int dq_repack_weights(int type, int64_t N, int64_t K, const void *gguf, void *packed,
                      hipStream_t stream);

/* --------------------------------------------------------------------------
 * Quantized activations.  dq_quantize_act writes, and dq_qgemm /
 * dq_debug_superblock_sums read, one device buffer of dq_act_size(M, K)
 * bytes laid out for the GEMM's loads: rows are grouped in blocks of 16
 * (MB = ceil(M/16) blocks; rows M .. 16*MB-1 are all-zero padding) and each
 * (super-block b, row block mb) pair is one record of DQ_ACT_RECORD bytes at
 * byte offset (b*MB + mb) * DQ_ACT_RECORD:
 *   [0, 4096)     codes (int8).  Row r (0..15) of the block holds the 256
 *                 codes of super-block b as 16 units of 16 bytes; unit u is
 *                 stored at r*256 + 16*(u XOR r).
 *   [4096, 4608)  code sums.  For row r and 32-wide group j (0..7) of the
 *                 super-block, at 4096 + r*32 + j*4: the sum s of the group's
 *                 32 codes as two IEEE binary16 values (lo, hi) with
 *                 lo = s AND 63 (two's complement) and hi = s - lo; both are
 *                 exact, and s = lo + hi.
 *   [4608, 4672)  d_x of rows 0..15 (binary32).
 *   [4672, 5120)  zero.
 * ------------------------------------------------------------------------ */
#define DQ_ACT_RECORD 5120

/* Bytes of the quantized-activation buffer for M rows of length K (host-only).
 * Source: as for dq_packed_size (sizes known before any allocation).
 * Errors: DQ_EINVAL (K, M < 0, bytes NULL, size beyond 2^32). */
int dq_act_size(int64_t M, int64_t K, size_t *bytes);

/* --------------------------------------------------------------------------
 * dq_quantize_act -- f32 activations -> int8 codes, one f32 scale per 256.
 *
 * Source: Architecture page, "Source map" (kernels/qgemm.mojo): activation
 * quantization, int8 with one scale per 256 values; "A forward pass", step 2:
 * one quantization feeds several projections (Q, K, V; gate and up).
 * Rule, per row m and 256-block b, all in IEEE binary32:
 *   amax = max |x|; if amax == 0: d = 0 and every code is 0;
 *   else inv = 127/amax (correctly rounded), q = clamp(rint(x*inv), -127, 127)
 *   with ties to even, d = amax/127.
 *   code sums per 32 consecutive values (int32, stored as described above).
 * The codes, scales and sums are bit-identical to any binary32 implementation
 * of these steps.  Inputs must be finite; amax below 127/FLT_MAX is out of
 * domain.
 *
 *   x  : device f32, M rows, row stride ldx >= K floats; read only.
 *   qa : device buffer of dq_act_size(M, K) bytes, 16-byte aligned; written
 *        fully (padding rows and the zero tail of each record included).
 * Errors: DQ_EINVAL (shape, ldx < K, NULL, alignment), DQ_EHIP.
 * ------------------------------------------------------------------------ */
int dq_quantize_act(int64_t M, int64_t K, const float *x, int64_t ldx, void *qa,
                    hipStream_t stream);

/* --------------------------------------------------------------------------
 * dq_swiglu_quantize_act -- the down projection's input, silu(gate) * up,
 * quantized as dq_quantize_act does, in one pass.
 *
 * Source: Architecture page, "A forward pass", step 2 (the FFN applies SiLU
 * to gate, multiplies by up and quantizes again for down); "Source map"
 * (SwiGLU among the GPU kernels).  Per element, all in IEEE binary32 with no
 * contraction:  x = (g / (1 + e)) * u,  e = exp(-g) computed as: clamp t to
 * [-87, 88]; n = rint(t * 1.44269502f); r = (t - n*0.693145751953125f)
 * - n*1.42860677e-06f; p = the degree-7 Taylor polynomial of e^r with
 * coefficients 1/k! rounded to binary32, by Horner from 1/7!; e = p * 2^n.
 * Then x is quantized by the dq_quantize_act rule; codes, scales and sums are
 * bit-identical to any binary32 implementation of these steps.  Inputs must
 * be finite.
 *
 *   gu : device f32, M rows of [gate (F values) | up (F values)], row stride
 *        ldgu >= 2F floats (the output of a stacked gate/up GEMM); read only.
 *   qa : device buffer of dq_act_size(M, F) bytes, 16-byte aligned; written
 *        fully, in the layout above.
 * Errors: DQ_EINVAL (F % 256, ldgu < 2F, NULL, alignment), DQ_EHIP.
 * ------------------------------------------------------------------------ */
int dq_swiglu_quantize_act(int64_t M, int64_t F, const float *gu, int64_t ldgu, void *qa,
                           hipStream_t stream);

/* --------------------------------------------------------------------------
 * dq_rmsnorm_quantize_act -- RMSNorm of each row, then the quantizer, in one
 * pass (the input of Q/K/V and of gate/up).
 *
 * Source: Architecture page, "A forward pass", step 2 (RMSNorm, then one
 * int8 quantization reused by Q, K and V); "Source map" (RMSNorm among the
 * GPU kernels).  Per row, IEEE binary32 with no contraction, the sum of
 * squares ss is formed block by block (256 values): in each block, the values
 * 4l .. 4l+3 give the lane sum s[l] = ((x0*x0 + x1*x1) + x2*x2) + x3*x3 (l =
 * 0..63); the block sum is the pairwise tree of six levels s[i] = s[2i] +
 * s[2i+1]; ss adds the block sums in increasing block order.  mean = ss / K;
 * rinv = 1 / sqrt(mean + eps) (both correctly rounded); y = (x * rinv) *
 * gamma.  Then y is quantized by the dq_quantize_act rule, bit-identical to
 * any binary32 implementation of these steps.  Inputs must be finite.
 *
 *   K     : a multiple of 256, at most 262144.
 *   x     : device f32, M rows, row stride ldx >= K floats; read only.
 *   gamma : device f32, K weights; read only.
 *   eps   : finite, >= 0.
 *   qa    : device buffer of dq_act_size(M, K) bytes, 16-byte aligned.
 * Errors: DQ_EINVAL (K, ldx < K, eps, NULL, alignment), DQ_EHIP.
 * ------------------------------------------------------------------------ */
int dq_rmsnorm_quantize_act(int64_t M, int64_t K, const float *x, int64_t ldx,
                            const float *gamma, float eps, void *qa, hipStream_t stream);

/* --------------------------------------------------------------------------
 * dq_qgemm -- y[m][n] = sum_k w^[n][k] * x^[m][k] for int8 activations and a
 * repacked K-quant weight matrix.
 *
 * Source: Architecture page, "Source map" (kernels/packed.mojo: the GEMM used
 * for every projection; gpu/kernels.mojo: an int8 matrix-core GEMM over Q4_K /
 * Q6_K blocks).  x^ = d[m][k/256] * q[m][k];  w^ = d*sc_j*q - dmin*m_j (Q4_K,
 * 32-wide sub-blocks) or d*sc_j*(q-32) (Q6_K, 16-wide sub-blocks).  The kernel
 * forms, for every (m, n, super-block b), the exact integer
 *   S = sum_j sc_j * dot_j  (dot_j = int32 dot of the codes of sub-block j)
 *   Mn = sum_j m_j * bsum_j (Q4_K only)
 * on int8 matrix cores and folds y += d_x*(d*S - dmin*Mn) in binary32.
 * |y - y_exact| stays far below 1e-4 * sum_k |w^ x^|.
 *
 *   qa     : the output of dq_quantize_act for these M rows and this K.
 *   packed : output of dq_repack_weights for (type, N, K).
 *   y      : device f32, M rows, row stride ldy >= N; columns [0, N) of
 *            each row are written, nothing else.
 * Errors: DQ_EUNSUPPORTED, DQ_EINVAL (shape, ldy < N, NULL, alignment), DQ_EHIP.
 * ------------------------------------------------------------------------ */
int dq_qgemm(int type, int64_t M, int64_t N, int64_t K, const void *qa, const void *packed,
             float *y, int64_t ldy, hipStream_t stream);

/* --------------------------------------------------------------------------
 * dq_qgemm_swiglu -- the stacked gate/up GEMM with the down projection's
 * input formed in its epilogue: h[m][i] = silu(g[m][i]) * u[m][i], where g
 * and u are the gate and up outputs, so the 2F-wide GEMM output is never
 * stored.
 *
 * Source: Architecture page, "A forward pass", step 2 (gate and up read one
 * quantized input; the FFN applies SiLU to gate and multiplies by up before
 * down's quantization) and "Source map" (SwiGLU among the GPU kernels).
 * The weight matrix is the 2F x K stack of gate and up with its 16-row tiles
 * interleaved: rows 32i .. 32i+15 are gate rows 16i .. 16i+15 and rows
 * 32i+16 .. 32i+31 are up rows 16i .. 16i+15 (the caller orders the GGUF rows
 * so before dq_repack_weights; a load-time layout choice).  g and u are the
 * f32 values dq_qgemm computes on that matrix, bit for bit, and
 * silu(g) * u = (g / (1 + exp(-g))) * u follows dq_swiglu_quantize_act's
 * binary32 steps exactly.  So dq_quantize_act(h) gives the codes, scales
 * and sums that dq_swiglu_quantize_act gives on dq_qgemm's output rearranged
 * to [gate | up].
 *
 *   qa     : the output of dq_quantize_act (or a fused producer) for M rows, K.
 *   packed : output of dq_repack_weights for (type, 2F, K), tiles interleaved
 *            as above.
 *   F      : the FFN width, a multiple of 16.
 *   h      : device f32, M rows, row stride ldh >= F; columns [0, F) of each
 *            row are written, nothing else.
 * Errors: DQ_EUNSUPPORTED, DQ_EINVAL (F % 16, shape, ldh < F, NULL,
 *         alignment), DQ_EHIP.
 * ------------------------------------------------------------------------ */
int dq_qgemm_swiglu(int type, int64_t M, int64_t F, int64_t K, const void *qa,
                    const void *packed, float *h, int64_t ldh, hipStream_t stream);

/* --------------------------------------------------------------------------
 * dq_qgemm_rows_workspace -- workspace bytes dq_qgemm_rows needs for M
 * gathered rows of length K (host-only): the index flags, then the quantized
 * activations of the gathered rows.
 * Source: as for dq_packed_size (sizes known before any allocation).
 * ------------------------------------------------------------------------ */
int dq_qgemm_rows_workspace(int64_t M, int64_t K, size_t *bytes);

/* --------------------------------------------------------------------------
 * dq_qgemm_rows -- output projection on the requested canvas rows only.
 *
 * Source: Architecture page, "A forward pass": the caller gives a canvas of L
 * tokens and the list of positions whose logits it needs; the final
 * projection runs on those rows only (heatdrop.ai card, "The interesting
 * bit": logits only for positions the sampler can commit).
 * Output row i is canvas row idx[i] quantized by the dq_quantize_act rule and
 * multiplied by the weights exactly as dq_qgemm does.
 *
 *   canvas : device f32, L rows, row stride ldc >= K floats; read only.
 *   idx    : device int32 [M], values in [0, L); any order; duplicates allowed.
 *            An index outside [0, L) is never dereferenced: its row is taken
 *            as zeros and int32 word i of the workspace's flag array (the
 *            first 4*M bytes of ws) is set to 1 (0 for valid rows).
 *   packed : output of dq_repack_weights for (type, N, K).
 *   y      : device f32, M rows, row stride ldy >= N.
 *   ws     : device workspace of at least dq_qgemm_rows_workspace(M, K) bytes,
 *            256-byte aligned; its contents are overwritten.
 * Errors: DQ_EUNSUPPORTED, DQ_EINVAL (shape, NULL, alignment),
 *         DQ_EWORKSPACE (ws NULL or ws_bytes too small), DQ_EHIP.
 * ------------------------------------------------------------------------ */
int dq_qgemm_rows(int type, int64_t L, int64_t M, int64_t N, int64_t K, const float *canvas,
                  int64_t ldc, const int32_t *idx, const void *packed, float *y, int64_t ldy,
                  void *ws, size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------
 * dq_qgemm_rows_noalloc -- dq_qgemm_rows without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The call itself
 * allocates nothing: the gathered rows' quantized activations (and, when
 * flags is NULL, the index flags) go to a device array built into the library,
 * DQ_NOALLOC_SCRATCH_BYTES bytes, one copy per GPU, held from the first call
 * on that GPU until the process ends.  Its device address is looked up on the
 * first call on each device (with that device current).
 *   Arguments and results as for dq_qgemm_rows, except:
 *   flags  : optional device int32 [M], 4-byte aligned: flags[i] = 1 if idx[i]
 *            is outside [0, L), else 0.  NULL keeps them in the array.
 *   stream : must belong to the current device (else DQ_EINVAL).
 * Limits: 256 * ceil(M*4/256) (without flags) + ceil(M/16) * (K/256) * 5120
 * bytes must fit in DQ_NOALLOC_SCRATCH_BYTES (e.g. M <= 64 at K <= 51200, or
 * M <= 256 at K <= 12800); larger calls return DQ_EWORKSPACE and enqueue
 * nothing.  Every call on a GPU shares that GPU's array: calls that overlap in
 * time on one GPU (different streams, or host threads without ordering) race
 * and give undefined results.  Each call overwrites the parts it uses before
 * reading them, so nothing needs clearing between calls.
 * Errors: as dq_qgemm_rows; DQ_EWORKSPACE for sizes beyond the array.
 * ------------------------------------------------------------------------ */
#define DQ_NOALLOC_SCRATCH_BYTES 4194304u
int dq_qgemm_rows_noalloc(int type, int64_t L, int64_t M, int64_t N, int64_t K,
                          const float *canvas, int64_t ldc, const int32_t *idx,
                          const void *packed, float *y, int64_t ldy, int32_t *flags,
                          hipStream_t stream);

/* --------------------------------------------------------------------------
 * Sampler statistics of requested rows of logits.
 *
 * Source: heatdrop.ai card, "The interesting bit" (the output projection
 * computes logits only for the positions the sampler can commit) and the
 * aiboss88 news page's capability list (each model's own sampler: LLaDA's
 * low-confidence remasking, Dream's entropy ordering).  What the samplers
 * read from a row is reduced on the device, so the M x N logits need not be
 * kept.  With z[n] = beta * y[n] (binary32; beta is the inverse temperature):
 *   token[i]        = the smallest n with z[n] = max z   (greedy prediction)
 *   stats[4*i + 0]  = max z
 *   stats[4*i + 1]  = log sum_n exp z[n]                 (log-partition)
 *   stats[4*i + 2]  = -sum_n p[n] log p[n], p = softmax(z)  (entropy)
 *   stats[4*i + 3]  = p[token[i]]                        (its confidence)
 * token and max are exact functions of z; the three sums are binary32 with a
 * relative error of a few 1e-6.  Logits must be finite and |z| < 3e38 (out
 * of that domain the results are unspecified).
 *
 * dq_logits_stats_workspace / dq_logits_stats -- the statistics of the M rows
 * of an f32 logits matrix y (row stride ldy >= N floats).
 *   beta  : finite, > 0.
 *   token : device int32 [M];  stats : device f32 [M x 4], 4-byte aligned.
 *   ws    : device workspace of at least dq_logits_stats_workspace(M, N)
 *           bytes, 16-byte aligned; its contents are overwritten.
 * Errors: DQ_EINVAL (M < 0, N < 1, ldy < N, beta, NULL, alignment, too many
 *         rows for one launch), DQ_EWORKSPACE, DQ_EHIP.
 * ------------------------------------------------------------------------ */
int dq_logits_stats_workspace(int64_t M, int64_t N, size_t *bytes);
int dq_logits_stats(int64_t M, int64_t N, const float *y, int64_t ldy, float beta,
                    int32_t *token, float *stats, void *ws, size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------
 * dq_qgemm_rows_sample_workspace / dq_qgemm_rows_sample -- the output
 * projection on the requested canvas rows (as dq_qgemm_rows) with the sampler
 * statistics above computed in the GEMM's epilogue: the logits are reduced
 * where they are formed and never written to memory.  The logits reduced are
 * bit-identical to the y that dq_qgemm_rows writes for the same arguments
 * when that call's row stride ldy is at most 2^25 floats (dq_qgemm_rows takes
 * another kernel, with another summation order, for longer rows).
 *   canvas, ldc, idx, packed : as for dq_qgemm_rows (idx flags likewise in the
 *           first 4*M bytes of ws).
 *   beta, token, stats       : as for dq_logits_stats.
 *   ws    : at least dq_qgemm_rows_sample_workspace(M, N, K) bytes, 256-byte
 *           aligned; its contents are overwritten.
 * Errors: DQ_EUNSUPPORTED, DQ_EINVAL (shape, beta, NULL, alignment),
 *         DQ_EWORKSPACE, DQ_EHIP.
 * ------------------------------------------------------------------------ */
int dq_qgemm_rows_sample_workspace(int64_t M, int64_t N, int64_t K, size_t *bytes);
int dq_qgemm_rows_sample(int type, int64_t L, int64_t M, int64_t N, int64_t K,
                         const float *canvas, int64_t ldc, const int32_t *idx, const void *packed,
                         float beta, int32_t *token, float *stats, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* --------------------------------------------------------------------------
 * dq_attention_workspace / dq_attention -- bidirectional attention of every
 * canvas position over all L positions.
 *
 * Source: Architecture page, "A forward pass", step 2 (RoPE rotates Q and K;
 * attention runs over all L positions with no mask) and "Source map" (NORM
 * and NEOX RoPE, bidirectional attention); aiboss88 news page, capability
 * list (attention on f16 tensor cores, 16 queries per warp, keys streamed
 * through shared memory with an online softmax).  For position l and head h
 * (kv head g = h / (H / Hkv)):
 *   q = RoPE(Q[l, h]), k_j = RoPE(K[j, g]) at positions l and j, rounded to
 *   binary16; v_j = V[j, g] rounded to binary16;
 *   out[l][h*D + d] = sum_j p_j v_j[d] / sum_j p_j,
 *   p_j = exp(q . k_j / sqrt(D) - max_j q . k_j / sqrt(D)),  j = 0 .. L-1.
 * RoPE of the pair (a, b) by (c, s) = rope[pos][i] is a' = fma(a, c, -(b*s)),
 * b' = fma(b, c, a*s) in binary32; pairs are (2i, 2i+1) for rope_mode 1
 * (NORM) and (i, i + D/2) for rope_mode 2 (NEOX); rope_mode 0 rotates nothing.
 * Products accumulate in binary32 and the probabilities enter the second
 * product as binary16, so |out - exact| stays below about 1e-3 of
 * sum_j p_j |v_j[d]| / sum_j p_j.
 *
 *   D     : head dimension; only 128 is built (else DQ_EUNSUPPORTED).
 *   qkv   : device f32, L rows [Q (H*D) | K (Hkv*D) | V (Hkv*D)], row stride
 *           ldqkv >= (H + 2 Hkv) D floats, a multiple of 4; 16-byte aligned
 *           (the Q/K/V projection's output as dq_qgemm writes it).
 *   rope  : device f32 [L][D/2][2] (cos, sin) of each position's angles,
 *           8-byte aligned; ignored (may be NULL) for rope_mode 0.
 *   out   : device f32, L rows of H*D, row stride ldo >= H D; only those
 *           columns are written.
 *   ws    : device workspace of at least dq_attention_workspace(L, H, Hkv, D)
 *           bytes (Hkv * ceil(L/32) * 20 KB: each kv head's keys and values,
 *           rotated and rounded to binary16, in blocks of 32 keys), 16-byte
 *           aligned; its contents are overwritten.
 * Errors: DQ_EUNSUPPORTED (D), DQ_EINVAL (shapes, H % Hkv, rope_mode, strides,
 *         NULL, alignment), DQ_EWORKSPACE, DQ_EHIP.
 * ------------------------------------------------------------------------ */
int dq_attention_workspace(int64_t L, int64_t H, int64_t Hkv, int64_t D, size_t *bytes);
int dq_attention(int64_t L, int64_t H, int64_t Hkv, int64_t D, const float *qkv, int64_t ldqkv,
                 const float *rope, int rope_mode, float *out, int64_t ldo, void *ws,
                 size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------
 * dq_row_bytes / dq_embed_rows -- embedding rows: the rows of a GGUF table
 * selected by token id, decoded to f32.
 *
 * Source: Architecture page, "A forward pass", step 1 (embedding rows are
 * decoded from the memory-mapped Q4_K table, one row per token) and "Source
 * map" (scalar F32 / F16 / BF16 / Q8_0 / Q4_K / Q5_K / Q6_K decoders).  The
 * table is N rows of dq_row_bytes(type, K) bytes in the public GGUF block
 * layouts, as stored in the file (not repacked).  Types (GGUF ids): F32 0,
 * F16 1, Q8_0 8 (34-byte blocks of 32: fp16 d, int8 q; w = d q), Q4_K 12,
 * Q5_K 13 (176-byte blocks: d, dmin, the Q4_K 6-bit scales, qh[32] fifth
 * bits, qs[128] nibbles; w = d sc q - dmin m), Q6_K 14, BF16 30.  Every value
 * is the correctly rounded binary32 of its definition (exact for all but Q4_K
 * and Q5_K, whose d sc q - dmin m is rounded once).
 *
 *   K     : values per row, a positive multiple of 256.
 *   table : device bytes, 16-byte aligned; read only.
 *   ids   : device int32 [M]; ids outside [0, N) give a row of zeros and,
 *           when flags is not NULL, flags[i] = 1 (0 for valid ids).
 *   out   : device f32, M rows of K, row stride ldo >= K.
 * Errors: DQ_EUNSUPPORTED (type), DQ_EINVAL (K, shapes, ldo, NULL,
 *         alignment), DQ_EHIP.
 * ------------------------------------------------------------------------ */
int dq_row_bytes(int type, int64_t K, size_t *bytes);
int dq_embed_rows(int type, int64_t N, int64_t K, const void *table, const int32_t *ids,
                  int64_t M, float *out, int64_t ldo, int32_t *flags, hipStream_t stream);

/* --------------------------------------------------------------------------
 * dq_debug_superblock_sums -- test hook.  Runs the dq_qgemm kernel with its
 * fold replaced by stores of the exact per-super-block integers, so that the
 * integer part of the production code path can be compared bit for bit:
 *   S[(m*N + n)*(K/256) + b]  = sum_j sc_j * dot_j
 *   Mn[(m*N + n)*(K/256) + b] = sum_j m_j * bsum_j   (Q4_K; 0 for Q6_K)
 * With every scale but sub-block j's set to 0 (and that one to 1) S equals
 * the sub-block dot dot_j, which is how per-sub-block dots are checked.
 * qa is a dq_quantize_act buffer (its d_x values are not used).  S and Mn are
 * device int32 arrays of M*N*(K/256) entries.
 * ------------------------------------------------------------------------ */
int dq_debug_superblock_sums(int type, int64_t M, int64_t N, int64_t K, const void *qa,
                             const void *packed, int32_t *S, int32_t *Mn, hipStream_t stream);

/* --------------------------------------------------------------------------
 * dq_debug_subdots -- test hook for the per-sub-block int32 dots.  Runs the
 * dq_qgemm kernel (the one the launcher picks for this shape) once per
 * sub-block position j, with the digit builder given scale 1 for sub-block j
 * and 0 for the others in place of the weights' scales, and stores the exact
 * integer S of each step, which is then that sub-block's dot:
 *   dots[((m*N + n)*(K/256) + b)*J + j] = sum over sub-block j of super-block b
 *                                          of q_w * q_x
 * with J = 8 sub-blocks of 32 for Q4_K (q_w in [0, 15]) and J = 16 of 16 for
 * Q6_K (q_w - 32 in [-32, 31]).  Unpack, operand layout and MFMA accumulation
 * are the production path's; only the scale bytes and the epilogue differ.
 * qa is a dq_quantize_act buffer (its d_x values are not used); dots is a
 * device int32 array of M*N*(K/256)*J entries.  J launches on the stream.
 * Errors: DQ_EUNSUPPORTED, DQ_EINVAL (shape, NULL, alignment, more than 2^40
 *         entries), DQ_EHIP.
 * ------------------------------------------------------------------------ */
int dq_debug_subdots(int type, int64_t M, int64_t N, int64_t K, const void *qa,
                     const void *packed, int32_t *dots, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DQ_H */
