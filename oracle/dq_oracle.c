/*
 * dq_oracle.c -- plain, slow, scalar CPU oracle for the K-quant x int8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or table with the HIP
 * library: every rule below is written out again from its definition.
 *
 * What it computes (sources named per function):
 *   - mojo-dllm "Architecture" page, "Source map": the scalar K-quant decoders
 *     are the test oracle; activations are quantized to int8 with one scale
 *     per 256 values; a row-major reference GEMM sits beside the packed one.
 *   - same page, "A forward pass", step 2: one quantization of the activations
 *     feeds several projections.
 *   - heatdrop.ai "vladimirrott/mojo-dllm" card, "Key highlights": the decoder
 *     and GEMM are checked against a dequantize-then-multiply reference.
 *   - The pages name the GGUF Q4_K and Q6_K block types but do not spell out
 *     their bytes.  The layouts below follow the public GGUF/ggml K-quant
 *     block definitions (super-block of 256 weights; Q4_K = 144 bytes with
 *     6-bit scales/mins, Q6_K = 210 bytes with int8 scales).
 *
 * Precision rules: decoding and the integer sub-block dots are exact.  The
 * activation quantizer uses IEEE binary32 for every step (one correctly
 * rounded division 127/amax, one multiply, round-half-to-even, clamp), so the
 * integer codes it produces are the ones any binary32 implementation of the
 * same steps produces.  The reference GEMM output is formed in binary64 from
 * fully dequantized weights and activations (the plain definition); a second
 * routine forms the same output in binary32 through the integer decomposition.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK 256 /* weights per super-block */
#define Q4K_BYTES 144
#define Q6K_BYTES 210
#define TYPE_Q4K 12 /* GGUF tensor type id of Q4_K */
#define TYPE_Q6K 14 /* GGUF tensor type id of Q6_K */

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 -> binary32 (exact: every half value is a float value). */
/* sign | 5-bit exponent (bias 15) | 10-bit fraction; exponent 0 is the      */
/* subnormal range f * 2^-24, exponent 31 is Inf/NaN.                        */
/* ------------------------------------------------------------------------ */
float dqo_fp16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return (float)(sign ? -v : v);
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ------------------------------------------------------------------------ */
/* Q4_K super-block (144 bytes): d (fp16), dmin (fp16), scales[12], qs[128]. */
/* Eight sub-blocks of 32 weights; sub-block j has a 6-bit scale sc[j] and a */
/* 6-bit min mn[j].  j < 4: sc = low 6 bits of scales[j], mn = low 6 bits of */
/* scales[j+4].  j >= 4: low 4 bits from scales[j+4] (sc: low nibble, mn:    */
/* high nibble), high 2 bits from the top 2 bits of scales[j-4] (sc) and of  */
/* scales[j] (mn).  qs byte 32c+l holds weight 64c+l in its low nibble and   */
/* weight 64c+32+l in its high nibble (c = 0..3, l = 0..31).                 */
/* Dequantized weight i (sub-block j = i/32): d*sc[j]*q[i] - dmin*mn[j].     */
/* ------------------------------------------------------------------------ */
void dqo_decode_q4k(const uint8_t *blk, float *d, float *dmin, uint8_t sc[8],
                    uint8_t mn[8], uint8_t q[256]) {
  const uint8_t *s = blk + 4;
  const uint8_t *qs = blk + 16;
  *d = dqo_fp16_to_f32(rd16(blk));
  *dmin = dqo_fp16_to_f32(rd16(blk + 2));
  for (int j = 0; j < 4; ++j) {
    sc[j] = s[j] & 63;
    mn[j] = s[j + 4] & 63;
  }
  for (int j = 4; j < 8; ++j) {
    sc[j] = (uint8_t)((s[j + 4] & 15) | ((s[j - 4] >> 6) << 4));
    mn[j] = (uint8_t)((s[j + 4] >> 4) | ((s[j] >> 6) << 4));
  }
  for (int c = 0; c < 4; ++c)
    for (int l = 0; l < 32; ++l) {
      q[64 * c + l] = qs[32 * c + l] & 15;
      q[64 * c + 32 + l] = qs[32 * c + l] >> 4;
    }
}

/* ------------------------------------------------------------------------ */
/* Q6_K super-block (210 bytes): ql[128], qh[64], scales[16] (int8), d fp16. */
/* Sixteen sub-blocks of 16 weights; weight i uses scales[i/16].  For half   */
/* h = 0,1 and l = 0..31 the 6-bit codes are                                 */
/*   i = 128h+l    : low  nibble of ql[64h+l]    | bits 0-1 of qh[32h+l] <<4 */
/*   i = 128h+32+l : low  nibble of ql[64h+32+l] | bits 2-3 of qh[32h+l] <<4 */
/*   i = 128h+64+l : high nibble of ql[64h+l]    | bits 4-5 of qh[32h+l] <<4 */
/*   i = 128h+96+l : high nibble of ql[64h+32+l] | bits 6-7 of qh[32h+l] <<4 */
/* Dequantized weight: d * scales[i/16] * (q[i] - 32).                       */
/* ------------------------------------------------------------------------ */
void dqo_decode_q6k(const uint8_t *blk, float *d, int8_t sc[16], uint8_t q[256]) {
  const uint8_t *ql = blk;
  const uint8_t *qh = blk + 128;
  for (int j = 0; j < 16; ++j) sc[j] = (int8_t)blk[192 + j];
  *d = dqo_fp16_to_f32(rd16(blk + 208));
  for (int h = 0; h < 2; ++h)
    for (int l = 0; l < 32; ++l) {
      uint8_t hb = qh[32 * h + l];
      q[128 * h + l] = (uint8_t)((ql[64 * h + l] & 15) | (((hb >> 0) & 3) << 4));
      q[128 * h + 32 + l] = (uint8_t)((ql[64 * h + 32 + l] & 15) | (((hb >> 2) & 3) << 4));
      q[128 * h + 64 + l] = (uint8_t)((ql[64 * h + l] >> 4) | (((hb >> 4) & 3) << 4));
      q[128 * h + 96 + l] = (uint8_t)((ql[64 * h + 32 + l] >> 4) | (((hb >> 6) & 3) << 4));
    }
}

static int block_bytes(int type) {
  return type == TYPE_Q4K ? Q4K_BYTES : (type == TYPE_Q6K ? Q6K_BYTES : 0);
}

/* Dequantize one weight row of K values (K/256 consecutive blocks) to f64.  */
/* Every value is exact in binary64 (at most 21 significant bits).           */
int dqo_dequant_row(int type, const uint8_t *row, int64_t K, double *w) {
  int bb = block_bytes(type);
  if (!bb || K % QK) return -1;
  for (int64_t b = 0; b < K / QK; ++b) {
    const uint8_t *blk = row + b * bb;
    double *o = w + b * QK;
    if (type == TYPE_Q4K) {
      float d, dmin;
      uint8_t sc[8], mn[8], q[256];
      dqo_decode_q4k(blk, &d, &dmin, sc, mn, q);
      for (int i = 0; i < QK; ++i)
        o[i] = (double)d * sc[i / 32] * q[i] - (double)dmin * mn[i / 32];
    } else {
      float d;
      int8_t sc[16];
      uint8_t q[256];
      dqo_decode_q6k(blk, &d, sc, q);
      /* the integer sc * (q - 32) first: the same exact value, with the sign */
      /* of a zero product taken from d alone                                 */
      for (int i = 0; i < QK; ++i) o[i] = (double)d * (double)(sc[i / 16] * ((int)q[i] - 32));
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Activation quantization: int8, one scale per 256 values of a row.         */
/* (Architecture page, "Source map", kernels/qgemm.mojo.)  Symmetric absmax: */
/*   amax = max |x| over the 256-block;                                      */
/*   amax == 0  ->  d = 0, q = 0;                                            */
/*   else inv = 127 / amax (binary32, correctly rounded),                    */
/*        q = clamp(rint(x * inv), -127, 127) (binary32 multiply, ties even),*/
/*        d = amax / 127 (binary32).                                         */
/* bsum[m][k/32] = sum of the 32 codes of that group (int32).                */
/* x is M rows with leading dimension ldx (floats); q is M x K (ld K);       */
/* d is M x K/256; bsum is M x K/32.                                         */
/* ------------------------------------------------------------------------ */
int dqo_quantize_act(int64_t M, int64_t K, const float *x, int64_t ldx, int8_t *q,
                     float *d, int32_t *bsum) {
  if (K % QK || ldx < K) return -1;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t b = 0; b < K / QK; ++b) {
      const float *xb = x + m * ldx + b * QK;
      int8_t *qb = q + m * K + b * QK;
      float amax = 0.0f;
      for (int i = 0; i < QK; ++i) {
        float a = fabsf(xb[i]);
        if (a > amax) amax = a;
      }
      if (amax == 0.0f) {
        d[m * (K / QK) + b] = 0.0f;
        for (int i = 0; i < QK; ++i) qb[i] = 0;
      } else {
        float inv = 127.0f / amax;
        for (int i = 0; i < QK; ++i) {
          float v = rintf(xb[i] * inv);
          if (v > 127.0f) v = 127.0f;
          if (v < -127.0f) v = -127.0f;
          qb[i] = (int8_t)v;
        }
        d[m * (K / QK) + b] = amax / 127.0f;
      }
      for (int g = 0; g < QK / 32; ++g) {
        int32_t s = 0;
        for (int i = 0; i < 32; ++i) s += qb[32 * g + i];
        bsum[m * (K / 32) + b * 8 + g] = s;
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* The producers of the GEMM inputs (Architecture page, "A forward pass",    */
/* step 2: RMSNorm, then one int8 quantization for Q, K and V; the FFN       */
/* applies SiLU to gate, multiplies by up, and quantizes again for down;     */
/* "Source map": RMSNorm and SwiGLU among the ops).  The codes must come out */
/* identical on every implementation, so each producer is defined here as a  */
/* fixed sequence of binary32 operations (no contraction), including the     */
/* order of its one reduction and its exponential.                           */
/* ------------------------------------------------------------------------ */

/* exp for SiLU, defined as: clamp t to [-87, 88]; n = rint(t * log2(e));   */
/* r = (t - n*L1) - n*L2 with L1 + L2 = ln 2 split so that n*L1 is exact     */
/* (Cody and Waite's range reduction); p = the degree-7 Taylor polynomial    */
/* of e^r with coefficients 1/k! rounded to binary32, evaluated by Horner;   */
/* result = p * 2^n, with 2^n built from its exponent bits (exact).          */
float dqo_exp_f32(float t) {
  if (t > 88.0f) t = 88.0f;
  if (t < -87.0f) t = -87.0f;
  const float n = rintf(t * 1.44269502f);
  const float r = (t - n * 0.693145751953125f) - n * 1.42860677e-06f;
  float p = 1.98412698e-04f;  /* 1/7! */
  p = p * r + 1.38888889e-03f; /* 1/6! */
  p = p * r + 8.33333377e-03f; /* 1/5! */
  p = p * r + 4.16666679e-02f; /* 1/4! */
  p = p * r + 1.66666672e-01f; /* 1/3! */
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  const int e = (int)n;
  const uint32_t bits = (uint32_t)(e + 127) << 23;
  float scale;
  memcpy(&scale, &bits, sizeof scale);
  return p * scale;
}

/* SwiGLU input of the down projection: silu(g) * u = (g / (1 + exp(-g))) * u */
float dqo_silu_mul(float g, float u) {
  const float e = dqo_exp_f32(-g);
  const float den = 1.0f + e;
  const float s = g / den;
  return s * u;
}

/* gu holds M rows of [gate (F values) | up (F values)], leading dimension  */
/* ldgu >= 2F; the down projection's input x = silu(gate) * up (M x F) is    */
/* quantized by dqo_quantize_act.                                            */
int dqo_swiglu_quantize_act(int64_t M, int64_t F, const float *gu, int64_t ldgu, int8_t *q,
                            float *d, int32_t *bsum) {
  if (F % QK || ldgu < 2 * F) return -1;
  float *x = (float *)malloc(sizeof(float) * (size_t)(M * F > 0 ? M * F : 1));
  if (!x) return -2;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < F; ++k) x[m * F + k] = dqo_silu_mul(gu[m * ldgu + k], gu[m * ldgu + F + k]);
  int rc = dqo_quantize_act(M, F, x, F, q, d, bsum);
  free(x);
  return rc;
}

/* RMSNorm of one row, then the quantizer.  The sum of squares is formed in  */
/* a fixed order, block by block (256 values each):                          */
/*   lane sum: for l = 0..63, s[l] = ((x0*x0 + x1*x1) + x2*x2) + x3*x3 over  */
/*     the block's values 4l .. 4l+3, one square and one addition at a time; */
/*   block sum: a pairwise tree over the 64 lane sums, six levels of         */
/*     s[i] = s[2i] + s[2i+1];                                               */
/*   ss: the block sums added in increasing block order, starting from      */
/*     block 0's.                                                            */
/* Then mean = ss / K;  rinv = 1 / sqrt(mean + eps)  (both correctly         */
/* rounded);  y[k] = (x[k] * rinv) * gamma[k].                               */
int dqo_rmsnorm_quantize_act(int64_t M, int64_t K, const float *x, int64_t ldx,
                             const float *gamma, float eps, int8_t *q, float *d,
                             int32_t *bsum) {
  if (K % QK || ldx < K) return -1;
  float *y = (float *)malloc(sizeof(float) * (size_t)(M * K > 0 ? M * K : 1));
  if (!y) return -2;
  for (int64_t m = 0; m < M; ++m) {
    const float *xr = x + m * ldx;
    float ss = 0.0f;
    for (int64_t b = 0; b < K / QK; ++b) {
      float s[64];
      for (int l = 0; l < 64; ++l) {
        const float *v = xr + b * QK + 4 * l;
        float t = v[0] * v[0];
        for (int i = 1; i < 4; ++i) {
          const float sq = v[i] * v[i];
          t = t + sq;
        }
        s[l] = t;
      }
      for (int n = 32; n >= 1; n /= 2)
        for (int i = 0; i < n; ++i) s[i] = s[2 * i] + s[2 * i + 1];
      ss = b == 0 ? s[0] : ss + s[0];
    }
    const float mean = ss / (float)K;
    const float rinv = 1.0f / sqrtf(mean + eps);
    for (int64_t k = 0; k < K; ++k) {
      const float t = xr[k] * rinv;
      y[m * K + k] = t * gamma[k];
    }
  }
  int rc = dqo_quantize_act(M, K, y, K, q, d, bsum);
  free(y);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Per-sub-block integer dots.  For activation row m, weight row n,          */
/* super-block b and sub-block j:                                            */
/*   Q4_K (J = 8, width 32):  dot = sum q_w * q_x        (q_w in [0,15])     */
/*   Q6_K (J = 16, width 16): dot = sum (q_w - 32) * q_x (q_w in [0,63])     */
/* out[((m*N + n)*(K/256) + b)*J + j], rows n in [n0, n1) only.              */
/* ------------------------------------------------------------------------ */
int dqo_subdots(int type, int64_t M, int64_t N, int64_t K, const int8_t *qx,
                const uint8_t *W, int64_t n0, int64_t n1, int32_t *out) {
  int bb = block_bytes(type);
  if (!bb || K % QK) return -1;
  int64_t nb = K / QK;
  int J = type == TYPE_Q4K ? 8 : 16, wid = QK / J;
  uint8_t q[256];
  for (int64_t n = n0; n < n1; ++n)
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t *blk = W + (n * nb + b) * bb;
      int off = 0;
      if (type == TYPE_Q4K) {
        float d, dm;
        uint8_t sc[8], mn[8];
        dqo_decode_q4k(blk, &d, &dm, sc, mn, q);
      } else {
        float d;
        int8_t sc[16];
        dqo_decode_q6k(blk, &d, sc, q);
        off = 32;
      }
      for (int64_t m = 0; m < M; ++m) {
        const int8_t *xb = qx + m * K + b * QK;
        for (int j = 0; j < J; ++j) {
          int32_t s = 0;
          for (int i = j * wid; i < (j + 1) * wid; ++i) s += ((int)q[i] - off) * xb[i];
          out[((m * N + n) * nb + b) * J + j] = s;
        }
      }
    }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-super-block integer sums (the combine of the integer decomposition):  */
/*   S[m,n,b]  = sum_j sc_j * dot_j                                          */
/*   Mn[m,n,b] = sum_j mn_j * bsum_j   (Q4_K; 0 for Q6_K)                    */
/* so that the output is y[m,n] = sum_b dx[m,b]*(d[n,b]*S - dmin[n,b]*Mn).   */
/* Layout [m][n][b]; rows n in [n0, n1).                                     */
/* ------------------------------------------------------------------------ */
int dqo_superblock_sums(int type, int64_t M, int64_t N, int64_t K, const int8_t *qx,
                        const int32_t *bsum, const uint8_t *W, int64_t n0, int64_t n1,
                        int32_t *S, int32_t *Mn) {
  int bb = block_bytes(type);
  if (!bb || K % QK) return -1;
  int64_t nb = K / QK;
  int J = type == TYPE_Q4K ? 8 : 16;
  int32_t *dots = (int32_t *)malloc(sizeof(int32_t) * J);
  uint8_t q[256];
  for (int64_t n = n0; n < n1; ++n)
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t *blk = W + (n * nb + b) * bb;
      uint8_t sc4[8], mn4[8];
      int8_t sc6[16];
      float d, dm;
      if (type == TYPE_Q4K)
        dqo_decode_q4k(blk, &d, &dm, sc4, mn4, q);
      else
        dqo_decode_q6k(blk, &d, sc6, q);
      for (int64_t m = 0; m < M; ++m) {
        const int8_t *xb = qx + m * K + b * QK;
        int wid = QK / J, off = type == TYPE_Q4K ? 0 : 32;
        for (int j = 0; j < J; ++j) {
          int32_t s = 0;
          for (int i = j * wid; i < (j + 1) * wid; ++i) s += ((int)q[i] - off) * xb[i];
          dots[j] = s;
        }
        int32_t s_acc = 0, m_acc = 0;
        for (int j = 0; j < J; ++j) {
          if (type == TYPE_Q4K) {
            s_acc += (int32_t)sc4[j] * dots[j];
            m_acc += (int32_t)mn4[j] * bsum[m * (K / 32) + b * 8 + j];
          } else {
            s_acc += (int32_t)sc6[j] * dots[j];
          }
        }
        S[(m * N + n) * nb + b] = s_acc;
        Mn[(m * N + n) * nb + b] = m_acc;
      }
    }
  free(dots);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Reference GEMM, plain definition in binary64:                             */
/*   y[m,n] = sum_k w^[n,k] * x^[m,k],  x^[m,k] = dx[m,k/256] * qx[m,k],     */
/*   T[m,n] = sum_k |w^[n,k] * x^[m,k]|  (the tolerance scale).              */
/* W is N rows of K/256 raw GGUF blocks.  Rows n in [n0, n1); y, T are M x N */
/* row-major (ld N).                                                         */
/* ------------------------------------------------------------------------ */
int dqo_qgemm_ref(int type, int64_t M, int64_t N, int64_t K, const int8_t *qx,
                  const float *dx, const uint8_t *W, int64_t n0, int64_t n1, double *y,
                  double *T) {
  int bb = block_bytes(type);
  if (!bb || K % QK) return -1;
  double *w = (double *)malloc(sizeof(double) * K);
  for (int64_t n = n0; n < n1; ++n) {
    dqo_dequant_row(type, W + n * (K / QK) * bb, K, w);
    for (int64_t m = 0; m < M; ++m) {
      double acc = 0.0, tol = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double xh = (double)dx[m * (K / QK) + k / QK] * qx[m * K + k];
        double p = w[k] * xh;
        acc += p;
        tol += fabs(p);
      }
      y[m * N + n] = acc;
      T[m * N + n] = tol;
    }
  }
  free(w);
  return 0;
}

/* Same as dqo_qgemm_ref for a list of P (m, n) output points.               */
int dqo_qgemm_ref_points(int type, int64_t K, int64_t P, const int64_t *mi, const int64_t *ni,
                         const int8_t *qx, const float *dx, const uint8_t *W, double *y,
                         double *T) {
  int bb = block_bytes(type);
  if (!bb || K % QK) return -1;
  double *w = (double *)malloc(sizeof(double) * K);
  for (int64_t p = 0; p < P; ++p) {
    int64_t m = mi[p], n = ni[p];
    dqo_dequant_row(type, W + n * (K / QK) * bb, K, w);
    double acc = 0.0, tol = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double xh = (double)dx[m * (K / QK) + k / QK] * qx[m * K + k];
      double pr = w[k] * xh;
      acc += pr;
      tol += fabs(pr);
    }
    y[p] = acc;
    T[p] = tol;
  }
  free(w);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* The same output through the integer decomposition, in binary32:           */
/*   for b in order: y += dx[m,b] * (d[n,b]*S[m,n,b] - dmin[n,b]*Mn[m,n,b])  */
/* with S, Mn the exact integers above (Mn = 0 for Q6_K).                    */
/* Rows n in [n0, n1); y is M x N row-major with leading dimension ldy.      */
/* ------------------------------------------------------------------------ */
int dqo_qgemm_f32(int type, int64_t M, int64_t N, int64_t K, const int8_t *qx,
                  const float *dx, const int32_t *bsum, const uint8_t *W, int64_t n0,
                  int64_t n1, float *y, int64_t ldy) {
  int bb = block_bytes(type);
  if (!bb || K % QK) return -1;
  int64_t nb = K / QK;
  int J = type == TYPE_Q4K ? 8 : 16, wid = QK / J, off = type == TYPE_Q4K ? 0 : 32;
  uint8_t *q = (uint8_t *)malloc((size_t)nb * QK);
  uint8_t *sc4 = (uint8_t *)malloc((size_t)nb * 8), *mn4 = (uint8_t *)malloc((size_t)nb * 8);
  int8_t *sc6 = (int8_t *)malloc((size_t)nb * 16);
  float *dd = (float *)malloc(sizeof(float) * nb), *dm = (float *)malloc(sizeof(float) * nb);
  for (int64_t n = n0; n < n1; ++n) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t *blk = W + (n * nb + b) * bb;
      if (type == TYPE_Q4K)
        dqo_decode_q4k(blk, &dd[b], &dm[b], sc4 + 8 * b, mn4 + 8 * b, q + QK * b);
      else {
        dqo_decode_q6k(blk, &dd[b], sc6 + 16 * b, q + QK * b);
        dm[b] = 0.0f;
      }
    }
    for (int64_t m = 0; m < M; ++m) {
      float acc = 0.0f;
      for (int64_t b = 0; b < nb; ++b) {
        const int8_t *xb = qx + m * K + b * QK;
        const uint8_t *qb = q + QK * b;
        int32_t s_acc = 0, m_acc = 0;
        for (int j = 0; j < J; ++j) {
          int32_t s = 0;
          for (int i = j * wid; i < (j + 1) * wid; ++i) s += ((int)qb[i] - off) * xb[i];
          if (type == TYPE_Q4K) {
            s_acc += (int32_t)sc4[8 * b + j] * s;
            m_acc += (int32_t)mn4[8 * b + j] * bsum[m * (K / 32) + b * 8 + j];
          } else {
            s_acc += (int32_t)sc6[16 * b + j] * s;
          }
        }
        float t = dd[b] * (float)s_acc - dm[b] * (float)m_acc;
        acc += dx[m * nb + b] * t;
      }
      y[m * ldy + n] = acc;
    }
  }
  free(q);
  free(sc4);
  free(mn4);
  free(sc6);
  free(dd);
  free(dm);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* What the samplers read from the logits of one requested row (heatdrop.ai  */
/* card, "The interesting bit": logits exist only for the positions the      */
/* sampler can commit; aiboss88 news page, capability list: LLaDA remasks    */
/* the lowest-confidence predictions, Dream orders positions by entropy).    */
/* With z[n] = beta * y[n], a binary32 product of the binary32 logit (the    */
/* inverse temperature beta scales the logits before the softmax):           */
/*   token   = the smallest n with z[n] = max z (greedy prediction);         */
/*   zmax    = z[token];                                                     */
/*   lse     = log sum_n exp(z[n])                  (log of the partition);  */
/*   entropy = -sum_n p[n] log p[n],  p[n] = exp(z[n] - lse), where          */
/*             log p[n] = z[n] - lse (so an underflowed p[n] adds nothing);  */
/*   p_top   = exp(zmax - lse)   (the softmax probability of the token: the  */
/*             confidence low-confidence remasking ranks by).                */
/* Everything after the product is binary64, summed in increasing n, with    */
/* the maximum taken out of the exponentials.  y is M rows, leading          */
/* dimension ldy; stats is M x 4 {zmax, lse, entropy, p_top}.                */
/* ------------------------------------------------------------------------ */
int dqo_logits_stats(int64_t M, int64_t N, const double *y, int64_t ldy, float beta,
                     int32_t *token, double *stats) {
  if (N <= 0 || ldy < N) return -1;
  double *z = (double *)malloc(sizeof(double) * (size_t)N);
  if (!z) return -2;
  for (int64_t m = 0; m < M; ++m) {
    const double *yr = y + m * ldy;
    int64_t best = 0;
    for (int64_t n = 0; n < N; ++n) {
      const float zf = beta * (float)yr[n];
      z[n] = (double)zf;
      if (z[n] > z[best]) best = n;
    }
    const double zmax = z[best];
    double part = 0.0;
    for (int64_t n = 0; n < N; ++n) part += exp(z[n] - zmax);
    const double lse = zmax + log(part);
    double h = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double logp = z[n] - lse;
      h -= exp(logp) * logp;
    }
    token[m] = (int32_t)best;
    stats[4 * m + 0] = zmax;
    stats[4 * m + 1] = lse;
    stats[4 * m + 2] = h;
    stats[4 * m + 3] = exp(zmax - lse);
  }
  free(z);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention over the canvas (Architecture page, "A forward pass", step 2:  */
/* RoPE rotates Q and K, then attention runs over all L positions with no    */
/* mask; "Source map": NORM and NEOX RoPE, bidirectional attention; aiboss88 */
/* news page, capability list: attention runs on f16 tensor cores).          */
/* ------------------------------------------------------------------------ */

/* binary32 -> binary16, round to nearest even (the IEEE conversion), as the */
/* 16-bit pattern.  Overflow gives Inf; NaN stays NaN.                       */
uint16_t dqo_f32_to_fp16(float f) {
  uint32_t x;
  memcpy(&x, &f, sizeof x);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u));
  const int e = (int)(ax >> 23) - 127; /* unbiased exponent */
  if (e > 15) return (uint16_t)(sign | 0x7c00u);
  uint32_t mant = (ax & 0x7fffffu) | 0x800000u; /* 24-bit significand (normal inputs) */
  int shift;                                    /* bits dropped from the significand */
  uint32_t hexp;
  if (e >= -14) { /* normal half: keep 11 bits */
    shift = 13;
    hexp = (uint32_t)(e + 15);
  } else { /* subnormal half: value = m * 2^-24 */
    if (ax < 0x33000000u) return (uint16_t)sign; /* below half the smallest subnormal */
    if ((ax >> 23) == 0) return (uint16_t)sign;  /* f32 subnormal: far below */
    shift = 13 + (-14 - e);
    hexp = 0;
  }
  uint32_t kept = mant >> shift;
  const uint32_t rem = mant & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (kept & 1u))) kept += 1u;
  /* kept holds the significand with its leading one (normal) or the       */
  /* subnormal count; a carry out of the significand bumps the exponent    */
  uint32_t h;
  if (hexp == 0)
    h = kept; /* kept == 0x400 becomes the smallest normal, as it should */
  else
    h = ((hexp << 10) + (kept - 0x400u)); /* kept in [0x400, 0x800] */
  if (h >= 0x7c00u) h = 0x7c00u;
  return (uint16_t)(sign | h);
}

static double f16r(float f) { return (double)dqo_fp16_to_f32(dqo_f32_to_fp16(f)); }

/* Rotation of one pair (a, b) by the table's (c, s) = (cos, sin) of the     */
/* position's angle, in binary32 with a fixed operation order:               */
/*   a' = fma(a, c, -(b*s)),  b' = fma(b, c, a*s).                           */
void dqo_rope_pair(float a, float b, float c, float s, float *ra, float *rb) {
  const float bs = b * s;
  const float as = a * s;
  *ra = fmaf(a, c, -bs);
  *rb = fmaf(b, c, as);
}

/* Rotate one head vector x[0..D) at position pos.  mode 1 (NORM) pairs    */
/* (2i, 2i+1), mode 2 (NEOX) pairs (i, i + D/2), i < D/2; mode 0 leaves x.   */
/* rope holds, per position, D/2 pairs (cos, sin) of the angles pos*f_i.     */
static void rope_vec(float *x, int64_t D, int mode, const float *rope, int64_t pos) {
  if (mode == 0) return;
  const int64_t P = D / 2;
  for (int64_t i = 0; i < P; ++i) {
    const float c = rope[(pos * P + i) * 2], s = rope[(pos * P + i) * 2 + 1];
    const int64_t ia = mode == 1 ? 2 * i : i, ib = mode == 1 ? 2 * i + 1 : i + P;
    float ra, rb;
    dqo_rope_pair(x[ia], x[ib], c, s, &ra, &rb);
    x[ia] = ra;
    x[ib] = rb;
  }
}

/* out[l][h*D + d] = sum_j p_j v_j[d] / sum_j p_j with p_j = exp(q.k_j / sqrt(D) */
/* - max), over all L keys j of the kv head h / (H / Hkv) (no mask).  q, k:    */
/* rotated (binary32, rope_vec), then rounded to binary16; v rounded to        */
/* binary16; everything after in binary64.  Row l of qkv holds               */
/* [Q (H*D) | K (Hkv*D) | V (Hkv*D)].  tol (optional, same shape as out)     */
/* receives sum_j p_j |v_j[d]| / sum_j p_j, the scale of the tolerance.      */
int dqo_attention(int64_t L, int64_t H, int64_t Hkv, int64_t D, const float *qkv, int64_t ldqkv,
                  const float *rope, int mode, double *out, int64_t ldo, double *tol) {
  if (L <= 0 || H <= 0 || Hkv <= 0 || H % Hkv || D <= 0 || D % 2 || mode < 0 || mode > 2 ||
      ldqkv < (H + 2 * Hkv) * D || ldo < H * D || (mode && !rope))
    return -1;
  double *kh = (double *)malloc(sizeof(double) * (size_t)(L * Hkv * D));
  double *vh = (double *)malloc(sizeof(double) * (size_t)(L * Hkv * D));
  double *qh = (double *)malloc(sizeof(double) * (size_t)D);
  double *sc = (double *)malloc(sizeof(double) * (size_t)L);
  float *tmp = (float *)malloc(sizeof(float) * (size_t)D);
  if (!kh || !vh || !qh || !sc || !tmp) {
    free(kh), free(vh), free(qh), free(sc), free(tmp);
    return -2;
  }
  for (int64_t l = 0; l < L; ++l)
    for (int64_t g = 0; g < Hkv; ++g) {
      const float *kr = qkv + l * ldqkv + (H + g) * D;
      const float *vr = qkv + l * ldqkv + (H + Hkv + g) * D;
      for (int64_t d = 0; d < D; ++d) tmp[d] = kr[d];
      rope_vec(tmp, D, mode, rope, l);
      for (int64_t d = 0; d < D; ++d) {
        kh[(l * Hkv + g) * D + d] = f16r(tmp[d]);
        vh[(l * Hkv + g) * D + d] = f16r(vr[d]);
      }
    }
  const double inv = 1.0 / sqrt((double)D);
  for (int64_t l = 0; l < L; ++l)
    for (int64_t h = 0; h < H; ++h) {
      const int64_t g = h / (H / Hkv);
      const float *qr = qkv + l * ldqkv + h * D;
      for (int64_t d = 0; d < D; ++d) tmp[d] = qr[d];
      rope_vec(tmp, D, mode, rope, l);
      for (int64_t d = 0; d < D; ++d) qh[d] = f16r(tmp[d]);
      double mx = -INFINITY;
      for (int64_t j = 0; j < L; ++j) {
        double s = 0.0;
        for (int64_t d = 0; d < D; ++d) s += qh[d] * kh[(j * Hkv + g) * D + d];
        sc[j] = s * inv;
        if (sc[j] > mx) mx = sc[j];
      }
      double den = 0.0;
      for (int64_t j = 0; j < L; ++j) {
        sc[j] = exp(sc[j] - mx);
        den += sc[j];
      }
      for (int64_t d = 0; d < D; ++d) {
        double num = 0.0, ab = 0.0;
        for (int64_t j = 0; j < L; ++j) {
          const double v = vh[(j * Hkv + g) * D + d];
          num += sc[j] * v;
          ab += sc[j] * fabs(v);
        }
        out[l * ldo + h * D + d] = num / den;
        if (tol) tol[l * ldo + h * D + d] = ab / den;
      }
    }
  free(kh), free(vh), free(qh), free(sc), free(tmp);
  return 0;
}

/* Elementwise dqo_f32_to_fp16 over n values (for the exhaustive pin). */
void dqo_f32_to_fp16_n(const float *x, uint16_t *h, int64_t n) {
  for (int64_t i = 0; i < n; ++i) h[i] = dqo_f32_to_fp16(x[i]);
}

/* Rotate in place the n_heads head vectors (D values each, consecutive)    */
/* of each of L rows of x (row stride ldx), row l at position l.             */
int dqo_rope_rows(int64_t L, int64_t n_heads, int64_t D, float *x, int64_t ldx, const float *rope,
                  int mode) {
  if (D <= 0 || D % 2 || mode < 0 || mode > 2 || ldx < n_heads * D || (mode && !rope)) return -1;
  for (int64_t l = 0; l < L; ++l)
    for (int64_t h = 0; h < n_heads; ++h) rope_vec(x + l * ldx + h * D, D, mode, rope, l);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* The decoder's other block types (Architecture page, "Source map": scalar  */
/* F32 / F16 / BF16 / Q8_0 / Q4_K / Q5_K / Q6_K decoders, the test oracle and */
/* the embedding rows; "A forward pass", step 1: embedding rows are decoded  */
/* from the memory-mapped Q4_K table, one row per token).  Byte layouts are  */
/* the public GGUF/ggml block definitions (GGUF type ids in parentheses):    */
/*   F32 (0): 4 bytes per value;  F16 (1): IEEE binary16;                    */
/*   BF16 (30): the top 16 bits of a binary32;                               */
/*   Q8_0 (8): 34 bytes per 32 values: d (fp16), q[32] (int8); w = d * q;    */
/*   Q5_K (13): 176 bytes per 256: d, dmin (fp16), scales[12] (the Q4_K       */
/*     6-bit packing), qh[32], qs[128]; chunk c = 0..3 of 64 weights: weight  */
/*     64c + l takes the low nibble of qs[32c + l] and bit 2c of qh[l] as its */
/*     fifth bit, weight 64c + 32 + l the high nibble and bit 2c + 1;         */
/*     w = d * sc_j * q - dmin * m_j with j = i / 32.                        */
/* ------------------------------------------------------------------------ */
#define TYPE_F32 0
#define TYPE_F16 1
#define TYPE_Q8_0 8
#define TYPE_Q5K 13
#define TYPE_BF16 30
#define Q8_0_BYTES 34
#define Q5K_BYTES 176

void dqo_decode_q8_0(const uint8_t *blk, float *d, int8_t q[32]) {
  *d = dqo_fp16_to_f32(rd16(blk));
  for (int i = 0; i < 32; ++i) q[i] = (int8_t)blk[2 + i];
}

void dqo_decode_q5k(const uint8_t *blk, float *d, float *dmin, uint8_t sc[8], uint8_t mn[8],
                    uint8_t q[256]) {
  const uint8_t *s = blk + 4;
  const uint8_t *qh = blk + 16;
  const uint8_t *qs = blk + 48;
  *d = dqo_fp16_to_f32(rd16(blk));
  *dmin = dqo_fp16_to_f32(rd16(blk + 2));
  for (int j = 0; j < 8; ++j) {
    if (j < 4) {
      sc[j] = s[j] & 63;
      mn[j] = s[j + 4] & 63;
    } else {
      sc[j] = (uint8_t)((s[j + 4] & 15) | ((s[j - 4] >> 6) << 4));
      mn[j] = (uint8_t)((s[j + 4] >> 4) | ((s[j] >> 6) << 4));
    }
  }
  for (int c = 0; c < 4; ++c)
    for (int l = 0; l < 32; ++l) {
      q[64 * c + l] = (uint8_t)((qs[32 * c + l] & 15) | (((qh[l] >> (2 * c)) & 1) << 4));
      q[64 * c + 32 + l] = (uint8_t)((qs[32 * c + l] >> 4) | (((qh[l] >> (2 * c + 1)) & 1) << 4));
    }
}

/* Bytes of one row of K values of the type (0 if unknown or K does not fit */
/* its blocks).                                                              */
int64_t dqo_row_bytes(int type, int64_t K) {
  switch (type) {
    case TYPE_F32: return 4 * K;
    case TYPE_F16:
    case TYPE_BF16: return 2 * K;
    case TYPE_Q8_0: return K % 32 ? 0 : K / 32 * Q8_0_BYTES;
    case TYPE_Q4K: return K % QK ? 0 : K / QK * Q4K_BYTES;
    case TYPE_Q5K: return K % QK ? 0 : K / QK * Q5K_BYTES;
    case TYPE_Q6K: return K % QK ? 0 : K / QK * Q6K_BYTES;
    default: return 0;
  }
}

/* One row of any of the types to binary64 values (every one exact).        */
int dqo_decode_row(int type, const uint8_t *row, int64_t K, double *w) {
  if (!dqo_row_bytes(type, K)) return -1;
  if (type == TYPE_Q4K || type == TYPE_Q6K) return dqo_dequant_row(type, row, K, w);
  for (int64_t i = 0; i < K; ++i) {
    if (type == TYPE_F32) {
      float f;
      memcpy(&f, row + 4 * i, 4);
      w[i] = f;
    } else if (type == TYPE_F16) {
      w[i] = dqo_fp16_to_f32(rd16(row + 2 * i));
    } else if (type == TYPE_BF16) {
      const uint32_t bits = (uint32_t)rd16(row + 2 * i) << 16;
      float f;
      memcpy(&f, &bits, 4);
      w[i] = f;
    }
  }
  if (type == TYPE_Q8_0) {
    for (int64_t b = 0; b < K / 32; ++b) {
      float d;
      int8_t q[32];
      dqo_decode_q8_0(row + b * Q8_0_BYTES, &d, q);
      for (int i = 0; i < 32; ++i) w[32 * b + i] = (double)d * q[i];
    }
  } else if (type == TYPE_Q5K) {
    for (int64_t b = 0; b < K / QK; ++b) {
      float d, dmin;
      uint8_t sc[8], mn[8], q[256];
      dqo_decode_q5k(row + b * Q5K_BYTES, &d, &dmin, sc, mn, q);
      for (int i = 0; i < QK; ++i)
        w[QK * b + i] = (double)d * sc[i / 32] * q[i] - (double)dmin * mn[i / 32];
    }
  }
  return 0;
}

/* Embedding rows: out[i][k] = row ids[i] of the N x K table, decoded and   */
/* rounded once to binary32 (out row stride ldo); an id outside [0, N) gives */
/* a row of zeros and flag[i] = 1 (else 0).                                  */
int dqo_embed_rows(int type, int64_t N, int64_t K, const uint8_t *table, const int32_t *ids,
                   int64_t M, float *out, int64_t ldo, int32_t *flag) {
  const int64_t rb = dqo_row_bytes(type, K);
  if (!rb || ldo < K) return -1;
  double *w = (double *)malloc(sizeof(double) * (size_t)K);
  if (!w) return -2;
  for (int64_t i = 0; i < M; ++i) {
    const int64_t id = ids[i];
    flag[i] = id < 0 || id >= N;
    if (flag[i]) {
      for (int64_t k = 0; k < K; ++k) out[i * ldo + k] = 0.0f;
      continue;
    }
    dqo_decode_row(type, table + id * rb, K, w);
    for (int64_t k = 0; k < K; ++k) out[i * ldo + k] = (float)w[k];
  }
  free(w);
  return 0;
}
