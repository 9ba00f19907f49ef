/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for the NVFP4-quantized dense MLP.
 *
 * TEST INFRASTRUCTURE. This file is the reference the GPU library is checked
 * against; it is not part of the product. Only the test suite, the smoke
 * check of the entry module and the CPU-baseline leg of the benchmark may
 * load it. It shares no code, header, table or helper with the HIP library.
 *
 * What it computes, and where that comes from:
 *
 *  - The NVFP4 encoding: 4-bit E2M1 elements (grid {0, .5, 1, 1.5, 2, 3, 4, 6},
 *    sign in bit 3), one E4M3FN scale byte per 16 consecutive elements of a
 *    row, and one fp32 global scale per tensor.  The pages call this format
 *    through library functions only: scale bytes are viewed as
 *    `float8_e4m3fn` and a row of width K has K/16 of them
 *    (sglang PR #35120 report, key source snippets, flashinfer_cutedsl.py
 *    activation-quant branch: `x_sf.view(torch.float8_e4m3fn).reshape(seq_len,
 *    hidden_size // _FP4_SF_VEC_SIZE)`; sglang PR #34859 digest, key source
 *    snippets, qwen2_moe.py `_silu_fp4_quant_fused`: K/64 groups of 4 scales).
 *    The exact fp32 operation order of the encoder is not printed on the
 *    pages; the one used here is the plainest reading (one scale per block
 *    from the block amax, one correctly rounded division per block, one
 *    multiply per element) and is listed among the readings of the design
 *    notes.
 *  - Quantize with the inverse global scale (`fp4_quantize(x,
 *    gate_up_proj.input_scale_inv)`, sglang PR #26626 digest, key source
 *    snippets, deepseek_v2.py DeepseekV2MLP.forward).
 *  - NVFP4 x NVFP4 GEMM with one fp32 `alpha` (`fp4_gemm` ->
 *    `flashinfer_fp4_gemm(input, weight, input_sf, weight_sf, alpha, ...)`,
 *    sglang PR #35120 report, key source snippets, modelopt_quant.py), and
 *    the W4A16 GEMM of bf16 activations against NVFP4 weights whose alpha
 *    holds the weight dequant factor only (same report, implementation
 *    breakdown items 2 and 3).
 *  - SiLU(gate) * up with gate the first half of the gate_up output
 *    (`gate_w, up_w = w.chunk(2)`, PR #26626 digest, key source snippets,
 *    modelopt_quant.py process_weights_after_loading; `act_fn(gate_up)` in
 *    PR #34859 digest, qwen2_moe.py forward), then re-quantization with
 *    `down_proj.input_scale_inv` and the down_proj GEMM on the pre-quantized
 *    (codes, scales) pair (PR #26626 digest, DeepseekV2MLP.forward).
 *  - Per-token dynamic activation scales (`nvfp4_quantize(hidden_states,
 *    a1_scale, per_token_activation=True)` returning a per-token scale that
 *    the GEMM takes as `per_token_scale`, while the second GEMM's input keeps
 *    its static `a2_scale`: PR #35120 report, key source snippets,
 *    flashinfer_cutedsl.py activation-quant branch). The pages print only the
 *    call; the reading used here is the per-tensor calibration applied to
 *    each token row: g_t = fl(amax_t / 2688), g_inv_t = fl(1 / g_t), the row
 *    quantized with g_inv_t, and the GEMM output of token t scaled by
 *    fl(g_t * g_w). A row of zeros has g_t = 0 and quantizes with g_inv = 0
 *    to zero codes and scales (the pages do not say; this keeps it finite).
 *  - Standalone SiLU(gate) * up + NVFP4 quantization of a bf16 gate_up
 *    output batched by expert with `masked_m`
 *    (`silu_and_mul_scaled_nvfp4_experts_quantize(gate_up.unsqueeze(0),
 *    masked_m, down_proj.input_scale_inv.reshape(1))`, sglang PR #34859
 *    digest, key source snippets, qwen2_moe.py `_silu_fp4_quant_fused`):
 *    gate_up is [E, M, 2I] bf16, expert e's first masked_m[e] rows are
 *    valid and quantized with that expert's inverse global scale; the
 *    reading used here leaves the rows past masked_m[e] unwritten.
 *  - Grouped (expert) NVFP4 GEMMs with masked_m: the MoE path runs W4A4 or
 *    W4A16 GEMMs per expert with each expert's own weights and alpha, over
 *    the expert's valid token rows (sglang PR #35120 report, implementation
 *    breakdown item 3; masked_m as in the PR #34859 digest's
 *    `_silu_fp4_quant_fused`). Read here as: expert e's first masked_m[e]
 *    rows of its activation block get that expert's GEMM; the other rows of
 *    the output are left unwritten. Routing is not part of it.
 *  - AWQ pre-quant scales of the W4A16 mode: the W4A16 branch of a linear
 *    layer's `apply` pre-scales its bf16 input by the layer's per-input-
 *    channel `pre_quant_scale` before calling the W4A16 GEMM (sglang
 *    PR #35120 report, implementation breakdown item 2). Read here as the
 *    bf16 elementwise product x' = bf16(x * s) (the fp32 product of two bf16
 *    values is exact; one rounding to nearest even), applied to the input
 *    of both GEMMs of the MLP: x with the gate_up layer's scale over H and
 *    the bf16 h with the down layer's scale over I.
 *
 * Arithmetic conventions:
 *  - Encoding steps are binary32 operations with round-to-nearest-even,
 *    subnormals kept (build with -ffp-contract=off, no fast-math; x86-64 SSE
 *    arithmetic has no excess precision).
 *  - Contractions are evaluated in double. Every element product and every
 *    16-element block sum is exact in double; only the sum over blocks
 *    rounds (relative 1e-16), and the result is rounded once to fp32.
 *  - Inputs must be finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* Element and scale formats                                                 */
/* ------------------------------------------------------------------------ */

/* The E2M1 magnitudes indexed by the low three bits of a code. */
static const double kE2M1Magnitude[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Value of a 4-bit E2M1 code: bit 3 is the sign, bits 0..2 index the grid. */
ORC_API double orc_e2m1_value(uint32_t code) {
  double m = kE2M1Magnitude[code & 7u];
  return (code & 8u) ? -m : m;
}

/* Value of an E4M3FN byte: 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is
 * NaN; there is no infinity. */
ORC_API double orc_e4m3_value(uint32_t byte) {
  uint32_t b = byte & 0xFFu;
  int sign = (int)(b >> 7);
  int e = (int)((b >> 3) & 15u);
  int m = (int)(b & 7u);
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* Nearest E4M3FN value to a non-negative finite v, ties to the even
 * mantissa, saturating to the largest finite value 448 (byte 0x7E).
 * The value is written n * 2^(e-3) with n an integer in [8, 16) for normal
 * numbers and n * 2^-9 with n in [0, 8) for subnormals; rounding the scaled
 * value to an integer under round-half-even picks the nearest neighbour. */
ORC_API uint32_t orc_e4m3_encode(float v) {
  double x = (double)v;
  if (!(x > 0.0)) return 0u; /* zero (and -0) encode to 0x00 */
  if (x >= 448.0) return 0x7Eu;
  int ex;
  (void)frexp(x, &ex); /* x = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;      /* floor(log2 x) */
  if (e < -6) {
    double n = nearbyint(ldexp(x, 9)); /* multiples of 2^-9 */
    /* n == 8 is the smallest normal 2^-6, whose byte is also 8 */
    return (uint32_t)n;
  }
  double n = nearbyint(ldexp(x, 3 - e)); /* in [8, 16] */
  if (n >= 16.0) { n = 8.0; e += 1; }
  /* x < 448 and the step at e = 8 is 32, so rounding never passes 448 */
  return (uint32_t)(((e + 7) << 3) | ((int)n - 8));
}

/* Nearest E2M1 grid value to y, ties to the even code, saturating at 6.
 * The sign bit of the code is the sign bit of y (so -0.1 gives code 0x8).
 * The search walks the midpoints between neighbouring grid values. */
ORC_API uint32_t orc_e2m1_encode(float y) {
  double a = fabs((double)y);
  uint32_t code = 7u;
  for (uint32_t i = 0; i < 7u; ++i) {
    double mid = 0.5 * (kE2M1Magnitude[i] + kE2M1Magnitude[i + 1]);
    if (a < mid) { code = i; break; }
    if (a == mid) { code = (i % 2u == 0u) ? i : i + 1u; break; }
  }
  return signbit(y) ? (code | 8u) : code;
}

/* bf16 <-> fp32. bf16 is the top half of a binary32, so widening is exact;
 * narrowing rounds to nearest, ties to even (finite inputs only). */
ORC_API float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
ORC_API uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lower = u & 0xFFFFu;
  uint32_t upper = u >> 16;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

/* ------------------------------------------------------------------------ */
/* Scales                                                                    */
/* ------------------------------------------------------------------------ */

/* Per-tensor calibration: the tensor's amax is mapped onto the largest
 * product of an element and a scale, 6 * 448 = 2688:
 *   g = fl(amax / 2688),  g_inv = fl(1 / g).
 * The quantizer takes g_inv, as `fp4_quantize` takes `input_scale_inv`. */
ORC_API void orc_global_scale(const float* x, int64_t n, float* g, float* g_inv) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float gg = amax / 2688.0f;
  *g = gg;
  *g_inv = 1.0f / gg;
}

/* GEMM output scale of two NVFP4 operands: the product of their global
 * scales, one fp32 multiply. */
ORC_API float orc_alpha(float g_a, float g_w) { return g_a * g_w; }

/* ------------------------------------------------------------------------ */
/* Quantize                                                                  */
/* ------------------------------------------------------------------------ */

/* Quantize one row-major fp32 matrix x [M, K] (K % 16 == 0) to
 *   codes  [M, K/2]  two codes per byte, element 2i in the low nibble,
 *   scales [M, K/16] one E4M3FN byte per 16-element block.
 * For every block:
 *   amax = max |x_k|
 *   sv   = fl(fl(amax * g_inv) / 6)       block scale in units of the global
 *   s    = E4M3(sv)                       nearest, ties even, saturating
 *   r    = fl(g_inv / s), or 0 if s == 0  one division per block
 *   y_k  = fl(x_k * r)
 *   c_k  = E2M1(y_k)                      nearest, ties even, saturating */
ORC_API void orc_quantize(const float* x, int64_t M, int64_t K, float g_inv,
                          uint8_t* codes, uint8_t* scales) {
  int64_t nb = K / 16;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t b = 0; b < nb; ++b) {
      const float* xb = x + i * K + b * 16;
      float amax = 0.0f;
      for (int k = 0; k < 16; ++k) {
        float a = fabsf(xb[k]);
        if (a > amax) amax = a;
      }
      float t = amax * g_inv;
      float sv = t / 6.0f;
      uint32_t sbyte = orc_e4m3_encode(sv);
      float s = (float)orc_e4m3_value(sbyte);
      float r = (s != 0.0f) ? g_inv / s : 0.0f;
      scales[i * nb + b] = (uint8_t)sbyte;
      for (int k = 0; k < 16; k += 2) {
        float y0 = xb[k] * r;
        float y1 = xb[k + 1] * r;
        uint32_t c0 = orc_e2m1_encode(y0);
        uint32_t c1 = orc_e2m1_encode(y1);
        codes[i * (K / 2) + b * 8 + k / 2] = (uint8_t)(c0 | (c1 << 4));
      }
    }
  }
}

/* Per-token dynamic quantization of x [M, K]: each row calibrated on its own
 * amax like orc_global_scale, then quantized like orc_quantize with its own
 * g_inv; g_rows[i] receives the row's g. */
ORC_API void orc_quantize_per_token(const float* x, int64_t M, int64_t K, uint8_t* codes,
                                    uint8_t* scales, float* g_rows) {
  for (int64_t i = 0; i < M; ++i) {
    const float* row = x + i * K;
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      float a = fabsf(row[k]);
      if (a > amax) amax = a;
    }
    float g = amax / 2688.0f;
    float g_inv = (g != 0.0f) ? 1.0f / g : 0.0f;
    g_rows[i] = g;
    orc_quantize(row, 1, K, g_inv, codes + i * (K / 2), scales + i * (K / 16));
  }
}

/* Element (row, k) of an NVFP4 matrix without its global scale: q * s. */
static double nvfp4_elem(const uint8_t* codes, const uint8_t* scales, int64_t K,
                         int64_t row, int64_t k) {
  uint8_t byte = codes[row * (K / 2) + k / 2];
  uint32_t code = (k & 1) ? (uint32_t)(byte >> 4) : (uint32_t)(byte & 15u);
  return orc_e2m1_value(code) * orc_e4m3_value(scales[row * (K / 16) + k / 16]);
}

/* Dense double copy of an NVFP4 matrix without its global scale. */
ORC_API void orc_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t M,
                            int64_t K, double* out) {
  for (int64_t i = 0; i < M; ++i)
    for (int64_t k = 0; k < K; ++k) out[i * K + k] = nvfp4_elem(codes, scales, K, i, k);
}

/* ------------------------------------------------------------------------ */
/* GEMMs:  out[i, j] = fl32(alpha * sum_k A[i, k] * W[j, k]),  W is [N, K]    */
/* ------------------------------------------------------------------------ */

/* W4A4, block-factored as the format suggests:
 *   sum_b (s_a[i,b] * s_w[j,b]) * sum_{k in b} q_a[i,k] * q_w[j,k]. */
ORC_API void orc_gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales,
                           const uint8_t* w_codes, const uint8_t* w_scales,
                           int64_t M, int64_t N, int64_t K, float alpha, float* out) {
  int64_t nb = K / 16;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < N; ++j) {
    for (int64_t i = 0; i < M; ++i) {
      double acc = 0.0;
      for (int64_t b = 0; b < nb; ++b) {
        double inner = 0.0;
        for (int64_t k = b * 16; k < b * 16 + 16; ++k) {
          uint8_t ab = a_codes[i * (K / 2) + k / 2];
          uint8_t wb = w_codes[j * (K / 2) + k / 2];
          uint32_t ac = (k & 1) ? (uint32_t)(ab >> 4) : (uint32_t)(ab & 15u);
          uint32_t wc = (k & 1) ? (uint32_t)(wb >> 4) : (uint32_t)(wb & 15u);
          inner += orc_e2m1_value(ac) * orc_e2m1_value(wc);
        }
        acc += orc_e4m3_value(a_scales[i * nb + b]) * orc_e4m3_value(w_scales[j * nb + b]) * inner;
      }
      out[i * N + j] = (float)((double)alpha * acc);
    }
  }
}

/* W4A4, second formulation: dequantize both operands to dense doubles and
 * take plain dot products over k.  Shares only the format decoders with the
 * block-factored version. */
ORC_API void orc_gemm_w4a4_dense(const uint8_t* a_codes, const uint8_t* a_scales,
                                 const uint8_t* w_codes, const uint8_t* w_scales,
                                 int64_t M, int64_t N, int64_t K, float alpha, float* out) {
  double* A = (double*)malloc(sizeof(double) * (size_t)(M * K));
  double* W = (double*)malloc(sizeof(double) * (size_t)(N * K));
  orc_dequantize(a_codes, a_scales, M, K, A);
  orc_dequantize(w_codes, w_scales, N, K, W);
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += A[i * K + k] * W[j * K + k];
      out[i * N + j] = (float)((double)alpha * acc);
    }
  free(A);
  free(W);
}

/* W4A16: bf16 activations x [M, K] against NVFP4 weights; alpha is the
 * weight's global scale alone.  Block-factored over the weight scales. */
ORC_API void orc_gemm_w4a16(const uint16_t* x, const uint8_t* w_codes, const uint8_t* w_scales,
                            int64_t M, int64_t N, int64_t K, float alpha, float* out) {
  int64_t nb = K / 16;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < N; ++j) {
    for (int64_t i = 0; i < M; ++i) {
      double acc = 0.0;
      for (int64_t b = 0; b < nb; ++b) {
        double inner = 0.0;
        for (int64_t k = b * 16; k < b * 16 + 16; ++k) {
          uint8_t wb = w_codes[j * (K / 2) + k / 2];
          uint32_t wc = (k & 1) ? (uint32_t)(wb >> 4) : (uint32_t)(wb & 15u);
          inner += (double)orc_bf16_to_f32(x[i * K + k]) * orc_e2m1_value(wc);
        }
        acc += orc_e4m3_value(w_scales[j * nb + b]) * inner;
      }
      out[i * N + j] = (float)((double)alpha * acc);
    }
  }
}

/* W4A16, dense formulation. */
ORC_API void orc_gemm_w4a16_dense(const uint16_t* x, const uint8_t* w_codes,
                                  const uint8_t* w_scales, int64_t M, int64_t N, int64_t K,
                                  float alpha, float* out) {
  double* W = (double*)malloc(sizeof(double) * (size_t)(N * K));
  orc_dequantize(w_codes, w_scales, N, K, W);
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += (double)orc_bf16_to_f32(x[i * K + k]) * W[j * K + k];
      out[i * N + j] = (float)((double)alpha * acc);
    }
  free(W);
}

/* ------------------------------------------------------------------------ */
/* SwiGLU and the MLP                                                        */
/* ------------------------------------------------------------------------ */

/* h[i, j] = fl32(silu(g) * u) with g = gu[i, j], u = gu[i, I + j] and
 * silu(g) = g / (1 + e^-g), evaluated in double. */
ORC_API void orc_swiglu(const float* gu, int64_t M, int64_t I, float* h) {
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < I; ++j) {
      double g = (double)gu[i * 2 * I + j];
      double u = (double)gu[i * 2 * I + I + j];
      double silu = g / (1.0 + exp(-g));
      h[i * I + j] = (float)(silu * u);
    }
}

/* W4A4 GEMM with a per-row output scale: row i of the output is the W4A4
 * GEMM of row i of A with alpha_rows[i] (block-factored as orc_gemm_w4a4). */
ORC_API void orc_gemm_w4a4_rows(const uint8_t* a_codes, const uint8_t* a_scales,
                                const uint8_t* w_codes, const uint8_t* w_scales, int64_t M,
                                int64_t N, int64_t K, const float* alpha_rows, float* out) {
  for (int64_t i = 0; i < M; ++i)
    orc_gemm_w4a4(a_codes + i * (K / 2), a_scales + i * (K / 16), w_codes, w_scales, 1, N, K,
                  alpha_rows[i], out + i * N);
}

/* W4A4 MLP forward with per-token dynamic scales for x (h keeps its static
 * g2_inv):
 *   x  -> NVFP4 per token, g_t                     (orc_quantize_per_token)
 *   gu = fl32(fl(g_t * g_wgu) * x_t @ Wgu^T)       per token row t
 *   h  = SwiGLU(gu); hq = NVFP4(h) with g2_inv; out = fl32(alpha_d * hq @ Wd^T)
 * Optional stage outputs (NULL to skip): xq/xs, g_rows, gu, h, hq/hs. */
ORC_API void orc_mlp_w4a4_per_token(const uint16_t* x, int64_t M, int64_t H, int64_t I,
                                    const uint8_t* wgu_codes, const uint8_t* wgu_scales, float g_wgu,
                                    const uint8_t* wd_codes, const uint8_t* wd_scales, float alpha_d,
                                    float g2_inv, float* out, uint8_t* xq_out, uint8_t* xs_out,
                                    float* g_out, float* gu_out, float* h_out, uint8_t* hq_out,
                                    uint8_t* hs_out) {
  float* xf = (float*)malloc(sizeof(float) * (size_t)(M * H));
  uint8_t* xq = (uint8_t*)malloc((size_t)(M * H / 2));
  uint8_t* xs = (uint8_t*)malloc((size_t)(M * H / 16));
  float* g = (float*)malloc(sizeof(float) * (size_t)M);
  float* a_rows = (float*)malloc(sizeof(float) * (size_t)M);
  float* gu = (float*)malloc(sizeof(float) * (size_t)(M * 2 * I));
  float* h = (float*)malloc(sizeof(float) * (size_t)(M * I));
  uint8_t* hq = (uint8_t*)malloc((size_t)(M * I / 2));
  uint8_t* hs = (uint8_t*)malloc((size_t)(M * I / 16));
  for (int64_t t = 0; t < M * H; ++t) xf[t] = orc_bf16_to_f32(x[t]);
  orc_quantize_per_token(xf, M, H, xq, xs, g);
  for (int64_t i = 0; i < M; ++i) a_rows[i] = orc_alpha(g[i], g_wgu);
  orc_gemm_w4a4_rows(xq, xs, wgu_codes, wgu_scales, M, 2 * I, H, a_rows, gu);
  orc_swiglu(gu, M, I, h);
  orc_quantize(h, M, I, g2_inv, hq, hs);
  orc_gemm_w4a4(hq, hs, wd_codes, wd_scales, M, H, I, alpha_d, out);
  if (xq_out) memcpy(xq_out, xq, (size_t)(M * H / 2));
  if (xs_out) memcpy(xs_out, xs, (size_t)(M * H / 16));
  if (g_out) memcpy(g_out, g, sizeof(float) * (size_t)M);
  if (gu_out) memcpy(gu_out, gu, sizeof(float) * (size_t)(M * 2 * I));
  if (h_out) memcpy(h_out, h, sizeof(float) * (size_t)(M * I));
  if (hq_out) memcpy(hq_out, hq, (size_t)(M * I / 2));
  if (hs_out) memcpy(hs_out, hs, (size_t)(M * I / 16));
  free(xf); free(xq); free(xs); free(g); free(a_rows); free(gu); free(h); free(hq); free(hs);
}

/* W4A4 MLP forward, x bf16 [M, H]:
 *   x  -> NVFP4 with g1_inv                                (activation quant)
 *   gu = fl32(alpha_gu * x @ Wgu^T)     Wgu [2I, H] rows [gate; up]
 *   h  = SwiGLU(gu)                     fp32 [M, I]
 *   hq = NVFP4(h) with g2_inv                               (re-quant)
 *   out = fl32(alpha_d * hq @ Wd^T)     Wd [H, I]
 * Optional stage outputs (NULL to skip): xq/xs, gu, h, hq/hs. */
ORC_API void orc_mlp_w4a4(const uint16_t* x, int64_t M, int64_t H, int64_t I,
                          const uint8_t* wgu_codes, const uint8_t* wgu_scales, float alpha_gu,
                          const uint8_t* wd_codes, const uint8_t* wd_scales, float alpha_d,
                          float g1_inv, float g2_inv, float* out,
                          uint8_t* xq_out, uint8_t* xs_out, float* gu_out, float* h_out,
                          uint8_t* hq_out, uint8_t* hs_out) {
  float* xf = (float*)malloc(sizeof(float) * (size_t)(M * H));
  uint8_t* xq = (uint8_t*)malloc((size_t)(M * H / 2));
  uint8_t* xs = (uint8_t*)malloc((size_t)(M * H / 16));
  float* gu = (float*)malloc(sizeof(float) * (size_t)(M * 2 * I));
  float* h = (float*)malloc(sizeof(float) * (size_t)(M * I));
  uint8_t* hq = (uint8_t*)malloc((size_t)(M * I / 2));
  uint8_t* hs = (uint8_t*)malloc((size_t)(M * I / 16));
  for (int64_t t = 0; t < M * H; ++t) xf[t] = orc_bf16_to_f32(x[t]);
  orc_quantize(xf, M, H, g1_inv, xq, xs);
  orc_gemm_w4a4(xq, xs, wgu_codes, wgu_scales, M, 2 * I, H, alpha_gu, gu);
  orc_swiglu(gu, M, I, h);
  orc_quantize(h, M, I, g2_inv, hq, hs);
  orc_gemm_w4a4(hq, hs, wd_codes, wd_scales, M, H, I, alpha_d, out);
  if (xq_out) memcpy(xq_out, xq, (size_t)(M * H / 2));
  if (xs_out) memcpy(xs_out, xs, (size_t)(M * H / 16));
  if (gu_out) memcpy(gu_out, gu, sizeof(float) * (size_t)(M * 2 * I));
  if (h_out) memcpy(h_out, h, sizeof(float) * (size_t)(M * I));
  if (hq_out) memcpy(hq_out, hq, (size_t)(M * I / 2));
  if (hs_out) memcpy(hs_out, hs, (size_t)(M * I / 16));
  free(xf); free(xq); free(xs); free(gu); free(h); free(hq); free(hs);
}

/* W4A16 MLP forward: bf16 activations throughout, no activation quant.
 *   gu  = fl32(alpha_gu * x @ Wgu^T)
 *   h   = bf16(SwiGLU(gu))             round to nearest even
 *   out = fl32(alpha_d * h @ Wd^T)
 * Optional stage outputs: gu (fp32), h (bf16 bits). */
ORC_API void orc_mlp_w4a16(const uint16_t* x, int64_t M, int64_t H, int64_t I,
                           const uint8_t* wgu_codes, const uint8_t* wgu_scales, float alpha_gu,
                           const uint8_t* wd_codes, const uint8_t* wd_scales, float alpha_d,
                           float* out, float* gu_out, uint16_t* h_out) {
  float* gu = (float*)malloc(sizeof(float) * (size_t)(M * 2 * I));
  float* h = (float*)malloc(sizeof(float) * (size_t)(M * I));
  uint16_t* hb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(M * I));
  orc_gemm_w4a16(x, wgu_codes, wgu_scales, M, 2 * I, H, alpha_gu, gu);
  orc_swiglu(gu, M, I, h);
  for (int64_t t = 0; t < M * I; ++t) hb[t] = orc_f32_to_bf16(h[t]);
  orc_gemm_w4a16(hb, wd_codes, wd_scales, M, H, I, alpha_d, out);
  if (gu_out) memcpy(gu_out, gu, sizeof(float) * (size_t)(M * 2 * I));
  if (h_out) memcpy(h_out, hb, sizeof(uint16_t) * (size_t)(M * I));
  free(gu); free(h); free(hb);
}

/* Threads the parallel loops above use. */
ORC_API int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Standalone SiLU(gate) * up + NVFP4 quantization by expert:
 *   gate_up bf16 [E, M, 2I] (row = [gate | up]), masked_m[E] valid rows per
 *   expert, g_inv[E] inverse global scale per expert.
 *   For e < E, t < masked_m[e]:  h = SwiGLU(fp32(gate_up[e, t]))  (fp32 [I]),
 *   then NVFP4(h) with g_inv[e] into codes [E, M, I/2], scales [E, M, I/16].
 *   Rows t >= masked_m[e] are left as they are. h_out (NULL to skip) gets h
 *   of the written rows, [E, M, I]. */
ORC_API void orc_silu_mul_quant_experts(const uint16_t* gate_up, int64_t E, int64_t M, int64_t I,
                                        const int32_t* masked_m, const float* g_inv, uint8_t* codes,
                                        uint8_t* scales, float* h_out) {
  float* gu = (float*)malloc(sizeof(float) * (size_t)(2 * I));
  float* h = (float*)malloc(sizeof(float) * (size_t)I);
  for (int64_t e = 0; e < E; ++e) {
    int64_t rows = masked_m[e] < 0 ? 0 : (masked_m[e] > M ? M : masked_m[e]);
    for (int64_t t = 0; t < rows; ++t) {
      const int64_t row = e * M + t;
      for (int64_t k = 0; k < 2 * I; ++k) gu[k] = orc_bf16_to_f32(gate_up[row * 2 * I + k]);
      orc_swiglu(gu, 1, I, h);
      orc_quantize(h, 1, I, g_inv[e], codes + row * (I / 2), scales + row * (I / 16));
      if (h_out) memcpy(h_out + row * I, h, sizeof(float) * (size_t)I);
    }
  }
  free(gu);
  free(h);
}

/* AWQ pre-quant scaling of a bf16 input: out[m, k] = bf16(x[m, k] * s[k]),
 * x [M, K] and s [K] bf16 (the product is exact in fp32, then rounded to
 * nearest even). */
ORC_API void orc_prescale_bf16(const uint16_t* x, const uint16_t* s, int64_t M, int64_t K, uint16_t* out) {
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k)
      out[m * K + k] = orc_f32_to_bf16(orc_bf16_to_f32(x[m * K + k]) * orc_bf16_to_f32(s[k]));
}

/* W4A16 MLP forward with AWQ pre-quant scales on both GEMM inputs:
 *   x' = prescale(x, s_gu);  gu = fl32(alpha_gu * x' @ Wgu^T);
 *   h  = bf16(SwiGLU(gu));   h' = prescale(h, s_d);
 *   out = fl32(alpha_d * h' @ Wd^T).
 * Optional stage outputs (NULL to skip): x', h' (bf16 bits). */
ORC_API void orc_mlp_w4a16_awq(const uint16_t* x, int64_t M, int64_t H, int64_t I,
                               const uint8_t* wgu_codes, const uint8_t* wgu_scales, float alpha_gu,
                               const uint16_t* s_gu, const uint8_t* wd_codes, const uint8_t* wd_scales,
                               float alpha_d, const uint16_t* s_d, float* out, uint16_t* xs_out,
                               uint16_t* hs_out) {
  uint16_t* xs = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(M * H));
  float* gu = (float*)malloc(sizeof(float) * (size_t)(M * 2 * I));
  float* h = (float*)malloc(sizeof(float) * (size_t)(M * I));
  uint16_t* hb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(M * I));
  uint16_t* hs = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(M * I));
  orc_prescale_bf16(x, s_gu, M, H, xs);
  orc_gemm_w4a16(xs, wgu_codes, wgu_scales, M, 2 * I, H, alpha_gu, gu);
  orc_swiglu(gu, M, I, h);
  for (int64_t t = 0; t < M * I; ++t) hb[t] = orc_f32_to_bf16(h[t]);
  orc_prescale_bf16(hb, s_d, M, I, hs);
  orc_gemm_w4a16(hs, wd_codes, wd_scales, M, H, I, alpha_d, out);
  if (xs_out) memcpy(xs_out, xs, sizeof(uint16_t) * (size_t)(M * H));
  if (hs_out) memcpy(hs_out, hs, sizeof(uint16_t) * (size_t)(M * I));
  free(xs); free(gu); free(h); free(hb); free(hs);
}

/* Grouped (expert) GEMM with masked rows:
 *   for e < E, t < clamp(masked_m[e], 0, M):
 *     out[e, t, :] = GEMM(a[e, t, :], W_e) with alpha[e]
 * mode 0 (W4A4): a_codes [E, M, K/2], a_scales [E, M, K/16]; mode 1 (W4A16):
 * a_bf16 [E, M, K]. W_e: codes [E, N, K/2], scales [E, N, K/16]. out
 * [E, M, N]; rows past masked_m are left as they are. */
ORC_API void orc_grouped_gemm(int mode, const uint8_t* a_codes, const uint8_t* a_scales, const uint16_t* a_bf16,
                              const uint8_t* w_codes, const uint8_t* w_scales, int64_t E, int64_t M, int64_t N,
                              int64_t K, const int32_t* masked_m, const float* alpha, float* out) {
  for (int64_t e = 0; e < E; ++e) {
    const int64_t rows = masked_m[e] < 0 ? 0 : (masked_m[e] > M ? M : masked_m[e]);
    if (rows == 0) continue;
    const uint8_t* wc = w_codes + e * N * (K / 2);
    const uint8_t* ws = w_scales + e * N * (K / 16);
    float* o = out + e * M * N;
    if (mode == 0)
      orc_gemm_w4a4(a_codes + e * M * (K / 2), a_scales + e * M * (K / 16), wc, ws, rows, N, K, alpha[e], o);
    else
      orc_gemm_w4a16(a_bf16 + e * M * K, wc, ws, rows, N, K, alpha[e], o);
  }
}
