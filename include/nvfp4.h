/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 dense-MLP library.
 *
 * The hot path of an NVFP4-quantized dense MLP in LLM inference:
 *   activation quantize -> gate_up GEMM -> SiLU(gate) * up -> NVFP4
 *   re-quantize -> down_proj GEMM,
 * plus a W4A16 variant (bf16 activations against NVFP4 weights) and a
 * one-time weight repack. The call sequence follows the fused MLP forward of
 * sglang PR #26626 ("fuse NVFP4 gate_up_gemm + Swish + output quant", key
 * source snippets: DeepseekV2MLP.forward) and the W4A16 dense path of the
 * PR #35120 report ("add FlashInfer CuTe DSL NVFP4 W4A16 mode", key source
 * snippets: fp4_gemm).
 *
 * Formats (all row-major, little-endian):
 *   bf16      uint16 bit patterns.
 *   NVFP4     codes  uint8 [rows, K/2]: two 4-bit E2M1 codes per byte, element
 *                    2i in the low nibble; bit 3 of a code is the sign, bits
 *                    0..2 index {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *             scales uint8 [rows, K/16]: one E4M3FN byte per 16 consecutive
 *                    elements of a row (the pages' `float8_e4m3fn` view with
 *                    K/16 scales per row, PR #35120 report, key source
 *                    snippets, flashinfer_cutedsl.py).
 *             value  = E2M1(code) * E4M3(scale) * g, with g the tensor's fp32
 *                    global scale.
 *   packed    an opaque weight buffer written by nvfp4_repack_weight; the same
 *             bytes as codes + scales, permuted for the kernels' loads.
 *
 * Scalars g_inv, alpha, g2_inv are 1-element fp32 arrays in DEVICE memory
 * (like `input_scale_inv` and `alpha` tensors on the pages), so a call never
 * synchronizes with the host.
 *
 * Ownership and execution: the caller allocates every buffer (inputs,
 * outputs, packed weights sized by nvfp4_repack_bytes, workspace sized by
 * mlp_workspace_bytes) and keeps it alive until the work on `stream` has
 * finished. Calls are asynchronous on `stream` (a hipStream_t; NULL is the
 * default stream). The library never allocates, frees, synchronizes or reads
 * the environment. Device pointers must be 16-byte aligned. Calls that share
 * no output buffer may run concurrently on different streams.
 *
 * Sizes: unless an entry point below states its own limit, every row count
 * and GEMM dimension (M, N, K, H, I, R, C) is at most 2^24 = 16,777,216; a
 * larger size is NVFP4_ERR_INVALID_ARG.
 *
 * Errors: every entry point returns NVFP4_OK or a negative code and leaves a
 * thread-local message for nvfp4_last_error(). Argument checks come before
 * any HIP call, so a rejected call has no effect on the device. There is no
 * fallback path: an unsupported device or combination is an error.
 */
#ifndef NVFP4_MI355X_H_
#define NVFP4_MI355X_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_OK 0
#define NVFP4_ERR_INVALID_ARG (-1) /* null/misaligned pointer, bad size or enum */
#define NVFP4_ERR_UNSUPPORTED (-2) /* device is not gfx950, or mode/dtype combination not offered */
#define NVFP4_ERR_HIP (-3)         /* a HIP runtime call or kernel launch failed */

/* Element types of dense buffers. */
#define NVFP4_DTYPE_BF16 0
#define NVFP4_DTYPE_F32 1

/* GEMM / MLP quantization modes (the pages' `quant_mode` "w4a4" | "w4a16",
 * PR #35120 report, implementation breakdown item 1). */
#define NVFP4_MODE_W4A4 0  /* NVFP4 activations x NVFP4 weights */
#define NVFP4_MODE_W4A16 1 /* bf16 activations x NVFP4 weights */
#define NVFP4_MODE_W4A4_DYN 2 /* W4A4 with per-token dynamic scales for x (mlp_forward only) */
#define NVFP4_MODE_W4A16_AWQ 3 /* W4A16 with AWQ pre-quant scales (mlp_forward_w4a16_awq, workspace size) */

/* Repack kinds. */
#define NVFP4_REPACK_PLAIN 0  /* any [R, C] weight, e.g. down_proj */
#define NVFP4_REPACK_SWIGLU 1 /* merged gate_up [2I, C], rows [gate; up] */

/* Kernel-class override for tests and benchmarks (per calling thread). */
#define NVFP4_PATH_AUTO 0    /* choose by M */
#define NVFP4_PATH_GEMV 1    /* decode GEMV sized for M <= 2: W4A4 on the FP4 matrix core with the
                                blocks kept apart, W4A16 on the vector ALU (any M) */
#define NVFP4_PATH_STREAM 2  /* weight-streaming MFMA kernel (any M; chosen for W4A4 M <= 128,
                                W4A16 SwiGLU GEMMs M <= 32 and W4A16 dense GEMMs M <= 96, except
                                the W4A4 SwiGLU GEMMs of 33 tokens and more and the down
                                projections of mlp_forward that run NVFP4_PATH_MID) */
#define NVFP4_PATH_TILED 3   /* LDS-tiled MFMA GEMM (any M) */
#define NVFP4_PATH_TILED64 4 /* the tiled GEMM with 64-bit addressing, which AUTO and the other
                                paths run only for operands of 2^31 bytes or more (any M; no
                                split-K; the grouped GEMM treats it as NVFP4_PATH_TILED) */
#define NVFP4_PATH_MID 5     /* 128 weight rows x 48 or 64 tokens per workgroup (whichever pads M
                                less; 48 on a tie; 128 for one-expert W4A4 dense GEMMs whose grid
                                would exceed 256 tiles), the activation brought into LDS once per
                                workgroup (any M; chosen for the W4A4 SwiGLU GEMMs of 33 to 512
                                tokens, the W4A16 SwiGLU GEMMs of 33 to 64 tokens, the W4A4
                                grouped GEMMs of 64 to 512 tokens per expert, and mlp_forward's
                                down projection (W4A4 from 17 tokens, W4A16 from 65 to 192)
                                wherever its grid has at most 256 output tiles and K splits into
                                two or more parts of 8 K tiles, split over the workspace; the
                                W4A16 grouped GEMM runs NVFP4_PATH_STREAM under it) */

/* Message of the last failed call on this thread ("" if none). */
const char* nvfp4_last_error(void);

/*
 * Per-tensor calibration of the global scale (static scales, like the
 * `input_scale` / `input_scale_inv` layer attributes on the pages):
 *   amax = max |x|,  g = fl(amax / 2688),  g_inv = fl(1 / g)
 * where 2688 = 6 * 448 maps amax onto the largest element times the largest
 * scale. x: n elements of x_dtype (bf16 or f32, finite, amax > 0).
 * g, g_inv: 1-element fp32 device outputs (g's memory is also used as the
 * reduction cell while the call runs).
 */
int nvfp4_calibrate(const void* x, int x_dtype, int64_t n, float* g, float* g_inv,
                    void* stream);

/*
 * NVFP4 quantize, `fp4_quantize(x, input_scale_inv)` of PR #26626
 * (DeepseekV2MLP.forward). For each 16-element block of a row:
 *   amax = max |x_k|;  sv = fl(fl(amax * g_inv) / 6);
 *   s = E4M3(sv) rounded to nearest, ties to even, saturating at 448;
 *   r = fl(g_inv / s) (0 if s == 0);  code_k = E2M1(fl(x_k * r)) rounded to
 *   nearest, ties to the even code, saturating at 6, sign kept (-0 -> 0x8).
 * x: [M, K] of x_dtype (bf16 activations, or f32 e.g. for weights); K % 16 == 0,
 * M <= 2^24, K <= 2^30.
 * codes: [M, K/2] out; scales: [M, K/16] out. Bit-exact with the oracle.
 */
int nvfp4_quantize(const void* x, int x_dtype, int64_t M, int64_t K, const float* g_inv,
                   uint8_t* codes, uint8_t* scales, void* stream);

/*
 * Per-token dynamic quantization (the pages' `nvfp4_quantize(hidden_states,
 * a1_scale, per_token_activation=True)`, PR #35120 report, key source
 * snippets, flashinfer_cutedsl.py; the pages print only the call): every row
 * t of x is calibrated on its own amax, g_t = fl(amax_t / 2688),
 * g_inv_t = fl(1 / g_t) (0 for an all-zero row, which quantizes to zeros),
 * and quantized with g_inv_t exactly as nvfp4_quantize does.
 * x [M, K] of x_dtype (finite), K % 16 == 0, M <= 2^24, K <= 2^30; codes [M, K/2], scales
 * [M, K/16] and row_g [M] (fp32 g_t, the GEMM's per-token factor) out.
 */
int nvfp4_quantize_per_token(const void* x, int x_dtype, int64_t M, int64_t K, uint8_t* codes,
                             uint8_t* scales, float* row_g, void* stream);

/*
 * Bytes of the packed weight for an [R, C] NVFP4 matrix: R * C * 9 / 16
 * (the codes and scales, permuted). R % 16 == 0 and C % 256 == 0; kind
 * SWIGLU also needs (R / 2) % 16 == 0. Returns 0 for invalid arguments.
 * nvfp4_packed_bytes is the same function under an older name.
 */
size_t nvfp4_repack_bytes(int kind, int64_t R, int64_t C);
size_t nvfp4_packed_bytes(int kind, int64_t R, int64_t C);

/*
 * One-time weight repack (the pages' load-time interleave of gate/up rows and
 * block-scale swizzle in process_weights_after_loading, PR #26626 key source
 * snippets, modelopt_quant.py; and the W4A16 prepack of the PR #35120 report,
 * implementation breakdown item 2). The layout is this library's own:
 *   tiles of 16 rows x 256 columns, 2304 bytes each, ordered
 *   (row group, column tile); inside a tile, lane l = 0..63 owns codes bytes
 *   [16l, 16l+16) and [1024+16l, 1024+16l+16) = row (l % 16), columns
 *   256t + 128c + 32(l / 16) + [0, 32) for c = 0, 1, and scale bytes
 *   [2048+4l, 2048+4l+4) = the scales of those four 16-column blocks.
 *   kind SWIGLU takes rows [gate (I rows); up (I rows)] and orders row groups
 *   gate 0, up 0, gate 1, up 1, ... (groups of 16), so a pair of adjacent
 *   groups holds the gate and up rows of 16 consecutive outputs.
 * codes [R, C/2], scales [R, C/16] in; packed out (nvfp4_repack_bytes bytes).
 * Deterministic; the inputs may be freed afterwards.
 */
int nvfp4_repack_weight(int kind, const uint8_t* codes, const uint8_t* scales, int64_t R,
                        int64_t C, void* packed, void* stream);

/* Inverse of nvfp4_repack_weight (for verification and export). */
int nvfp4_unpack_weight(int kind, const void* packed, int64_t R, int64_t C, uint8_t* codes,
                        uint8_t* scales, void* stream);

/*
 * NVFP4 GEMM, `fp4_gemm(input, weight, input_sf, weight_sf, alpha, out_dtype,
 * quant_mode)` of the PR #35120 report (key source snippets):
 *   out[m, n] = alpha * sum_k A[m, k] * W[n, k]
 * mode W4A4:  a = activation codes [M, K/2], a_scales = [M, K/16];
 *             W4A4 alpha = g_a * g_w.
 * mode W4A16: a = bf16 activations [M, K], a_scales must be NULL (the pages'
 *             optional `input_sf`); alpha = g_w (weight dequant factor only).
 * w_packed: PLAIN packed weight of [N, K]. K % 256 == 0, N % 16 == 0, M >= 0.
 * out: [M, N] of out_dtype (f32 or bf16, round to nearest even).
 * Accumulation is fp32; the order is fixed per (M, path), so results are
 * deterministic.
 */
int nvfp4_gemm(int mode, const void* a, const uint8_t* a_scales, const void* w_packed,
               int64_t M, int64_t N, int64_t K, const float* alpha, void* out, int out_dtype,
               void* stream);

/*
 * Fused gate_up GEMM + SiLU(gate) * up + NVFP4 re-quantization,
 * `nvfp4_gemm_swiglu_nvfp4_quant(x_fp4, x_scale, W_il, S_il, alpha,
 * down_proj.input_scale_inv)` of PR #26626 (DeepseekV2MLP.forward). W4A4 only,
 * as on the pages (PR #35120 report, implementation breakdown item 5).
 *   gate/up[m, j] = alpha * (A @ W^T) for rows j and I + j of [gate; up],
 *   h = SiLU(gate) * up in fp32, then quantized with g2_inv as nvfp4_quantize
 *   does; h never reaches memory in another form.
 * a_codes [M, K/2], a_scales [M, K/16]; w_gu_packed: SWIGLU packed [2I, K];
 * I % 16 == 0, K % 256 == 0. h_codes [M, I/2], h_scales [M, I/16] out.
 */
int gemm_swiglu_nvfp4_quant(const uint8_t* a_codes, const uint8_t* a_scales,
                            const void* w_gu_packed, int64_t M, int64_t I, int64_t K,
                            const float* alpha, const float* g2_inv, uint8_t* h_codes,
                            uint8_t* h_scales, void* stream);

/*
 * W4A4 GEMM and fused gate_up + SwiGLU + NVFP4 re-quantization on
 * activations with per-token dynamic scales (row_g from
 * nvfp4_quantize_per_token, the pages' `per_token_scale` argument of the
 * GEMM): token t's output scale is fl(g_w * row_g[t]), g_w (device fp32) the
 * weight's global scale; otherwise as nvfp4_gemm (mode W4A4) and
 * gemm_swiglu_nvfp4_quant.
 */
int nvfp4_gemm_rowscale(const uint8_t* a_codes, const uint8_t* a_scales, const float* row_g,
                        const void* w_packed, int64_t M, int64_t N, int64_t K, const float* g_w,
                        void* out, int out_dtype, void* stream);
int gemm_swiglu_nvfp4_quant_rowscale(const uint8_t* a_codes, const uint8_t* a_scales,
                                     const float* row_g, const void* w_gu_packed, int64_t M,
                                     int64_t I, int64_t K, const float* g_w, const float* g2_inv,
                                     uint8_t* h_codes, uint8_t* h_scales, void* stream);

/*
 * gate_up GEMM + SiLU(gate) * up to a dense h [M, I] of h_dtype (bf16: the
 * W4A16 chain's activation; f32: calibration of g2 and checks of the
 * re-quantization). mode and a/a_scales as in nvfp4_gemm. Uses the same
 * accumulation as gemm_swiglu_nvfp4_quant for the same (M, path).
 */
int gemm_swiglu(int mode, const void* a, const uint8_t* a_scales, const void* w_gu_packed,
                int64_t M, int64_t I, int64_t K, const float* alpha, void* h, int h_dtype,
                void* stream);

/* Workspace bytes mlp_forward (or mlp_forward_w4a16_awq, mode
 * NVFP4_MODE_W4A16_AWQ) needs: W4A4 holds x and h in NVFP4 (W4A4_DYN also
 * x's per-token scales); W4A16 holds h in bf16 (W4A16_AWQ also x', the
 * pre-scaled x). Then the split-K partial tiles and two sets of arrival
 * counters (down projection, gate_up), sized for the largest plan over the
 * kernel paths. Each region starts 256-byte aligned. Last, in every mode and
 * for every shape, a tail of 4 MiB counted back from the END of the
 * workspace as passed (ws + ws_bytes): the status word (its last 4 bytes,
 * mlp_workspace_status) and the single-launch decode kernel's records (see
 * mlp_forward). Returns 0 for an unknown mode or bad sizes. */
size_t mlp_workspace_bytes(int mode, int64_t M, int64_t H, int64_t I);

/* Status bits of a workspace's status word. */
#define NVFP4_STATUS_DECODE_WAIT_EXPIRED 1u /* a single-launch decode gave up a bounded wait:
                                               its rows of out are NaN */

/*
 * The status word of an mlp_forward workspace: the device address of its
 * last 4 bytes (4-byte aligned), computed from the arguments alone (no HIP
 * call); NULL if ws is NULL or ws_bytes < 512. Kernels OR status bits into
 * it; the library never clears it. It starts as the workspace's first
 * contents (0 in a zero-filled one); the caller reads it (after the stream
 * has finished) and clears it when it likes.
 */
uint32_t* mlp_workspace_status(void* ws, size_t ws_bytes);

/*
 * Dense MLP forward, the pages' fused path (PR #26626, DeepseekV2MLP.forward):
 *   W4A4:  x -> nvfp4_quantize(g1_inv) -> gemm_swiglu_nvfp4_quant(alpha_gu,
 *          g2_inv) -> nvfp4_gemm(alpha_d) -> out
 *   W4A16: x -> gemm_swiglu(bf16 h, alpha_gu = g_wgu) -> nvfp4_gemm(W4A16,
 *          alpha_d = g_wd) -> out; g1_inv and g2_inv must be NULL.
 *   W4A4_DYN: x -> nvfp4_quantize_per_token -> gemm_swiglu_nvfp4_quant_rowscale(
 *          g_w = alpha_gu = g_wgu, g2_inv) -> nvfp4_gemm(alpha_d) -> out;
 *          g1_inv must be NULL (h keeps its static g2_inv, as on the pages).
 * x bf16 [M, H]; w_gu_packed: SWIGLU packed [2I, H]; w_d_packed: PLAIN packed
 * [H, I]; H % 256 == 0, I % 256 == 0. out [M, H] of out_dtype.
 * W4A4 and W4A16 at M = 1 under NVFP4_PATH_AUTO (and outside stream capture)
 * run as one launch: its workgroups pass h and the down projection's partial
 * sums to each other through 64-bit records in the workspace's tail, each
 * tagged with a 32-bit number new to the call. The tail must therefore hold zeros
 * the first time it is used this way (memory with other contents could hold
 * a current tag by chance). No other call writes the tail, so a workspace
 * stays ready for the next decode whatever calls (of any mode, M, H and I)
 * run in between, as long as every call on the buffer passes the same
 * ws_bytes (the tail is placed from ws + ws_bytes). A wait of that kernel is bounded: if one ever gives up,
 * that unit's rows of out are NaN and NVFP4_STATUS_DECODE_WAIT_EXPIRED is set
 * in the status word. Calls that share a workspace must not overlap (the
 * same holds on every path). Outside the tail the workspace may hold
 * anything: the split-K counters are cleared by the gate_up GEMM's first
 * launch. NVFP4_MODE_W4A16_AWQ is not accepted here (mlp_forward_w4a16_awq
 * takes its scales).
 */
int mlp_forward(int mode, const uint16_t* x, int64_t M, int64_t H, int64_t I,
                const void* w_gu_packed, const float* alpha_gu, const void* w_d_packed,
                const float* alpha_d, const float* g1_inv, const float* g2_inv, void* ws,
                size_t ws_bytes, void* out, int out_dtype, void* stream);

/*
 * mlp_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The workspace is the library's own scratch array:
 * one static device array of NVFP4_NOALLOC_SCRATCH_BYTES per GPU, held from
 * the library's first use on that GPU until the process ends, its address
 * taken once per device (hipGetSymbolAddress). Nothing is allocated per call.
 * Arguments and results as mlp_forward. Limit: the workspace the call's
 * kernel path needs (activations, split-K partials and the 4 MiB tail, as
 * mlp_workspace_bytes counts them for that path) must fit the scratch; a
 * larger call is NVFP4_ERR_INVALID_ARG with nothing launched. At hidden 5120
 * (intermediate 17408) and 7168 (18432) this covers every token count up to
 * 256 in the W4A4 modes and up to 768 in W4A16.
 * Every call on one GPU shares that GPU's scratch and leaves its contents
 * there: calls that overlap in time on one GPU (on different streams, or
 * from different threads) race and give wrong results; serialize them. The
 * scratch's tail is cleared once, by a fill kernel on the stream of the
 * first call on each device. Its status word is not exposed.
 */
#define NVFP4_NOALLOC_SCRATCH_BYTES (64u << 20)
int mlp_forward_noalloc(int mode, const uint16_t* x, int64_t M, int64_t H, int64_t I,
                        const void* w_gu_packed, const float* alpha_gu, const void* w_d_packed,
                        const float* alpha_d, const float* g1_inv, const float* g2_inv, void* out,
                        int out_dtype, void* stream);

/*
 * Standalone SiLU(gate) * up + NVFP4 quantization of a bf16 gate_up output
 * batched by expert, `silu_and_mul_scaled_nvfp4_experts_quantize(gate_up,
 * masked_m, input_scale_inv)` as the PR #34859 digest calls it (key source
 * snippets, qwen2_moe.py `_silu_fp4_quant_fused`, with one expert for a dense
 * MLP): for expert e and row t < masked_m[e]
 *   h = SiLU(gate) * up in fp32 (gate = first I columns of the row),
 *   codes/scales of the row = NVFP4(h) with g_inv[e] as nvfp4_quantize does.
 * gate_up: bf16 [E, M, 2I] row-major, 16-byte aligned, I % 16 == 0.
 * masked_m: device int32 [E], rows of expert e to process (clamped to
 *   [0, M]); NULL processes all M rows of every expert.
 * g_inv: device fp32 [E], inverse global scale per expert.
 * codes: [E, M, I/2] out (16-byte aligned); scales: [E, M, I/16] out
 *   (linear, one E4M3 byte per 16 elements). Rows past masked_m[e] are not
 *   written. Errors: NVFP4_ERR_INVALID_ARG for bad sizes, alignment or null
 *   pointers (nothing launched).
 */
int silu_mul_nvfp4_quant(const void* gate_up, int64_t E, int64_t M, int64_t I, const int32_t* masked_m,
                         const float* g_inv, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * Grouped (expert) NVFP4 GEMM with masked rows, the per-expert GEMMs of the
 * MoE path (PR #35120 report, implementation breakdown item 3; `masked_m` as
 * in the PR #34859 digest, qwen2_moe.py `_silu_fp4_quant_fused`). Routing
 * is not part of it. For expert e and row t < clamp(masked_m[e], 0, M):
 *   out[e, t, :] = alpha[e] * a[e, t, :] @ W_e^T   (as nvfp4_gemm in `mode`)
 * a: W4A4 codes [E, M, K/2] with a_scales [E, M, K/16]; W4A16 bf16 [E, M, K]
 *   (a_scales NULL).
 * w_packed: E packed PLAIN weights [N, K] back to back, each
 *   nvfp4_repack_bytes(NVFP4_REPACK_PLAIN, N, K) bytes.
 * masked_m: device int32 [E] (NULL: every row valid); alpha: device fp32 [E].
 * out: [E, M, N] of out_dtype; rows past masked_m[e] are not written.
 * All experts run in one launch (0 <= E <= 65535). Under NVFP4_PATH_AUTO:
 * W4A4 on the mid-size kernel from 64 to 512 tokens per expert (M),
 * otherwise the weight-streaming kernel up to 256 tokens and the tiled
 * kernel above; NVFP4_PATH_STREAM / _TILED / _MID (W4A4) force one. Every
 * workgroup reads its expert's row count on the device. Errors as nvfp4_gemm;
 * NVFP4_ERR_UNSUPPORTED when one expert's operands reach 2^31 bytes.
 */
int nvfp4_grouped_gemm(int mode, const void* a, const uint8_t* a_scales, const void* w_packed, int64_t E,
                       int64_t M, int64_t N, int64_t K, const int32_t* masked_m, const float* alpha, void* out,
                       int out_dtype, void* stream);

/*
 * AWQ pre-quant scaling of a W4A16 layer's bf16 input: the W4A16 branch of
 * a linear layer's apply multiplies its input by the layer's per-input-
 * channel `pre_quant_scale` before the W4A16 GEMM (PR #35120 report,
 * implementation breakdown item 2):
 *   out[m, k] = bf16(x[m, k] * s[k])   (exact fp32 product, rounded to nearest even)
 * x, out: bf16 [M, K] (out may be x); s: bf16 [K]; K % 8 == 0, M <= 2^24,
 * K <= 2^30; all 16-byte
 * aligned. Feed out to nvfp4_gemm(NVFP4_MODE_W4A16, ...).
 */
int nvfp4_prescale_bf16(const void* x, const void* s, int64_t M, int64_t K, void* out, void* stream);

/*
 * W4A16 MLP forward with AWQ pre-quant scales on the inputs of both GEMMs
 * (the same reading applied to the gate_up layer and the down layer):
 *   x' = bf16(x * s_gu);  h = bf16(SiLU(gate) * up) of the W4A16 gate_up of x';
 *   h' = bf16(h * s_d);   out = W4A16 down projection of h'.
 * As mlp_forward(NVFP4_MODE_W4A16, ...) otherwise (g_gu, g_d: the weights'
 * global scales as alpha). s_gu: bf16 [H]; s_d: bf16 [I]; both 16-byte
 * aligned device memory. Workspace: mlp_workspace_bytes(NVFP4_MODE_W4A16_AWQ,
 * M, H, I) (it also holds x'). x' is one more launch before the gate_up GEMM;
 * h' is applied in the gate_up epilogue.
 */
int mlp_forward_w4a16_awq(const uint16_t* x, int64_t M, int64_t H, int64_t I, const void* w_gu_packed,
                          const float* g_gu, const uint16_t* s_gu, const void* w_d_packed, const float* g_d,
                          const uint16_t* s_d, void* ws, size_t ws_bytes, void* out, int out_dtype, void* stream);

/* Test hook for the bounded waits of the single-launch decodes (mlp_forward,
 * W4A4 or W4A16, M = 1), for calls from the calling thread: with withhold != 0 its
 * workgroups tag their records with a number the waiting workgroups never
 * look for, and each wait gives up after spin_limit polls, so every wait
 * expires, sets NVFP4_STATUS_DECODE_WAIT_EXPIRED and writes NaN, and every
 * workgroup still exits. withhold = 0 restores normal operation. Returns
 * NVFP4_OK, or NVFP4_ERR_INVALID_ARG for spin_limit < 1 with withhold set. */
int nvfp4_set_decode_wait_test(int withhold, int spin_limit);

/* Select the kernel class used by the GEMM entry points (NVFP4_PATH_*) for
 * calls made from the calling thread (each thread starts at
 * NVFP4_PATH_AUTO); meant for tests and benchmarks. Returns the previous
 * value, or NVFP4_ERR_INVALID_ARG. */
int nvfp4_set_path(int path);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_MI355X_H_ */
