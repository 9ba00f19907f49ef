// kernels.h -- host-side launchers of the HIP kernels (internal interface
// between the C ABI layer and the kernel translation units). Every launcher
// assumes its arguments were validated by the caller and only launches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

enum Mode : int { kW4A4 = 0, kW4A16 = 1 };
// GEMM epilogues: dense output of alpha * acc, or SwiGLU of a gate/up group
// pair written as NVFP4 codes + scales, bf16 or f32.
enum Epi : int { kOutF32 = 0, kOutBF16 = 1, kSwigluNvfp4 = 2, kSwigluBF16 = 3, kSwigluF32 = 4 };

// quantize.hip
hipError_t launch_calibrate(const void* x, bool f32_in, int64_t n, float* g, float* g_inv,
                            hipStream_t s);
hipError_t launch_quantize(const void* x, bool f32_in, int64_t M, int64_t K, const float* g_inv,
                           uint8_t* codes, uint8_t* scales, hipStream_t s);
// Per-token dynamic quantization: each row calibrated on its own amax
// (g_t = amax_t / 2688, g_inv_t = 1 / g_t, 0 for a zero row) and quantized
// with g_inv_t; row_g[t] = g_t.
hipError_t launch_quantize_per_token(const void* x, bool f32_in, int64_t M, int64_t K, uint8_t* codes,
                                     uint8_t* scales, float* row_g, hipStream_t s);

// silu_quant.hip: SiLU(gate) * up of a bf16 gate_up [E, M, 2I] quantized
// to NVFP4 with g_inv[e], rows t < masked_m[e] (all rows if masked_m is
// null); grid (I / 2048, M, E) within the launch limits (M, E < 65536).
hipError_t launch_silu_mul_quant(const void* gate_up, int64_t E, int64_t M, int64_t I, const int32_t* masked_m,
                                 const float* g_inv, uint8_t* codes, uint8_t* scales, hipStream_t s);

// prescale.hip: AWQ pre-quant scaling out[m, k] = bf16(x[m, k] * s[k]) of
// bf16 x [M, K], K % 8 == 0 (out may be x).
hipError_t launch_prescale_bf16(const void* x, const void* s, int64_t M, int64_t K, void* out, hipStream_t st);

// repack.hip
hipError_t launch_repack(int kind, const uint8_t* codes, const uint8_t* scales, int64_t R,
                         int64_t C, uint8_t* packed, bool unpack, uint8_t* out_codes,
                         uint8_t* out_scales, hipStream_t s);

// Arguments shared by the GEMM-class kernels.
struct GemmArgs {
  const void* a;             // W4A4: codes [M, K/2]; W4A16: bf16 [M, K]
  const uint8_t* a_scales;   // W4A4: [M, K/16]
  const uint8_t* w;          // packed weight
  int64_t M;                 // tokens
  int64_t N;                 // packed weight rows (2I for the SwiGLU kinds)
  int64_t K;
  const float* alpha;
  const float* g2_inv;       // SwiGLU + NVFP4 output only
  void* out;                 // [M, N] dense, or h [M, I] (dense or codes)
  uint8_t* out_scales;       // h scales [M, I/16]
  // Split-K (weight-streaming and mid-size kernels: dense epilogues; tiled
  // kernels: any epilogue, on the tiles their launcher splits): ksplit > 1
  // divides the K
  // tiles over that many workgroups per output tile. Each workgroup stores
  // its partial result tile to part (split tile u, split s at
  // ((u * ksplit + s) * tile_floats)); the last of the ksplit workgroups of
  // a tile to finish (counted in counters[u], which must be zero at launch
  // and are left zero) adds the partials in split order and runs the
  // epilogue.
  float* part = nullptr;
  uint32_t* counters = nullptr;
  int ksplit = 1;
  // Words that workgroup (0, 0, 0) clears before its own work (the split-K
  // counters of the GEMM launched next on the same stream).
  uint32_t* zero_ptr = nullptr;
  int zero_n = 0;
  // Per-token dynamic activation scales (W4A4): when set, token t's output
  // is scaled by alpha * row_scale[t] (row_scale[t] = the token's global
  // scale, alpha = the weight's).
  const float* row_scale = nullptr;
  // Grouped (expert) GEMMs: when set, only the first clamp(*m_dev, 0, M)
  // token rows are valid (read as zeros past them, never stored); a
  // workgroup with no valid row exits at once. Weight-streaming and tiled
  // kernels, ksplit = 1.
  const int32_t* m_dev = nullptr;
  // Grouped (expert) GEMMs in one launch of the weight-streaming kernel:
  // when experts > 1, blockIdx.z is the expert e, and a, a_scales, w and
  // out advance by e times these byte strides, alpha and m_dev by e
  // elements (unsplit: ksplit = 1).
  int experts = 0;
  int64_t e_a = 0, e_as = 0, e_w = 0, e_out = 0;
  // W4A16 SwiGLU epilogue with bf16 h: when set, h is multiplied by the
  // next layer's AWQ pre-quant scale (bf16 [I]) and rounded again to bf16.
  const uint16_t* h_prescale = nullptr;
  // W4A4 decode GEMV with the SwiGLU-NVFP4 epilogue at M = 1 only: when
  // set, `a` is bf16 [M, K] and each workgroup quantizes it to NVFP4 with
  // this global scale inverse as it stages it (the same arithmetic as
  // launch_quantize); a_scales is unused.
  const float* a_g_inv = nullptr;
};

// Split-K is valid with the buffers given and every split non-empty: tiles
// per split ceil(T / ksplit), (ksplit - 1) of them fewer than T; for the
// dense epilogues, or any epilogue where the kernel combines the partial
// sums before it (the tiled kernels: swiglu_ok).
inline bool splitk_valid(const GemmArgs& a, int epi, bool swiglu_ok = false) {
  if (a.ksplit == 1) return true;
  const int64_t T = a.K / 256, per = (T + a.ksplit - 1) / a.ksplit;
  return a.ksplit > 1 && (swiglu_ok || epi == kOutF32 || epi == kOutBF16) && a.part && a.counters &&
         (a.ksplit - 1) * per < T;
}
// Launch shape of the weight-streaming kernel's dense GEMM: output tiles
// (workgroups before any K split), floats of one partial result tile, waves
// per workgroup.
struct TileShape {
  int64_t units, tile_floats, waves;
};
TileShape stream_shape(int mode, int64_t M, int64_t N);
TileShape tiled16_shape(int64_t M, int64_t N);
TileShape mid_shape(int mode, int64_t M, int64_t N);  // dense epilogue, one expert

// The number of K splits that brings a dense GEMM of `units` output tiles to
// about `target` workgroups, each split keeping at least `min_tiles` tiles.
inline int splitk_ways(int64_t units, int64_t T, int64_t target, int64_t min_tiles) {
  int64_t ks = units >= target ? 1 : (target + units - 1) / units;
  if (ks > 8) ks = 8;
  while (ks > 1 && ((ks - 1) * ((T + ks - 1) / ks) >= T || (T + ks - 1) / ks < min_tiles)) --ks;
  return (int)ks;
}

// epi: Epi enum of device_common.h; mode: Mode enum.
hipError_t launch_stream_gemm(int mode, int epi, const GemmArgs& a, hipStream_t s);
// Its one-token-group launches (W4A4 up to 16 tokens, W4A16 at any count),
// stream_nt1.hip.
hipError_t launch_stream_nt1(int mode, int epi, const GemmArgs& a, hipStream_t s);
// LDS the W4A16 GEMV may stage token rows in (one row of K bf16 at least).
constexpr int64_t kValuGemvLdsBytes = 65536;
hipError_t launch_valu_gemv(int mode, int epi, const GemmArgs& a, hipStream_t s);
// LDS the W4A4 GEMV stages its token rows in: with up to 2 rows per
// workgroup, the codes, scales and a zero region of K / 2 bytes.
constexpr int64_t kFp4GemvLdsBytes = 65536;
bool fp4_gemv_supported(int64_t M, int64_t K);
hipError_t launch_fp4_gemv(int epi, const GemmArgs& a, hipStream_t s);
hipError_t launch_tiled_gemm(int mode, int epi, const GemmArgs& a, hipStream_t s);
// mid.hip: the W4A4 mid-size kernel (unsplit, one expert).
bool mid_supported(const GemmArgs& a);
hipError_t launch_mid_gemm(int mode, int epi, const GemmArgs& a, hipStream_t s);

// The tiled kernels run one workgroup per CU, so output tiles go in rounds
// of kTiledSlots; tiled_tail(units) is the tile count of the last, partial
// round of a grid of more than one round (0 if none).
constexpr int64_t kTiledSlots = 256;
inline int64_t tiled_tail(int64_t units) { return units > kTiledSlots ? units % kTiledSlots : 0; }

// W4A4 only; packed weight, activation codes and scales each < 2^31 bytes.
// With ksplit > 1: a grid of less than one round (dense epilogues) splits
// every tile; a larger one splits only its tiled_tail tiles (any epilogue:
// the partials are combined before it). part and counters are sized for
// the split tiles.
hipError_t launch_tiled2_gemm(int epi, const GemmArgs& a, hipStream_t s);
TileShape tiled2_shape(int64_t M, int64_t N);
// W4A16 only; packed weight and the activation rows (+256 of padding) each
// < 2^31 bytes. With ksplit > 1: a grid of less than one round (dense
// epilogues) splits every tile; a larger one splits only its tiled_tail
// tiles (any epilogue). part and counters are sized for the split tiles.
hipError_t launch_tiled16_gemm(int epi, const GemmArgs& a, hipStream_t s);

// decode.hip: the W4A4 MLP forward of one token in one launch (gate_up
// units hand h to the down units, and those their partial sums to the last
// K split, as 64-bit records tagged with the launch's epoch).
constexpr int kDecodeMaxSplits = 8;
struct DecodeArgs {
  const void* x;          // bf16 [1, H]
  const float* g1_inv;    // global scale inverse of x
  const uint8_t* w_gu;    // SWIGLU packed [2I, H]
  const uint8_t* w_d;     // PLAIN packed [H, I]
  const float* alpha_gu;
  const float* alpha_d;
  const float* g2_inv;    // global scale inverse of h
  uint8_t* h_codes;       // [I / 2], written (as by the two-launch path)
  uint8_t* h_scales;      // [I / 16], written
  void* out;              // [1, H], f32 or bf16
  uint64_t* records;      // decode_record_words(H, I) words: zeros or left by earlier launches
  int64_t H, I;
  int ksplit;             // decode_splits(H, I), or another count the launcher accepts
  uint64_t epoch;         // low 32 bits nonzero, differing from the last 2^32 - 1 launches' on records
  uint32_t* status;       // OR-ed with kDecodeWaitExpired by a unit whose bounded wait gave up
  int spin_limit;         // polls of one wait before it gives up (kDecodeSpinLimit)
  uint32_t tag_skew;      // 0; nonzero only to test the expired wait: producers then tag their
                          // records (epoch ^ tag_skew), which no consumer waits for
};
constexpr uint32_t kDecodeWaitExpired = 1;
constexpr int kDecodeSpinLimit = 1 << 20;
bool decode_supported(int64_t H, int64_t I);
int decode_splits(int64_t H, int64_t I);
int64_t decode_record_words(int64_t H, int64_t I);
hipError_t launch_decode_mlp(int epi, const DecodeArgs& d, hipStream_t s);

// decode16.hip: the W4A16 MLP forward of one token in one launch (gate_up
// units hand the bf16 h to the down units, and those their partial sums to
// the last K split, as tagged records, as in decode.hip).
struct Decode16Args {
  const void* x;          // bf16 [1, H]
  const uint8_t* w_gu;    // SWIGLU packed [2I, H]
  const uint8_t* w_d;     // PLAIN packed [H, I]
  const float* alpha_gu;  // g of the gate_up weight
  const float* alpha_d;   // g of the down weight
  uint16_t* h;            // bf16 [I], written (as by the two-launch path)
  void* out;              // [1, H], f32 or bf16
  uint64_t* records;      // decode16_record_words(H, I) words: zeros or left by earlier launches
  int64_t H, I;
  int ksplit;             // decode16_splits(H, I)
  uint64_t epoch;         // as DecodeArgs::epoch
  uint32_t* status;       // OR-ed with kDecodeWaitExpired by a unit whose bounded wait gave up
  int spin_limit;         // polls of one wait before it gives up
  uint32_t tag_skew;      // as DecodeArgs::tag_skew
};
bool decode16_supported(int64_t H, int64_t I);
int decode16_splits(int64_t H, int64_t I);
int64_t decode16_record_words(int64_t H, int64_t I);
hipError_t launch_decode_mlp16(int epi, const Decode16Args& d, hipStream_t s);

}  // namespace nvfp4
