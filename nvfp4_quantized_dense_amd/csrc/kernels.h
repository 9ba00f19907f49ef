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
};

// epi: Epi enum of device_common.h; mode: Mode enum.
hipError_t launch_stream_gemm(int mode, int epi, const GemmArgs& a, hipStream_t s);
// LDS the W4A16 GEMV may stage token rows in (one row of K bf16 at least).
constexpr int64_t kValuGemvLdsBytes = 65536;
hipError_t launch_valu_gemv(int mode, int epi, const GemmArgs& a, hipStream_t s);
// LDS the W4A4 GEMV stages its token rows in: with up to 2 rows per
// workgroup, the codes, scales and a zero region of K / 2 bytes.
constexpr int64_t kFp4GemvLdsBytes = 65536;
bool fp4_gemv_supported(int64_t M, int64_t K);
hipError_t launch_fp4_gemv(int epi, const GemmArgs& a, hipStream_t s);
hipError_t launch_tiled_gemm(int mode, int epi, const GemmArgs& a, hipStream_t s);
// W4A4 only; packed weight, activation codes and scales each < 2^31 bytes.
hipError_t launch_tiled2_gemm(int epi, const GemmArgs& a, hipStream_t s);

}  // namespace nvfp4
