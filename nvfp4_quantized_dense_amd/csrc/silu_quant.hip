// silu_quant.hip -- standalone SiLU(gate) * up + NVFP4 quantization of a
// bf16 gate_up output batched by expert (the fused activation + quantize
// call that feeds a down projection taking pre-quantized input, PR #34859
// digest, qwen2_moe.py `_silu_fp4_quant_fused`).
//
// HBM-bound elementwise work (per output element 4 bytes read, 0.5625
// written): one thread per 8 outputs of a row, reading the matching 16-byte
// chunks of the gate and up halves; chunks 2b and 2b + 1 (neighbouring
// lanes) form 16-block b and exchange their amax. The SiLU * mul and the
// block encoder are the ones of the fused GEMM epilogue (silu_mul,
// block_scale, e2m1_pack8), so the codes match the fused path's for the
// same fp32 h. Rows past masked_m are skipped by whole workgroups.
#include "device_common.h"
#include "kernels.h"


namespace nvfp4 {

// One 8-output chunk: SiLU * mul of its gate and up words, the 16-block
// exchange with the neighbouring lane, the encoding and the stores.
__device__ __forceinline__ void silu_quant_chunk(const u32x4& gw, const u32x4& uw, bool live, float gi,
                                                 uint32_t* codes, uint8_t* scales, int64_t c) {
  float h[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[2 * i] = live ? silu_mul(__uint_as_float(gw[i] << 16), __uint_as_float(uw[i] << 16)) : 0.0f;
    h[2 * i + 1] =
        live ? silu_mul(__uint_as_float(gw[i] & 0xFFFF0000u), __uint_as_float(uw[i] & 0xFFFF0000u)) : 0.0f;
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(h[i]) & 0x7FFFFFFFu);
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  const BlockScale bs = block_scale(__uint_as_float(m), gi);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = h[i] * bs.r;
  const uint32_t packed = e2m1_pack8(y);
  if (live) {
    codes[c] = packed;
    if ((c & 1) == 0) scales[c >> 1] = (uint8_t)bs.byte;
  }
}

// grid (ceil(I / 8 / (256 U)), M, E); row t of expert e. Each thread takes
// U chunks 256 apart (every lane pair stays a block), all loads issued
// before the arithmetic.
template <int U>
__global__ __launch_bounds__(256) void k_silu_mul_quant(const uint32_t* __restrict__ gate_up, int64_t M,
                                                        int64_t I, const int32_t* __restrict__ masked_m,
                                                        const float* __restrict__ g_inv,
                                                        uint32_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int64_t e = blockIdx.z, t = blockIdx.y;
  if (masked_m != nullptr && t >= (int64_t)masked_m[e]) return;
  const int64_t n8 = I / 8;
  const int64_t row = e * M + t;
  const float gi = g_inv[e];
  // bf16 pairs as 32-bit words: the row holds 2I bf16 = I words, gate first.
  const u32x4* gp = reinterpret_cast<const u32x4*>(gate_up + row * I);
  const u32x4* up = reinterpret_cast<const u32x4*>(gate_up + row * I + I / 2);
  const int64_t c0 = (int64_t)blockIdx.x * 256 * U + threadIdx.x;
  u32x4 gw[U], uw[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t c = c0 + 256 * k;
    if (c < n8) {
      gw[k] = __builtin_nontemporal_load(gp + c);
      uw[k] = __builtin_nontemporal_load(up + c);
    } else {
      gw[k] = uw[k] = u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t c = c0 + 256 * k;
    silu_quant_chunk(gw[k], uw[k], c < n8, gi, codes + row * n8, scales + row * (I / 16), c);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// Chunks per thread: 1, 2, 4 and 8 measured 194, 179, 182 and 303 us on
// 8192 rows of 18432 outputs (with the exact SiLU, when the arithmetic was
// the limit).
constexpr int kSiluU = 2;

hipError_t launch_silu_mul_quant(const void* gate_up, int64_t E, int64_t M, int64_t I, const int32_t* masked_m,
                                 const float* g_inv, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (E == 0 || M == 0 || I == 0) return hipSuccess;
  const dim3 grid((unsigned)((I / 8 + 256 * kSiluU - 1) / (256 * kSiluU)), (unsigned)M, (unsigned)E);
  k_silu_mul_quant<kSiluU><<<grid, 256, 0, s>>>(reinterpret_cast<const uint32_t*>(gate_up), M, I, masked_m,
                                                g_inv, reinterpret_cast<uint32_t*>(codes), scales);
  return hipGetLastError();
}

}  // namespace nvfp4
