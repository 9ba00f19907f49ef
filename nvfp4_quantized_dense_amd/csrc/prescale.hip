// prescale.hip -- AWQ pre-quant scaling of a W4A16 layer's bf16 input
// (the W4A16 branch of a linear layer's apply pre-scales its input by the
// layer's per-input-channel pre_quant_scale before the W4A16 GEMM, PR #35120
// report, implementation breakdown item 2): out = bf16(x * s), the fp32
// product of two bf16 values being exact and the conversion rounding to
// nearest even. HBM-bound: one thread per 8 elements (16-byte accesses).
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

__global__ __launch_bounds__(256) void k_prescale_bf16(const u32x4* __restrict__ x, const u32x4* __restrict__ s,
                                                       int64_t n8, int64_t k8, u32x4* __restrict__ out) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const u32x4 xv = x[i], sv = s[i % k8];
  u32x4 o;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float lo = __uint_as_float(xv[w] << 16) * __uint_as_float(sv[w] << 16);
    const float hi = __uint_as_float(xv[w] & 0xFFFF0000u) * __uint_as_float(sv[w] & 0xFFFF0000u);
    const __bf16 bl = (__bf16)lo, bh = (__bf16)hi;
    o[w] = (uint32_t)__builtin_bit_cast(uint16_t, bl) | ((uint32_t)__builtin_bit_cast(uint16_t, bh) << 16);
  }
  out[i] = o;
#endif  // __HIP_DEVICE_COMPILE__
}

hipError_t launch_prescale_bf16(const void* x, const void* s, int64_t M, int64_t K, void* out, hipStream_t st) {
  const int64_t n8 = M * K / 8;
  if (n8 == 0) return hipSuccess;
  k_prescale_bf16<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(
      reinterpret_cast<const u32x4*>(x), reinterpret_cast<const u32x4*>(s), n8, K / 8, reinterpret_cast<u32x4*>(out));
  return hipGetLastError();
}

}  // namespace nvfp4
