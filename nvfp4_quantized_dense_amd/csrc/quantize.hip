// quantize.hip -- NVFP4 activation/weight quantization and per-tensor
// calibration of the global scale.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

// One thread per 8 consecutive elements; the two threads of a 16-element
// block are neighbouring lanes and exchange their partial amax. K % 16 == 0
// keeps every block inside one row, so the flat index is all that is needed.
template <bool F32_IN>
__global__ __launch_bounds__(256) void k_quantize(const void* __restrict__ x, int64_t n8,
                                                  const float* __restrict__ g_inv_p,
                                                  uint32_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = t < n8;
  float v[8];
  if (live) {
    if constexpr (F32_IN) {
      const f32x4* p = reinterpret_cast<const f32x4*>(x) + 2 * t;
      f32x4 a = __builtin_nontemporal_load(p);
      f32x4 b = __builtin_nontemporal_load(p + 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
    } else {
      u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + t);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(a[i] << 16);
        v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  // amax over the block: |x| as bits compares like the value (no NaN).
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  const BlockScale bs = block_scale(__uint_as_float(m), *g_inv_p);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = v[i] * bs.r;
  const uint32_t packed = e2m1_pack8(y);
  if (live) {
    codes[t] = packed;
    if ((t & 1) == 0) scales[t >> 1] = (uint8_t)bs.byte;
  }
}

// Per-token dynamic quantization: one workgroup per row. The row's amax
// (bits of |x| compare like the values), g = amax / 2688 and g_inv = 1 / g
// (0 for a zero row) as k_finalize_scale computes them, then the row is
// quantized exactly as k_quantize does with that g_inv; row_g[row] = g.
template <bool F32_IN>
__global__ __launch_bounds__(256) void k_quantize_per_token(const void* __restrict__ x, int64_t K,
                                                            uint32_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            float* __restrict__ row_g) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t n8 = K / 8;
  auto load8 = [&](int64_t c, float (&v)[8]) {
    if constexpr (F32_IN) {
      const f32x4* p = reinterpret_cast<const f32x4*>(x) + 2 * (row * n8 + c);
      const f32x4 a = p[0], b = p[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
    } else {
      const u32x4 a = reinterpret_cast<const u32x4*>(x)[row * n8 + c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(a[i] << 16);
        v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
      }
    }
  };
  uint32_t m = 0;
  for (int64_t c = tid; c < n8; c += 256) {
    float v[8];
    load8(c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  __shared__ uint32_t wmax[4];
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float g = __uint_as_float(m) / 2688.0f;
  const float g_inv = g != 0.0f ? 1.0f / g : 0.0f;
  if (tid == 0) row_g[row] = g;
  // Quantize: chunks c and c ^ 1 (neighbouring lanes, 256 is even) form a block.
  for (int64_t c = tid; c < n8; c += 256) {
    float v[8];
    load8(c, v);
    uint32_t bm = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) bm = max(bm, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    bm = max(bm, (uint32_t)__shfl_xor((int)bm, 1));
    const BlockScale bs = block_scale(__uint_as_float(bm), g_inv);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = v[i] * bs.r;
    const uint32_t packed = e2m1_pack8(y);
    codes[row * n8 + c] = packed;
    if ((c & 1) == 0) scales[row * (K / 16) + (c >> 1)] = (uint8_t)bs.byte;
  }
}

__global__ void k_fill_u32(uint32_t* p, uint32_t v) { *p = v; }

// Grid-stride max of |x| into a 32-bit cell (bits of a non-negative float
// order like their values).
template <bool F32_IN>
__global__ __launch_bounds__(256) void k_amax(const void* __restrict__ x, int64_t n,
                                              uint32_t* __restrict__ cell) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    uint32_t b;
    if constexpr (F32_IN) {
      b = __float_as_uint(reinterpret_cast<const float*>(x)[i]) & 0x7FFFFFFFu;
    } else {
      b = ((uint32_t)reinterpret_cast<const uint16_t*>(x)[i] & 0x7FFFu) << 16;
    }
    m = max(m, b);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if ((threadIdx.x & 63) == 0) atomicMax(cell, m);
}

// g = fl(amax / 2688), g_inv = fl(1 / g); the cell aliases g.
__global__ void k_finalize_scale(float* g, float* g_inv) {
  float amax = __uint_as_float(*reinterpret_cast<uint32_t*>(g));
  float gg = amax / 2688.0f;
  *g = gg;
  *g_inv = 1.0f / gg;
}

hipError_t launch_calibrate(const void* x, bool f32_in, int64_t n, float* g, float* g_inv,
                            hipStream_t s) {
  uint32_t* cell = reinterpret_cast<uint32_t*>(g);
  k_fill_u32<<<1, 1, 0, s>>>(cell, 0u);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  if (f32_in) k_amax<true><<<(unsigned)blocks, 256, 0, s>>>(x, n, cell);
  else k_amax<false><<<(unsigned)blocks, 256, 0, s>>>(x, n, cell);
  k_finalize_scale<<<1, 1, 0, s>>>(g, g_inv);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, bool f32_in, int64_t M, int64_t K, const float* g_inv,
                           uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t n8 = M * K / 8;
  if (n8 == 0) return hipSuccess;
  const int64_t blocks = (n8 + 255) / 256;
  uint32_t* c32 = reinterpret_cast<uint32_t*>(codes);
  if (f32_in) k_quantize<true><<<(unsigned)blocks, 256, 0, s>>>(x, n8, g_inv, c32, scales);
  else k_quantize<false><<<(unsigned)blocks, 256, 0, s>>>(x, n8, g_inv, c32, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_per_token(const void* x, bool f32_in, int64_t M, int64_t K, uint8_t* codes,
                                     uint8_t* scales, float* row_g, hipStream_t s) {
  if (M == 0 || K == 0) return hipSuccess;
  uint32_t* c32 = reinterpret_cast<uint32_t*>(codes);
  if (f32_in) k_quantize_per_token<true><<<(unsigned)M, 256, 0, s>>>(x, K, c32, scales, row_g);
  else k_quantize_per_token<false><<<(unsigned)M, 256, 0, s>>>(x, K, c32, scales, row_g);
  return hipGetLastError();
}

}  // namespace nvfp4
