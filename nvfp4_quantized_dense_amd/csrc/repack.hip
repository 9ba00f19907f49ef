// repack.hip -- one-time permutation of canonical NVFP4 weights (codes
// [R, C/2], scales [R, C/16]) into the packed tile layout the GEMM kernels
// stream, and its inverse.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

// Canonical row held by packed row r of row group g. PLAIN: identity.
// SWIGLU: groups alternate gate group p (rows 16p..) and up group p (rows
// I + 16p..), I = R / 2.
template <int KIND>
__device__ __forceinline__ int64_t src_row(int64_t g, int r, int64_t R) {
  if constexpr (KIND == 0) {
    return g * kTileRows + r;
  } else {
    return (g & 1) * (R / 2) + (g >> 1) * kTileRows + r;
  }
}

// One thread per (tile, lane): copies the lane's two 16-byte code chunks and
// four scale bytes between the canonical and packed layouts.
template <int KIND, bool UNPACK>
__global__ __launch_bounds__(256) void k_repack(const uint8_t* __restrict__ codes,
                                                const uint8_t* __restrict__ scales, int64_t R,
                                                int64_t C, uint8_t* __restrict__ packed,
                                                uint8_t* __restrict__ out_codes,
                                                uint8_t* __restrict__ out_scales) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t T = C / kTileK;
  const int64_t ntiles = (R / kTileRows) * T;
  if (gid >= ntiles * 64) return;
  const int64_t tile = gid >> 6;
  const int lane = (int)(gid & 63);
  const int64_t g = tile / T, t = tile % T;
  const int64_t row = src_row<KIND>(g, lane & 15, R);
  const int q = lane >> 4;
  uint8_t* tp = packed + tile * kTileBytes;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int64_t src = row * (C / 2) + t * 128 + c * 64 + q * 16;
    u32x4* dst = reinterpret_cast<u32x4*>(tp + c * 1024 + 16 * lane);
    if constexpr (UNPACK) {
      *reinterpret_cast<u32x4*>(out_codes + src) = *dst;
    } else {
      *dst = *reinterpret_cast<const u32x4*>(codes + src);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t ssrc = row * (C / 16) + t * 16 + c * 8 + q * 2 + b;
      uint8_t* sdst = tp + kTileCodeBytes + 4 * lane + 2 * c + b;
      if constexpr (UNPACK) out_scales[ssrc] = *sdst;
      else *sdst = scales[ssrc];
    }
  }
}

hipError_t launch_repack(int kind, const uint8_t* codes, const uint8_t* scales, int64_t R,
                         int64_t C, uint8_t* packed, bool unpack, uint8_t* out_codes,
                         uint8_t* out_scales, hipStream_t s) {
  const int64_t threads = (R / kTileRows) * (C / kTileK) * 64;
  if (threads == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (kind == 0) {
    if (unpack) k_repack<0, true><<<blocks, 256, 0, s>>>(codes, scales, R, C, packed, out_codes, out_scales);
    else k_repack<0, false><<<blocks, 256, 0, s>>>(codes, scales, R, C, packed, out_codes, out_scales);
  } else {
    if (unpack) k_repack<1, true><<<blocks, 256, 0, s>>>(codes, scales, R, C, packed, out_codes, out_scales);
    else k_repack<1, false><<<blocks, 256, 0, s>>>(codes, scales, R, C, packed, out_codes, out_scales);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
