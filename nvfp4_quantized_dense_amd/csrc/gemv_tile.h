// gemv_tile.h -- building blocks of the W4A16 VALU GEMV (used by gemv.hip
// and by the single-launch W4A16 decode MLP in decode16.hip).
//
// The weight streams with 16-byte loads; the arithmetic is on the vector ALU
// with packed dot products: codes are widened exactly (E2M1 -> bf16, two per
// instruction), multiplied against the bf16 activation pairs with
// v_dot2_f32_bf16 (products of a grid value and a bf16 value are exact in
// fp32), and each 16-element block sum is scaled once by its E4M3 factor.
// Lane l owns row l % 16 of each row group and columns 32 (l / 16) + [0, 32)
// of each 128-column half tile (the packed layout's lane order).
#pragma once
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

#if defined(__HIP_DEVICE_COMPILE__)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + w.lo * x.lo + w.hi * x.hi with bf16 pairs (v_dot2c_f32_bf16). The
// activation dword passes through an empty asm barrier first: without it the
// compiler has been seen to fold the four dwords of a loaded 16-byte
// activation vector into its first one when they feed this builtin. The
// barrier emits nothing and leaves the instruction's scheduling (and its
// wait states) to the compiler.
__device__ __forceinline__ float dot2_bf16(bf16x2 w, uint32_t x, float acc) {
  asm volatile("" : "+v"(x));
  return __builtin_amdgcn_fdot2_f32_bf16(w, __builtin_bit_cast(bf16x2, x), acc, false);
}

struct GemvSrc {
  Rsrc w, a;
};

// Weight loads of one K tile for one wave: NG row groups.
template <int NG>
struct GemvTile {
  u32x4 wc[NG][2];
  uint32_t wsd[NG];
};

// Tile t of row groups of T tiles (out of range from tile t_end on: zeros,
// no memory access).
template <int NG>
__device__ __forceinline__ void gemv_load(GemvTile<NG>& d, const GemvSrc& src, int64_t rg0,
                                          int T, int t_end, int t, int lane) {
  const uint32_t tw = t < t_end ? (uint32_t)(t * kTileBytes) : kOutOfRange;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint32_t gbase = (uint32_t)((rg0 + g) * T * kTileBytes);
    d.wc[g][0] = bload16_nt(src.w, tw + 16 * lane, gbase);
    d.wc[g][1] = bload16_nt(src.w, tw + 1024 + 16 * lane, gbase);
    d.wsd[g] = bload4_nt(src.w, tw + kTileCodeBytes + 4 * lane, gbase);
  }
}

// Tile t (< T) of one wave. xs: the MT staged token rows, K bf16 each.
template <int NG, int MT>
__device__ __forceinline__ void gemv_compute(float (&acc)[NG][MT], const GemvTile<NG>& d,
                                             const uint8_t* xs, int T, int t, int lane) {
  const int q = lane >> 4;
  const int tc = t;
  float ws[NG][4];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    ws[g][0] = e4m3_to_f32<0>(d.wsd[g]); ws[g][1] = e4m3_to_f32<1>(d.wsd[g]);
    ws[g][2] = e4m3_to_f32<2>(d.wsd[g]); ws[g][3] = e4m3_to_f32<3>(d.wsd[g]);
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    u32x4 xv[MT][4];
    const int tx = (tc * kTileK + c * 128 + q * 32) * 2;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        xv[m][u] = *reinterpret_cast<const u32x4*>(xs + (size_t)m * T * kTileK * 2 + tx + 16 * u);
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        float bs[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) bs[m] = 0.0f;
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
          const int u = 2 * blk + uu;
          const uint32_t v = d.wc[g][c][u];
          bf16x2 w[4];
          w[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 0);
          w[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 1);
          w[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 2);
          w[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 3);
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int p = 0; p < 4; ++p) bs[m] = dot2_bf16(w[p], xv[m][u][p], bs[m]);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[g][m] = __builtin_fmaf(bs[m], ws[g][2 * c + blk], acc[g][m]);
      }
  }
}

#endif  // __HIP_DEVICE_COMPILE__

}  // namespace nvfp4
