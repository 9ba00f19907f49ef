// gemv.hip -- VALU GEMV for the smallest token counts (M <= 4), no MFMA.
//
// The decode fast path streams the packed weight with 16-byte loads and
// does the arithmetic on the vector ALU with packed dot products: codes are
// widened exactly (E2M1 -> f16/bf16, two per instruction), multiplied
// against the activation pairs with v_dot2_f32_{f16,bf16}, and each
// 16-element block sum is scaled once by its E4M3 factor(s). In W4A4 the
// activation codes enter unscaled as well, and the block sum is scaled by
// s_w * s_a (a product of two E4M3 values, exact in fp32); the block sum
// itself, of 16 products of grid values, is exact.
//
// Lane l owns row l % 16 of each row group and columns 32 (l / 16) + [0, 32)
// of each 128-column half tile (the packed layout's lane order); the four
// lanes of a row and the NW waves (which divide the K tiles) are summed at
// the end in a fixed order.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

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

template <int MODE, int EPI, int MT, int NW>
__global__ __launch_bounds__(NW * 64) void k_valu_gemv(GemmArgs args) {
  constexpr int NG = EpiTraits<EPI>::swiglu ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int64_t K = args.K;
  const int64_t T = K / kTileK;
  const int64_t rg0 = (int64_t)blockIdx.x * NG;
  const int64_t tok0 = (int64_t)blockIdx.y * MT;

  int64_t trow[MT];
  bool tvalid[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    tvalid[m] = tok0 + m < args.M;
    trow[m] = tvalid[m] ? tok0 + m : 0;  // rows past M read row 0, then zeroed
  }

  float acc[NG][MT];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[g][m] = 0.0f;

  for (int64_t t = wave; t < T; t += NW) {
    u32x4 wc[NG][2];
    uint32_t wsd[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const uint8_t* tp = args.w + ((rg0 + g) * T + t) * kTileBytes;
      wc[g][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tp + 16 * lane));
      wc[g][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tp + 1024 + 16 * lane));
      wsd[g] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(tp + kTileCodeBytes + 4 * lane));
    }
    float ws[NG][4];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      ws[g][0] = e4m3_to_f32<0>(wsd[g]); ws[g][1] = e4m3_to_f32<1>(wsd[g]);
      ws[g][2] = e4m3_to_f32<2>(wsd[g]); ws[g][3] = e4m3_to_f32<3>(wsd[g]);
    }
    if constexpr (MODE == kW4A4) {
      const uint8_t* ac = reinterpret_cast<const uint8_t*>(args.a);
      u32x4 xc[MT][2];
      float xs[MT][4];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint8_t* row = ac + trow[m] * (K / 2) + t * 128 + q * 16;
        u32x4 c0 = *reinterpret_cast<const u32x4*>(row);
        u32x4 c1 = *reinterpret_cast<const u32x4*>(row + 64);
        const uint8_t* srow = args.a_scales + trow[m] * (K / 16) + t * 16 + q * 2;
        uint32_t sd = (uint32_t)*reinterpret_cast<const uint16_t*>(srow) |
                      ((uint32_t)*reinterpret_cast<const uint16_t*>(srow + 8) << 16);
        const u32x4 z = {0, 0, 0, 0};
        xc[m][0] = tvalid[m] ? c0 : z;
        xc[m][1] = tvalid[m] ? c1 : z;
        sd = tvalid[m] ? sd : 0u;
        xs[m][0] = e4m3_to_f32<0>(sd); xs[m][1] = e4m3_to_f32<1>(sd);
        xs[m][2] = e4m3_to_f32<2>(sd); xs[m][3] = e4m3_to_f32<3>(sd);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          // activation pairs of this block, unscaled
          f16x2 xp[MT][8];
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int uu = 0; uu < 2; ++uu) {
              const uint32_t d = xc[m][c][2 * blk + uu];
              xp[m][4 * uu + 0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0);
              xp[m][4 * uu + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1);
              xp[m][4 * uu + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2);
              xp[m][4 * uu + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3);
            }
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            float bs[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) bs[m] = 0.0f;
#pragma unroll
            for (int uu = 0; uu < 2; ++uu) {
              const uint32_t d = wc[g][c][2 * blk + uu];
              f16x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0);
              f16x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1);
              f16x2 w2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2);
              f16x2 w3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3);
#pragma unroll
              for (int m = 0; m < MT; ++m) {
                bs[m] = __builtin_amdgcn_fdot2(w0, xp[m][4 * uu + 0], bs[m], false);
                bs[m] = __builtin_amdgcn_fdot2(w1, xp[m][4 * uu + 1], bs[m], false);
                bs[m] = __builtin_amdgcn_fdot2(w2, xp[m][4 * uu + 2], bs[m], false);
                bs[m] = __builtin_amdgcn_fdot2(w3, xp[m][4 * uu + 3], bs[m], false);
              }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
              acc[g][m] = __builtin_fmaf(bs[m], ws[g][2 * c + blk] * xs[m][2 * c + blk], acc[g][m]);
          }
        }
    } else {
      const uint16_t* xa = reinterpret_cast<const uint16_t*>(args.a);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 xv[MT][4];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const u32x4* row = reinterpret_cast<const u32x4*>(xa + trow[m] * K + t * kTileK + c * 128 + q * 32);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            u32x4 v = row[u];
            xv[m][u] = tvalid[m] ? v : u32x4{0, 0, 0, 0};
          }
        }
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
              const uint32_t d = wc[g][c][u];
              bf16x2 w[4];
              w[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 0);
              w[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 1);
              w[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 2);
              w[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 3);
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
  }

  // Sum the four lanes of each row (xor 16, then 32), then the waves.
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      acc[g][m] += __shfl_xor(acc[g][m], 16);
      acc[g][m] += __shfl_xor(acc[g][m], 32);
    }
  __shared__ float red[NW][NG][MT][16];
  if (q == 0) {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int m = 0; m < MT; ++m) red[wave][g][m][lane] = acc[g][m];
  }
  __syncthreads();
  if (wave > 0) return;

  // Wave 0 rebuilds the MFMA result layout (lane l: token l % 16, rows
  // 4 (l / 16) + r) so the shared epilogues apply unchanged.
  const int tl = lane & 15;
  const bool lvalid = tl < MT && tok0 + tl < args.M;
  const int tm = tl < MT ? tl : 0;
  f32x4 res[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red[w][g][tm][4 * q + r];
      res[g][r] = lvalid ? s : 0.0f;
    }
  const float alpha = *args.alpha;
  const int64_t token = tok0 + tl;
  if constexpr (EpiTraits<EPI>::swiglu) {
    const float g2i = (EPI == kSwigluNvfp4) ? *args.g2_inv : 0.0f;
    store_swiglu<EPI>(res[0], res[1], alpha, g2i, lvalid, token, (int64_t)blockIdx.x * kTileRows,
                      lane, args.N / 2, args.out, args.out_scales);
  } else {
    store_dense<EPI>(res[0], alpha, lvalid, token, rg0 * kTileRows + 4 * q, args.N, args.out);
  }
}

template <int MODE, int EPI, int MT>
static hipError_t launch_mt(const GemmArgs& a, hipStream_t s) {
  constexpr int NG = EpiTraits<EPI>::swiglu ? 2 : 1;
  constexpr int NW = 4;
  dim3 grid((unsigned)(a.N / kTileRows / NG), (unsigned)((a.M + MT - 1) / MT));
  k_valu_gemv<MODE, EPI, MT, NW><<<grid, NW * 64, 0, s>>>(a);
  return hipGetLastError();
}

template <int MODE, int EPI>
static hipError_t launch_me(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 1) return launch_mt<MODE, EPI, 1>(a, s);
  if (a.M == 2) return launch_mt<MODE, EPI, 2>(a, s);
  return launch_mt<MODE, EPI, 4>(a, s);
}

hipError_t launch_valu_gemv(int mode, int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (mode == kW4A4) {
    switch (epi) {
      case kOutF32: return launch_me<kW4A4, kOutF32>(a, s);
      case kOutBF16: return launch_me<kW4A4, kOutBF16>(a, s);
      case kSwigluNvfp4: return launch_me<kW4A4, kSwigluNvfp4>(a, s);
      case kSwigluBF16: return launch_me<kW4A4, kSwigluBF16>(a, s);
      case kSwigluF32: return launch_me<kW4A4, kSwigluF32>(a, s);
    }
  } else {
    switch (epi) {
      case kOutF32: return launch_me<kW4A16, kOutF32>(a, s);
      case kOutBF16: return launch_me<kW4A16, kOutBF16>(a, s);
      case kSwigluBF16: return launch_me<kW4A16, kSwigluBF16>(a, s);
      case kSwigluF32: return launch_me<kW4A16, kSwigluF32>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
