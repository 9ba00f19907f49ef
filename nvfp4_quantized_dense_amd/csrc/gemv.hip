// gemv.hip -- VALU GEMV for the smallest token counts (decode), no MFMA.
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
// of each 128-column half tile (the packed layout's lane order). NW waves
// divide a row group's K tiles; each wave keeps the next tile's loads in
// flight while it computes the current one (two register sets, no branch
// around the prefetch: past the last tile it loads from out of range, which
// returns zeros without a memory access). Token rows past M are out of range
// of the activation buffers as well and read as zeros. The four lanes of a
// row and the NW waves are summed at the end in a fixed order.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

#if defined(__HIP_DEVICE_COMPILE__)
namespace {

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

template <int MODE, int MT>
struct GemvSrc {
  Rsrc w, a, s;
  uint32_t a_row[MT];  // lane offset of each token row in the activation codes (W4A4) or bf16 (W4A16)
  uint32_t s_row[MT];  // lane offset of each token row in the activation scales (W4A4)
};

// Loads of one K tile for one wave: NG weight tiles and (W4A4) the NVFP4
// activation slices of MT tokens.
template <int MODE, int NG, int MT>
struct GemvTile {
  u32x4 wc[NG][2];
  uint32_t wsd[NG];
  u32x4 xc[MODE == kW4A4 ? MT : 1][2];
  uint32_t xsd[MODE == kW4A4 ? MT : 1];
};

template <int MODE, int NG, int MT>
__device__ __forceinline__ void gemv_load(GemvTile<MODE, NG, MT>& d, const GemvSrc<MODE, MT>& src,
                                          int64_t rg0, int64_t T, int64_t t, int lane) {
  const int q = lane >> 4;
  const bool in = t < T;
  const uint32_t tw = in ? (uint32_t)(t * kTileBytes) : kOutOfRange;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint32_t gbase = (uint32_t)((rg0 + g) * T * kTileBytes);
    d.wc[g][0] = bload16_nt(src.w, tw + 16 * lane, gbase);
    d.wc[g][1] = bload16_nt(src.w, tw + 1024 + 16 * lane, gbase);
    d.wsd[g] = bload4_nt(src.w, tw + kTileCodeBytes + 4 * lane, gbase);
  }
  if constexpr (MODE == kW4A4) {
    const uint32_t ta = in ? (uint32_t)(t * 128 + q * 16) : kOutOfRange;
    const uint32_t ts = in ? (uint32_t)(t * 16 + q * 2) : kOutOfRange;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      d.xc[m][0] = bload16(src.a, src.a_row[m] + ta);
      d.xc[m][1] = bload16(src.a, src.a_row[m] + ta + 64);
      d.xsd[m] = bload2(src.s, src.s_row[m] + ts) | (bload2(src.s, src.s_row[m] + ts + 8) << 16);
    }
  }
}

template <int MODE, int NG, int MT>
__device__ __forceinline__ void gemv_compute(float (&acc)[NG][MT], const GemvTile<MODE, NG, MT>& d,
                                             const GemvSrc<MODE, MT>& src, int64_t t, int lane) {
  float ws[NG][4];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    ws[g][0] = e4m3_to_f32<0>(d.wsd[g]); ws[g][1] = e4m3_to_f32<1>(d.wsd[g]);
    ws[g][2] = e4m3_to_f32<2>(d.wsd[g]); ws[g][3] = e4m3_to_f32<3>(d.wsd[g]);
  }
  if constexpr (MODE == kW4A4) {
    float xs[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      xs[m][0] = e4m3_to_f32<0>(d.xsd[m]); xs[m][1] = e4m3_to_f32<1>(d.xsd[m]);
      xs[m][2] = e4m3_to_f32<2>(d.xsd[m]); xs[m][3] = e4m3_to_f32<3>(d.xsd[m]);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        f16x2 xp[MT][8];  // activation pairs of this block, unscaled
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int uu = 0; uu < 2; ++uu) {
            const uint32_t v = d.xc[m][c][2 * blk + uu];
            xp[m][4 * uu + 0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 0);
            xp[m][4 * uu + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 1);
            xp[m][4 * uu + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 2);
            xp[m][4 * uu + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 3);
          }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          float bs[MT];
#pragma unroll
          for (int m = 0; m < MT; ++m) bs[m] = 0.0f;
#pragma unroll
          for (int uu = 0; uu < 2; ++uu) {
            const uint32_t v = d.wc[g][c][2 * blk + uu];
            const f16x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 0);
            const f16x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 1);
            const f16x2 w2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 2);
            const f16x2 w3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 3);
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
    const int q = lane >> 4;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 xv[MT][4];
      const uint32_t tx = (uint32_t)((t * kTileK + c * 128 + q * 32) * 2);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int u = 0; u < 4; ++u) xv[m][u] = bload16(src.a, src.a_row[m] + tx + 16 * u);
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
}

}  // namespace
#endif  // __HIP_DEVICE_COMPILE__

template <int MODE, int EPI, int MT, int NW>
__global__ __launch_bounds__(NW * 64) void k_valu_gemv(GemmArgs args) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NG = EpiTraits<EPI>::swiglu ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4;
  const int64_t K = args.K, T = K / kTileK;
  const int64_t rg0 = (int64_t)blockIdx.x * NG;
  const int64_t tok0 = (int64_t)blockIdx.y * MT;

  GemvSrc<MODE, MT> src;
  src.w = make_rsrc(args.w, (uint32_t)(args.N / kTileRows * T * kTileBytes));
  if constexpr (MODE == kW4A4) {
    src.a = make_rsrc(args.a, (uint32_t)(args.M * (K / 2)));
    src.s = make_rsrc(args.a_scales, (uint32_t)(args.M * (K / 16)));
  } else {
    src.a = make_rsrc(args.a, (uint32_t)(args.M * K * 2));
    src.s = src.a;
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    // rows past M start past the end of the buffer: they read as zeros
    src.a_row[m] = (uint32_t)((tok0 + m) * (MODE == kW4A4 ? K / 2 : K * 2));
    src.s_row[m] = (uint32_t)((tok0 + m) * (K / 16));
  }

  float acc[NG][MT];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[g][m] = 0.0f;

  // Tiles t = wave, wave + NW, ...; two register sets alternate.
  int64_t t = wave;
  GemvTile<MODE, NG, MT> ta, tb;
  gemv_load<MODE, NG, MT>(ta, src, rg0, T, t, lane);
  while (t < T) {
    gemv_load<MODE, NG, MT>(tb, src, rg0, T, t + NW, lane);
    gemv_compute<MODE, NG, MT>(acc, ta, src, t, lane);
    t += NW;
    if (t >= T) break;
    gemv_load<MODE, NG, MT>(ta, src, rg0, T, t + NW, lane);
    gemv_compute<MODE, NG, MT>(acc, tb, src, t, lane);
    t += NW;
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
#endif  // __HIP_DEVICE_COMPILE__
}

template <int MODE, int EPI, int MT, int NW>
static hipError_t launch_mt_nw(const GemmArgs& a, hipStream_t s) {
  constexpr int NG = EpiTraits<EPI>::swiglu ? 2 : 1;
  dim3 grid((unsigned)(a.N / kTileRows / NG), (unsigned)((a.M + MT - 1) / MT));
  k_valu_gemv<MODE, EPI, MT, NW><<<grid, NW * 64, 0, s>>>(a);
  return hipGetLastError();
}

// Waves per workgroup: enough that the grid keeps about 16 waves per CU
// streaming (small grids such as down_proj's get 16-wave workgroups).
// (16-wave workgroups only where the tile fits 128 VGPRs per lane.)
template <int MODE, int EPI, int MT>
static hipError_t launch_mt(const GemmArgs& a, hipStream_t s) {
  constexpr int NG = EpiTraits<EPI>::swiglu ? 2 : 1;
  const int64_t wgs = a.N / kTileRows / NG * ((a.M + MT - 1) / MT);
  if (wgs >= 1024) return launch_mt_nw<MODE, EPI, MT, 4>(a, s);
  if constexpr (MT <= 2) {
    if (wgs < 512) return launch_mt_nw<MODE, EPI, MT, 16>(a, s);
  }
  return launch_mt_nw<MODE, EPI, MT, 8>(a, s);
}

template <int MODE, int EPI>
static hipError_t launch_me(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 1) return launch_mt<MODE, EPI, 1>(a, s);
  if (a.M == 2) return launch_mt<MODE, EPI, 2>(a, s);
  return launch_mt<MODE, EPI, 4>(a, s);
}

// Needs the packed weight and the activations below 2^31 bytes (32-bit
// buffer offsets); the caller checks.
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
