// fp4gemv.hip -- W4A4 GEMV for the smallest token counts (decode) on the
// FP4 matrix core, with the per-16 E4M3 scales applied exactly (the block
// masking is described in fp4_tile.h).
//
// Work split as in the VALU GEMV: a workgroup owns NG row groups (gate and
// up for SwiGLU), its NW waves divide the K tiles, each wave double-buffers
// its tiles (the prefetch past the last tile reads out of range: zeros, no
// memory access), and the partial sums are reduced in a fixed order.
#include "fp4_tile.h"

namespace nvfp4 {

template <int EPI, int MT, int NW, bool QX>
__global__ __launch_bounds__(NW * 64) void k_fp4_gemv(GemmArgs args) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NG = EpiTraits<EPI>::swiglu ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4;
  const int64_t rg0 = (int64_t)blockIdx.x * NG;
  const int64_t tok0 = (int64_t)blockIdx.y * MT;
  extern __shared__ __attribute__((aligned(16))) uint8_t xl[];  // activation image, see lds_*_off
  __shared__ float red[NW * NG * MT * 16];

  clear_words(args.zero_ptr, args.zero_n);
  const float alpha = uniform_now(args.alpha);
  const float g2i = EPI == kSwigluNvfp4 ? uniform_now(args.g2_inv) : 0.0f;
  f32x4 acc[NG][MT];
  f4_gemv_acc<NG, MT, NW, QX>(args, rg0, tok0, xl, lane, wave, acc);

  const int tl = lane & 15;
  const bool lvalid = tl < MT && tok0 + tl < args.M;
  f32x4 res[NG];
  if (!f4_reduce<NG, MT, NW>(acc, red, wave, lane, lvalid, res)) return;
  const int64_t token = tok0 + tl;
  if constexpr (EpiTraits<EPI>::swiglu) {
    store_swiglu<EPI>(res[0], res[1], row_alpha(alpha, args.row_scale, lvalid, token), g2i, lvalid, token,
                      (int64_t)blockIdx.x * kTileRows,
                      lane, args.N / 2, args.out, args.out_scales);
  } else {
    store_dense<EPI>(res[0], row_alpha(alpha, args.row_scale, lvalid, token), lvalid, token, rg0 * kTileRows + 4 * q,
                     args.N, args.out);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

bool fp4_gemv_supported(int64_t M, int64_t K) { return fp4_lds_bytes(M <= 1 ? 1 : 2, K) <= kFp4GemvLdsBytes; }

template <int EPI, int MT, int NW>
static hipError_t fp4_launch_nw(const GemmArgs& a, hipStream_t s) {
  constexpr int NG = EpiTraits<EPI>::swiglu ? 2 : 1;
  dim3 grid((unsigned)(a.N / kTileRows / NG), (unsigned)((a.M + MT - 1) / MT));
  const size_t lds = (size_t)fp4_lds_bytes(MT, a.K);
  if constexpr (EPI == kSwigluNvfp4 && MT == 1) {
    if (a.a_g_inv) {
      k_fp4_gemv<EPI, MT, NW, true><<<grid, NW * 64, lds, s>>>(a);
      return hipGetLastError();
    }
  }
  k_fp4_gemv<EPI, MT, NW, false><<<grid, NW * 64, lds, s>>>(a);
  return hipGetLastError();
}

// Waves per workgroup: 4 (measured best from 320 to 1152 workgroups, the
// decode shapes), 16 for grids too small to spread over the CUs otherwise.
static int fp4_waves(int64_t wgs) { return wgs < 128 ? 16 : 4; }

template <int EPI, int MT>
static hipError_t fp4_launch_mt(const GemmArgs& a, hipStream_t s) {
  constexpr int NG = EpiTraits<EPI>::swiglu ? 2 : 1;
  const int64_t wgs = a.N / kTileRows / NG * ((a.M + MT - 1) / MT);
  if (fp4_waves(wgs) == 16) return fp4_launch_nw<EPI, MT, 16>(a, s);
  return fp4_launch_nw<EPI, MT, 4>(a, s);
}

template <int EPI>
static hipError_t fp4_launch_e(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 1) return fp4_launch_mt<EPI, 1>(a, s);
  return fp4_launch_mt<EPI, 2>(a, s);
}

// W4A4 only. Needs the packed weight and the activations below 2^31 bytes
// (32-bit buffer offsets) and fp4_gemv_supported(M, K); the caller checks.
hipError_t launch_fp4_gemv(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (!fp4_gemv_supported(a.M, a.K) || a.ksplit != 1 || (a.a_g_inv && (epi != kSwigluNvfp4 || a.M > 1)))
    return hipErrorInvalidValue;
  switch (epi) {
    case kOutF32: return fp4_launch_e<kOutF32>(a, s);
    case kOutBF16: return fp4_launch_e<kOutBF16>(a, s);
    case kSwigluNvfp4: return fp4_launch_e<kSwigluNvfp4>(a, s);
    case kSwigluBF16: return fp4_launch_e<kSwigluBF16>(a, s);
    case kSwigluF32: return fp4_launch_e<kSwigluF32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
