// stream.hip -- weight-streaming MFMA GEMM for small token counts.
//
// Decode-sized GEMMs are bound by HBM reads of the packed weight (0.5625
// bytes per element), so each workgroup streams whole packed tiles with
// 16-byte loads and spends the MFMA unit only on the contraction: the weight
// rows are the 16-row A operand of v_mfma_f32_16x16x32 (f16 for W4A4, bf16
// for W4A16) and up to four groups of 16 tokens are the B operand. Tokens
// beyond M are zero columns. Activations are read from global memory (they
// are tiny and stay in L2) in their NVFP4 or bf16 form and dequantized in
// registers exactly like the weights.
//
// Work split: a workgroup owns NG packed row groups (2 for the SwiGLU pair
// gate/up) and NW waves divide the K tiles between them; the partial sums
// are combined through LDS in a fixed order, so results are deterministic.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

template <int MODE, int EPI, int NT, int NW>
__global__ __launch_bounds__(NW * 64) void k_stream(GemmArgs args) {
  constexpr int NG = EpiTraits<EPI>::swiglu ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int tl = lane & 15;
  const int64_t K = args.K;
  const int64_t T = K / kTileK;
  const int64_t rg0 = (int64_t)blockIdx.x * NG;
  const int64_t tok0 = (int64_t)blockIdx.y * 16 * NT;

  int64_t tok[NT];
  bool tvalid[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    tok[j] = tok0 + 16 * j + tl;
    tvalid[j] = tok[j] < args.M;
  }

  f32x4 acc[NG][NT];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint8_t* wbase = args.w;
  for (int64_t t = wave; t < T; t += NW) {
    // Weight tiles: two 16-byte code chunks and one scale dword per lane.
    u32x4 wc[NG][2];
    uint32_t wsd[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const uint8_t* tp = wbase + ((rg0 + g) * T + t) * kTileBytes;
      wc[g][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tp + 16 * lane));
      wc[g][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tp + 1024 + 16 * lane));
      wsd[g] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(tp + kTileCodeBytes + 4 * lane));
    }
    if constexpr (MODE == kW4A4) {
      const uint8_t* ac = reinterpret_cast<const uint8_t*>(args.a);
      u32x4 xc[NT][2];
      uint32_t xsd[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        // Rows past M read row 0 (always present) and are zeroed: no address
        // beyond the activation is ever formed.
        const int64_t trow = tvalid[j] ? tok[j] : 0;
        const uint8_t* row = ac + trow * (K / 2) + t * 128 + q * 16;
        u32x4 c0 = *reinterpret_cast<const u32x4*>(row);
        u32x4 c1 = *reinterpret_cast<const u32x4*>(row + 64);
        const uint8_t* srow = args.a_scales + trow * (K / 16) + t * 16 + q * 2;
        uint32_t lo = *reinterpret_cast<const uint16_t*>(srow);
        uint32_t hi = *reinterpret_cast<const uint16_t*>(srow + 8);
        const u32x4 z = {0, 0, 0, 0};
        xc[j][0] = tvalid[j] ? c0 : z;
        xc[j][1] = tvalid[j] ? c1 : z;
        xsd[j] = tvalid[j] ? (lo | (hi << 16)) : 0u;
      }
      _Float16 ws[NG][4], xs[NT][4];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        ws[g][0] = scale_f16<0>(wsd[g]); ws[g][1] = scale_f16<1>(wsd[g]);
        ws[g][2] = scale_f16<2>(wsd[g]); ws[g][3] = scale_f16<3>(wsd[g]);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        xs[j][0] = scale_f16<0>(xsd[j]); xs[j][1] = scale_f16<1>(xsd[j]);
        xs[j][2] = scale_f16<2>(xsd[j]); xs[j][3] = scale_f16<3>(xsd[j]);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int sb = 2 * c + (u >> 1);
          f16x8 A[NG], B[NT];
#pragma unroll
          for (int g = 0; g < NG; ++g) A[g] = deq8_f16(wc[g][c][u], ws[g][sb]);
#pragma unroll
          for (int j = 0; j < NT; ++j) B[j] = deq8_f16(xc[j][c][u], xs[j][sb]);
#pragma unroll
          for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[g][j] = mfma16x16x32(A[g], B[j], acc[g][j]);
        }
    } else {
      const uint16_t* xa = reinterpret_cast<const uint16_t*>(args.a);
      float ws[NG][4];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        ws[g][0] = e4m3_to_f32<0>(wsd[g]); ws[g][1] = e4m3_to_f32<1>(wsd[g]);
        ws[g][2] = e4m3_to_f32<2>(wsd[g]); ws[g][3] = e4m3_to_f32<3>(wsd[g]);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 xv[NT][4];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int64_t trow = tvalid[j] ? tok[j] : 0;
          const u32x4* row = reinterpret_cast<const u32x4*>(xa + trow * K + t * kTileK + c * 128 + q * 32);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            u32x4 v = row[u];
            xv[j][u] = tvalid[j] ? v : u32x4{0, 0, 0, 0};
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int sb = 2 * c + (u >> 1);
          bf16x8 A[NG];
#pragma unroll
          for (int g = 0; g < NG; ++g) A[g] = deq8_bf16(wc[g][c][u], ws[g][sb]);
#pragma unroll
          for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[g][j] = mfma16x16x32(A[g], as_bf16x8(xv[j][u]), acc[g][j]);
        }
      }
    }
  }

  // Combine the waves' partial sums in wave order.
  if constexpr (NW > 1) {
    __shared__ f32x4 red[NW - 1][NG * NT][64];
    if (wave > 0) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int j = 0; j < NT; ++j) red[wave - 1][g * NT + j][lane] = acc[g][j];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < NW - 1; ++w)
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          f32x4 p = red[w][g * NT + j][lane];
          acc[g][j] = f32x4{acc[g][j][0] + p[0], acc[g][j][1] + p[1], acc[g][j][2] + p[2],
                            acc[g][j][3] + p[3]};
        }
  }

  const float alpha = *args.alpha;
  if constexpr (EpiTraits<EPI>::swiglu) {
    const float g2i = (EPI == kSwigluNvfp4) ? *args.g2_inv : 0.0f;
    const int64_t I = args.N / 2;
    const int64_t j0 = (int64_t)blockIdx.x * kTileRows;
#pragma unroll
    for (int j = 0; j < NT; ++j)
      store_swiglu<EPI>(acc[0][j], acc[1][j], alpha, g2i, tvalid[j], tok[j], j0, lane, I, args.out,
                        args.out_scales);
  } else {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        store_dense<EPI>(acc[g][j], alpha, tvalid[j], tok[j], (rg0 + g) * kTileRows + 4 * q, args.N,
                         args.out);
  }
}

template <int MODE, int EPI, int NT>
static hipError_t launch_nt(const GemmArgs& a, hipStream_t s) {
  constexpr int NG = EpiTraits<EPI>::swiglu ? 2 : 1;
  constexpr int NW = 4;
  dim3 grid((unsigned)(a.N / kTileRows / NG), (unsigned)((a.M + 16 * NT - 1) / (16 * NT)));
  k_stream<MODE, EPI, NT, NW><<<grid, NW * 64, 0, s>>>(a);
  return hipGetLastError();
}

template <int MODE, int EPI>
static hipError_t launch_mode_epi(const GemmArgs& a, hipStream_t s) {
  const int64_t groups = (a.M + 15) / 16;
  if (groups <= 1) return launch_nt<MODE, EPI, 1>(a, s);
  if (groups == 2) return launch_nt<MODE, EPI, 2>(a, s);
  if (groups == 3) return launch_nt<MODE, EPI, 3>(a, s);
  return launch_nt<MODE, EPI, 4>(a, s);
}

hipError_t launch_stream_gemm(int mode, int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (mode == kW4A4) {
    switch (epi) {
      case kOutF32: return launch_mode_epi<kW4A4, kOutF32>(a, s);
      case kOutBF16: return launch_mode_epi<kW4A4, kOutBF16>(a, s);
      case kSwigluNvfp4: return launch_mode_epi<kW4A4, kSwigluNvfp4>(a, s);
      case kSwigluBF16: return launch_mode_epi<kW4A4, kSwigluBF16>(a, s);
      case kSwigluF32: return launch_mode_epi<kW4A4, kSwigluF32>(a, s);
    }
  } else {
    switch (epi) {
      case kOutF32: return launch_mode_epi<kW4A16, kOutF32>(a, s);
      case kOutBF16: return launch_mode_epi<kW4A16, kOutBF16>(a, s);
      case kSwigluBF16: return launch_mode_epi<kW4A16, kSwigluBF16>(a, s);
      case kSwigluF32: return launch_mode_epi<kW4A16, kSwigluF32>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
