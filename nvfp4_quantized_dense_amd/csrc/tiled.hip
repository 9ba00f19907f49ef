// tiled.hip -- LDS-tiled MFMA GEMM for large token counts (prefill).
//
// A workgroup computes a 128-row x 128-token output tile. Per 256-column K
// tile it copies the packed weight tiles (8 row groups) and the activation
// tile into LDS in their 4-bit form (the activation is rearranged into the
// same lane order as the packed weight, so every fragment read is one
// conflict-free 16-byte LDS access per lane), then each of the four waves
// dequantizes its fragments in registers and runs v_mfma_f32_16x16x32 on a
// 64 x 64 sub-tile. W4A4 computes in f16 (both operands exact), W4A16 in
// bf16 with the bf16 activation staged as is.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int kBG = 8;  // row groups (of 16) per workgroup
constexpr int kBT = 8;  // token groups (of 16) per workgroup

template <int MODE, int EPI>
__global__ __launch_bounds__(256) void k_tiled(GemmArgs args) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1;  // row half of the tile
  const int wt = wave & 1;   // token half of the tile
  const int q = lane >> 4;
  const int tl = lane & 15;
  const int64_t K = args.K, T = K / kTileK, N = args.N, M = args.M;
  const int64_t ngroups = N / kTileRows;
  const int64_t rg0 = (int64_t)blockIdx.x * kBG;
  const int64_t tok0 = (int64_t)blockIdx.y * (kBT * 16);

  __shared__ __attribute__((aligned(16))) uint8_t sW[kBG * kTileBytes];
  // W4A4: per token group 2048 code bytes in lane order + 256 scale bytes.
  // W4A16: per token group [c][u][lane] 16-byte bf16 fragments.
  constexpr int kABytes = (MODE == kW4A4) ? kBT * kTileBytes : kBT * 2 * 4 * 64 * 16;
  __shared__ __attribute__((aligned(16))) uint8_t sA[kABytes];

  f32x4 acc[4][4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t t = 0; t < T; ++t) {
    // Stage the packed weight tiles; groups past N read as zero.
    for (int p = tid; p < kBG * (kTileBytes / 16); p += 256) {
      const int g = p / (kTileBytes / 16);
      const int off = (p % (kTileBytes / 16)) * 16;
      u32x4 v = {0, 0, 0, 0};
      if (rg0 + g < ngroups)
        v = *reinterpret_cast<const u32x4*>(args.w + ((rg0 + g) * T + t) * kTileBytes + off);
      *reinterpret_cast<u32x4*>(sW + g * kTileBytes + off) = v;
    }
    if constexpr (MODE == kW4A4) {
      const uint8_t* ac = reinterpret_cast<const uint8_t*>(args.a);
      // Codes: each token row contributes 2 chunks x 4 lanes of 16 bytes.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = tid + 256 * i;
        const int tt = p >> 3, c = (p >> 2) & 1, qq = p & 3;
        const int64_t token = tok0 + tt;
        u32x4 v = {0, 0, 0, 0};
        if (token < M) v = *reinterpret_cast<const u32x4*>(ac + token * (K / 2) + t * 128 + c * 64 + qq * 16);
        *reinterpret_cast<u32x4*>(sA + (tt >> 4) * kTileBytes + c * 1024 + (qq * 16 + (tt & 15)) * 16) = v;
      }
      // Scales: 16 bytes per token row, split into the four lanes' dwords.
      if (tid < kBT * 16) {
        const int tt = tid;
        const int64_t token = tok0 + tt;
        u32x4 d = {0, 0, 0, 0};
        if (token < M) d = *reinterpret_cast<const u32x4*>(args.a_scales + token * (K / 16) + t * 16);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const uint32_t lo = (qq < 2 ? d[0] : d[1]) >> (16 * (qq & 1));
          const uint32_t hi = (qq < 2 ? d[2] : d[3]) >> (16 * (qq & 1));
          *reinterpret_cast<uint32_t*>(sA + (tt >> 4) * kTileBytes + kTileCodeBytes + (qq * 16 + (tt & 15)) * 4) =
              (lo & 0xFFFFu) | (hi << 16);
        }
      }
    } else {
      const uint16_t* xa = reinterpret_cast<const uint16_t*>(args.a);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int p = tid + 256 * i;
        const int tt = p >> 5, e = p & 31;
        const int c = e >> 4, qq = (e >> 2) & 3, u = e & 3;
        const int64_t token = tok0 + tt;
        u32x4 v = {0, 0, 0, 0};
        if (token < M) v = *reinterpret_cast<const u32x4*>(xa + token * K + t * kTileK + c * 128 + qq * 32 + u * 8);
        *reinterpret_cast<u32x4*>(sA + ((((tt >> 4) * 2 + c) * 4 + u) * 64 + qq * 16 + (tt & 15)) * 16) = v;
      }
    }
    __syncthreads();

    // Fragments of this wave: row groups 4 wr + g, token groups 4 wt + j.
    uint32_t wsd[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      wsd[g] = *reinterpret_cast<const uint32_t*>(sW + (4 * wr + g) * kTileBytes + kTileCodeBytes + 4 * lane);
    if constexpr (MODE == kW4A4) {
      uint32_t xsd[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xsd[j] = *reinterpret_cast<const uint32_t*>(sA + (4 * wt + j) * kTileBytes + kTileCodeBytes + 4 * lane);
      _Float16 ws[4][4], xs[4][4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        ws[g][0] = scale_f16<0>(wsd[g]); ws[g][1] = scale_f16<1>(wsd[g]);
        ws[g][2] = scale_f16<2>(wsd[g]); ws[g][3] = scale_f16<3>(wsd[g]);
        xs[g][0] = scale_f16<0>(xsd[g]); xs[g][1] = scale_f16<1>(xsd[g]);
        xs[g][2] = scale_f16<2>(xsd[g]); xs[g][3] = scale_f16<3>(xsd[g]);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 wc[4], xc[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
          wc[g] = *reinterpret_cast<const u32x4*>(sW + (4 * wr + g) * kTileBytes + c * 1024 + 16 * lane);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xc[j] = *reinterpret_cast<const u32x4*>(sA + (4 * wt + j) * kTileBytes + c * 1024 + 16 * lane);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int sb = 2 * c + (u >> 1);
          f16x8 A[4], B[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) A[g] = deq8_f16(wc[g][u], ws[g][sb]);
#pragma unroll
          for (int j = 0; j < 4; ++j) B[j] = deq8_f16(xc[j][u], xs[j][sb]);
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[g][j] = mfma16x16x32(A[g], B[j], acc[g][j]);
        }
      }
    } else {
      float ws[4][4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        ws[g][0] = e4m3_to_f32<0>(wsd[g]); ws[g][1] = e4m3_to_f32<1>(wsd[g]);
        ws[g][2] = e4m3_to_f32<2>(wsd[g]); ws[g][3] = e4m3_to_f32<3>(wsd[g]);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 wc[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
          wc[g] = *reinterpret_cast<const u32x4*>(sW + (4 * wr + g) * kTileBytes + c * 1024 + 16 * lane);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int sb = 2 * c + (u >> 1);
          bf16x8 A[4], B[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) A[g] = deq8_bf16(wc[g][u], ws[g][sb]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            B[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(sA + ((((4 * wt + j) * 2 + c) * 4 + u) * 64 + lane) * 16));
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[g][j] = mfma16x16x32(A[g], B[j], acc[g][j]);
        }
      }
    }
    __syncthreads();
  }

  const float alpha = *args.alpha;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t token = tok0 + 16 * (4 * wt + j) + tl;
    const bool tv = token < M;
    const float at = row_alpha(alpha, args.row_scale, tv, token);  // per-token factor, if any
    if constexpr (EpiTraits<EPI>::swiglu) {
      const float g2i = (EPI == kSwigluNvfp4) ? *args.g2_inv : 0.0f;
#pragma unroll
      for (int g = 0; g < 4; g += 2) {
        const int64_t grp = rg0 + 4 * wr + g;  // gate group (even), up group grp + 1
        store_swiglu<EPI>(acc[g][j], acc[g + 1][j], at, g2i, tv && grp < ngroups, token,
                          (grp >> 1) * kTileRows, lane, N / 2, args.out, args.out_scales, args.h_prescale);
      }
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t grp = rg0 + 4 * wr + g;
        store_dense<EPI>(acc[g][j], at, tv && grp < ngroups, token, grp * kTileRows + 4 * q, N,
                         args.out);
      }
    }
  }
}

template <int MODE, int EPI>
static hipError_t launch_t(const GemmArgs& a, hipStream_t s) {
  const int64_t ngroups = a.N / kTileRows;
  dim3 grid((unsigned)((ngroups + kBG - 1) / kBG), (unsigned)((a.M + kBT * 16 - 1) / (kBT * 16)));
  k_tiled<MODE, EPI><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_tiled_gemm(int mode, int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (mode == kW4A4) {
    switch (epi) {
      case kOutF32: return launch_t<kW4A4, kOutF32>(a, s);
      case kOutBF16: return launch_t<kW4A4, kOutBF16>(a, s);
      case kSwigluNvfp4: return launch_t<kW4A4, kSwigluNvfp4>(a, s);
      case kSwigluBF16: return launch_t<kW4A4, kSwigluBF16>(a, s);
      case kSwigluF32: return launch_t<kW4A4, kSwigluF32>(a, s);
    }
  } else {
    switch (epi) {
      case kOutF32: return launch_t<kW4A16, kOutF32>(a, s);
      case kOutBF16: return launch_t<kW4A16, kOutBF16>(a, s);
      case kSwigluBF16: return launch_t<kW4A16, kSwigluBF16>(a, s);
      case kSwigluF32: return launch_t<kW4A16, kSwigluF32>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
