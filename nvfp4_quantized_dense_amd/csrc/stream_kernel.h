// stream_kernel.h -- weight-streaming MFMA GEMM for small token counts:
// the kernel and its launch templates, shared by stream.hip (2-4 token
// groups) and stream_nt1.hip (one token group), which are compiled with
// different instruction-scheduling strategies.
//
// Small-batch GEMMs are bound by HBM reads of the packed weight (0.5625
// bytes per element), so each workgroup streams whole packed tiles with
// 16-byte loads and spends the MFMA unit only on the contraction: the weight
// rows are the 16-row A operand of v_mfma_f32_16x16x32 (f16 for W4A4, bf16
// for W4A16) and up to four groups of 16 tokens are the B operand. Token rows
// past M lie out of range of the activation buffers and read as zeros.
// Activations are read from global memory (they are small and stay in L2) in
// their NVFP4 or bf16 form and dequantized in registers like the weights.
//
// Work split: a workgroup owns G packed row groups (gate/up pairs for the
// SwiGLU epilogues) and NW waves divide the K tiles between them; each wave
// loads a tile (weights and activations together, branch-free: past the last
// tile the loads are out of range) and multiplies it. Partial sums are
// combined through LDS in a fixed order (deterministic). Several row groups
// per workgroup read each activation slice once for all of them and keep more
// weight bytes in flight per wave.
#pragma once

#include "device_common.h"
#include "kernels.h"
#include "stream_groups.h"

namespace nvfp4 {

#if defined(__HIP_DEVICE_COMPILE__)
namespace {

template <int MODE, int NT>
struct StreamSrc {
  Rsrc w, a, s;
  uint32_t a_row[NT];  // lane offset of this lane's token row, per token group
  uint32_t s_row[NT];
};

// One K tile for one wave: NG weight tiles and the activation slices of
// NT token groups (W4A4: codes and scales; W4A16: bf16, 64 bytes per lane
// and half tile).
template <int MODE, int NG, int NT>
struct StreamTile {
  u32x4 wc[NG][2];
  uint32_t wsd[NG];
  u32x4 xc[NT][MODE == kW4A4 ? 2 : 8];
  uint32_t xsd[MODE == kW4A4 ? NT : 1][2];
};

// Tile t of row groups of T tiles. From tile t_end on every load is out of
// range: zeros, no memory access, and the tile adds +0.
template <int MODE, int NG, int NT>
__device__ __forceinline__ void stream_load(StreamTile<MODE, NG, NT>& d, const StreamSrc<MODE, NT>& src,
                                            int64_t rg0, int T, int t_end, int t, int lane) {
  const int q = lane >> 4;
  const bool in = t < t_end;
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
    for (int j = 0; j < NT; ++j) {
      d.xc[j][0] = bload16(src.a, src.a_row[j] + ta);
      d.xc[j][1] = bload16(src.a, src.a_row[j] + ta + 64);
      d.xsd[j][0] = bload2(src.s, src.s_row[j] + ts);
      d.xsd[j][1] = bload2(src.s, src.s_row[j] + ts + 8);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t tx = in ? (uint32_t)((t * kTileK + c * 128 + q * 32) * 2) : kOutOfRange;
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u) d.xc[j][4 * c + u] = bload16(src.a, src.a_row[j] + tx + 16 * u);
    }
  }
}

template <int MODE, int NG, int NT>
__device__ __forceinline__ void stream_compute(f32x4 (&acc)[NG][NT], const StreamTile<MODE, NG, NT>& d) {
  if constexpr (MODE == kW4A4) {
    // E4M3 scale bytes to f16, two per instruction (exact).
    _Float16 ws[NG][4], xs[NT][4];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d.wsd[g], 1.0f, false);
      const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d.wsd[g], 1.0f, true);
      ws[g][0] = lo.x; ws[g][1] = lo.y; ws[g][2] = hi.x; ws[g][3] = hi.y;
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const f16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d.xsd[j][0], 1.0f, false);
      const f16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d.xsd[j][1], 1.0f, false);
      xs[j][0] = a0.x; xs[j][1] = a0.y; xs[j][2] = a1.x; xs[j][3] = a1.y;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sb = 2 * c + (u >> 1);
        f16x8 A[NG], B[NT];
#pragma unroll
        for (int g = 0; g < NG; ++g) A[g] = deq8_f16(d.wc[g][c][u], ws[g][sb]);
#pragma unroll
        for (int j = 0; j < NT; ++j) B[j] = deq8_f16(d.xc[j][c][u], xs[j][sb]);
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int j = 0; j < NT; ++j) acc[g][j] = mfma16x16x32(A[g], B[j], acc[g][j]);
      }
  } else {
    float ws[NG][4];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      ws[g][0] = e4m3_to_f32<0>(d.wsd[g]); ws[g][1] = e4m3_to_f32<1>(d.wsd[g]);
      ws[g][2] = e4m3_to_f32<2>(d.wsd[g]); ws[g][3] = e4m3_to_f32<3>(d.wsd[g]);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sb = 2 * c + (u >> 1);
        bf16x8 A[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) A[g] = deq8_bf16(d.wc[g][c][u], ws[g][sb]);
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int j = 0; j < NT; ++j) acc[g][j] = mfma16x16x32(A[g], as_bf16x8(d.xc[j][4 * c + u]), acc[g][j]);
      }
    }
  }
}

}  // namespace
#endif  // __HIP_DEVICE_COMPILE__

// The SwiGLU kernels of 2-3 token groups are held to 3 waves per SIMD
// (105-159 VGPRs, none spilled): the forward at 32 tokens 78.9 -> 77.5 us
// (hidden 7168), 66.5 -> 65.1 us (hidden 5120). At 4 groups the same cap
// spills 2-6 registers and is not applied.
template <int MODE, int EPI, int NT, int NW, int G>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu((NT == 2 || NT == 3) && EpiTraits<EPI>::swiglu ? 3 : 1)))
void k_stream(GemmArgs args_in) {
#if defined(__HIP_DEVICE_COMPILE__)
  GemmArgs args = args_in;
  int kz = (int)blockIdx.z;  // K split of this workgroup
  if (args.experts > 1) {
    expert_slice(args, blockIdx.z);  // grouped GEMM: grid z walks the experts (each unsplit)
    kz = 0;
  }
  constexpr int NG = G;
  static_assert(!EpiTraits<EPI>::swiglu || G % 2 == 0, "SwiGLU takes gate/up group pairs");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4;
  const int tl = lane & 15;
  const int64_t K = args.K, T = K / kTileK;
  const int64_t rg0 = (int64_t)blockIdx.x * NG;
  const int64_t tok0 = (int64_t)blockIdx.y * 16 * NT;
  const float alpha = uniform_now(args.alpha);
  const float g2i = EPI == kSwigluNvfp4 ? uniform_now(args.g2_inv) : 0.0f;

  const int64_t M = valid_rows(args);
  StreamSrc<MODE, NT> src;
  src.w = make_rsrc(args.w, (uint32_t)(args.N / kTileRows * T * kTileBytes));
  if constexpr (MODE == kW4A4) {
    src.a = make_rsrc(args.a, (uint32_t)(M * (K / 2)));
    src.s = make_rsrc(args.a_scales, (uint32_t)(M * (K / 16)));
  } else {
    src.a = make_rsrc(args.a, (uint32_t)(M * K * 2));
    src.s = src.a;
  }
  int64_t tok[NT];
  bool tvalid[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    tok[j] = tok0 + 16 * j + tl;
    tvalid[j] = tok[j] < M;
    src.a_row[j] = (uint32_t)(tok[j] * (MODE == kW4A4 ? K / 2 : K * 2));  // past M: out of range
    src.s_row[j] = (uint32_t)(tok[j] * (K / 16));
  }

  f32x4 acc[NG][NT];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Tiles t = wave, wave + NW, ...: one tile in flight per wave (measured
  // faster than two at M = 2..16: fewer outstanding requests stream better,
  // and one register set leaves room for more waves). The scheduling
  // barriers keep the arithmetic after the wait for its tile and the next
  // tile's loads after the arithmetic.
  clear_words(args.zero_ptr, args.zero_n);
  if (args.m_dev != nullptr && tok0 >= M) return;  // no valid row (grouped GEMMs run unsplit)
  // K tiles [t0, t1) of this workgroup's split (all of them without split-K).
  const int nt = (int)T;
  const int ks = args.ksplit;
  const int tper = (nt + ks - 1) / ks;
  const int t0 = kz * tper;
  const int t1 = t0 + tper < nt ? t0 + tper : nt;
  int t = t0 + wave;
  StreamTile<MODE, NG, NT> ta;
  stream_load<MODE, NG, NT>(ta, src, rg0, nt, t1, t, lane);
  while (t < t1) {
    stream_compute<MODE, NG, NT>(acc, ta);
    __builtin_amdgcn_sched_barrier(0);
    t += NW;
    stream_load<MODE, NG, NT>(ta, src, rg0, nt, t1, t, lane);
    __builtin_amdgcn_sched_barrier(0);
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
          const f32x4 p = red[w][g * NT + j][lane];
          acc[g][j] = f32x4{acc[g][j][0] + p[0], acc[g][j][1] + p[1], acc[g][j][2] + p[2],
                            acc[g][j][3] + p[3]};
        }
  }

  if constexpr (!EpiTraits<EPI>::swiglu) {
    if (ks > 1) {
      const int64_t unit = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
      if (!splitk_last<NG * NT>(reinterpret_cast<f32x4(&)[NG * NT]>(acc), args.part, args.counters, ks, unit,
                                kz, lane))
        return;
    }
  }
  if constexpr (EpiTraits<EPI>::swiglu) {
    const int64_t I = args.N / 2;
#pragma unroll
    for (int pp = 0; pp < NG / 2; ++pp)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        store_swiglu<EPI>(acc[2 * pp][j], acc[2 * pp + 1][j], row_alpha(alpha, args.row_scale, tvalid[j], tok[j]),
                          g2i, tvalid[j], tok[j], (rg0 / 2 + pp) * kTileRows, lane, I, args.out, args.out_scales,
                          args.h_prescale);
  } else {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        store_dense<EPI>(acc[g][j], row_alpha(alpha, args.row_scale, tvalid[j], tok[j]), tvalid[j], tok[j],
                         (rg0 + g) * kTileRows + 4 * q, args.N, args.out);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int MODE, int EPI, int NT, int NW, int G>
static hipError_t launch_nt_nw(const GemmArgs& a, hipStream_t s) {
  dim3 grid((unsigned)(a.N / kTileRows / G), (unsigned)((a.M + 16 * NT - 1) / (16 * NT)),
            (unsigned)(a.experts > 1 ? a.experts : a.ksplit));
  k_stream<MODE, EPI, NT, NW, G><<<grid, NW * 64, 0, s>>>(a);
  return hipGetLastError();
}

// Waves per workgroup: 8 for one token group (measured best at M = 2..16
// on the decode shapes), except the W4A16 SwiGLU kernels: their register
// sets (95 VGPRs with one gate/up pair, 155 with two) leave room for 5 or 3
// waves per SIMD, so 8-wave workgroups ran their 1088 or 544 workgroups in
// over two rounds; 4-wave ones fit one round (gate_up at 2 / 4 / 16 tokens,
// hidden 5120: 24.8 / 25.7 / 36.0 -> 24.3 / 25.0 / 33.9 us). The W4A4
// SwiGLU kernel also runs 4-wave workgroups above 8 tokens (gate_up at 16
// tokens 24.1 -> 22.9 us, hidden 5120; 30.7 -> 30.2 us, hidden 7168; at 4
// tokens they were slower, 20.4 -> 20.9 us). 4 waves for more token groups
// (their register sets leave room for fewer waves per SIMD). Row groups per
// workgroup: stream_groups.
template <int MODE, int EPI, int NT>
static hipError_t launch_nt(const GemmArgs& a, hipStream_t s) {
  constexpr bool sw = EpiTraits<EPI>::swiglu;
  if constexpr (NT == 1) {
    constexpr int kNW = MODE == kW4A16 && sw ? 4 : 8;
    if constexpr (MODE == kW4A4 && sw) {
      if (a.M > 8 && stream_groups(MODE, sw, a.M, a.N, a.experts) == 2) return launch_nt_nw<MODE, EPI, NT, 4, 2>(a, s);
    }
    switch (stream_groups(MODE, sw, a.M, a.N, a.experts)) {
      case 1:
        if constexpr (!sw) return launch_nt_nw<MODE, EPI, NT, 8, 1>(a, s);
        break;
      case 2: return launch_nt_nw<MODE, EPI, NT, kNW, 2>(a, s);
      case 4: return launch_nt_nw<MODE, EPI, NT, kNW, 4>(a, s);
      case 5:
        if constexpr (MODE == kW4A16 && !sw) return launch_nt_nw<MODE, EPI, NT, kNW, 5>(a, s);
        break;
      case 7:
        if constexpr (MODE == kW4A16 && !sw) return launch_nt_nw<MODE, EPI, NT, kNW, 7>(a, s);
        break;
      case 8:
        if constexpr (MODE == kW4A16 && !sw) return launch_nt_nw<MODE, EPI, NT, kNW, 8>(a, s);
        break;
    }
    return hipErrorInvalidValue;
  }
  // 2-4 token groups: 2 row groups per workgroup for either epilogue (the
  // dense W4A4 down projection at 64 / 128 tokens, hidden 7168: 71.2 / 138.2
  // -> 41.9 / 79.5 us against 1 row group); 1 when N / 16 is odd (dense only:
  // SwiGLU row groups come in gate/up pairs).
  // At 2 token groups the W4A4 SwiGLU kernel takes two gate/up pairs
  // (forward at 32 tokens 83.6 -> 79.9 us, hidden 7168; 69.7 -> 65.8 us,
  // hidden 5120; mixed at 4 groups).
  if constexpr (!sw) {
    if ((a.N / kTileRows) % 2 != 0) return launch_nt_nw<MODE, EPI, NT, 4, 1>(a, s);
  } else if constexpr (MODE == kW4A4 && NT == 2) {
    if ((a.N / kTileRows) % 4 == 0) return launch_nt_nw<MODE, EPI, NT, 4, 4>(a, s);
  }
  return launch_nt_nw<MODE, EPI, NT, 4, 2>(a, s);
}

}  // namespace nvfp4
