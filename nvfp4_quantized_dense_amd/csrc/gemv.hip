// gemv.hip -- VALU GEMV for W4A16 at the smallest token counts (decode).
//
// The weight streams with 16-byte loads; the arithmetic is on the vector ALU
// with packed dot products: codes are widened exactly (E2M1 -> bf16, two per
// instruction), multiplied against the bf16 activation pairs with
// v_dot2_f32_bf16 (products of a grid value and a bf16 value are exact in
// fp32), and each 16-element block sum is scaled once by its E4M3 factor.
// (W4A4 runs on the FP4 matrix core instead, in fp4gemv.hip.)
//
// Lane l owns row l % 16 of each row group and columns 32 (l / 16) + [0, 32)
// of each 128-column half tile (the packed layout's lane order). NW waves
// divide a row group's K tiles; each wave has one tile in flight at a time
// (past the last tile the load is out of range: zeros without a memory
// access, and never computed). The workgroup's MT token rows are
// staged once in LDS (rows past M read as zeros): their reads then wait on
// the LDS counter, not behind the weight prefetch on the in-order vector
// memory counter. The four lanes of a row and the NW waves are summed at the
// end in a fixed order.
#include "gemv_tile.h"

namespace nvfp4 {

template <int EPI, int MT, int NW>
__global__ __launch_bounds__(NW * 64) void k_valu_gemv(GemmArgs args) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NG = EpiTraits<EPI>::swiglu ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4;
  const int64_t K = args.K, T = K / kTileK;
  const int64_t rg0 = (int64_t)blockIdx.x * NG;
  const int64_t tok0 = (int64_t)blockIdx.y * MT;

  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];  // MT rows of K bf16, 16 spare bytes
  GemvSrc src;
  src.w = make_rsrc(args.w, (uint32_t)(args.N / kTileRows * T * kTileBytes));
  src.a = make_rsrc(args.a, (uint32_t)(args.M * K * 2));

  float acc[NG][MT];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[g][m] = 0.0f;

  clear_words(args.zero_ptr, args.zero_n);
  const float alpha = uniform_now(args.alpha);
  const float g2i = EPI == kSwigluNvfp4 ? uniform_now(args.g2_inv) : 0.0f;
  // K tiles [t0, t1): all of them (the staging and loop are written for a
  // tile range).
  const int nt = (int)T;
  const int t0 = 0, t1 = nt;
  int t = t0 + wave;
  GemvTile<NG> ta;
  {
    // Staging of tiles [t0, t1) of the token rows in 16-byte chunks (rows
    // past M start past the end of the buffer and read as zeros), at their
    // place in full rows of K bf16. The first four chunks per thread are
    // requested before the first weight tile, so that writing them to LDS
    // waits for these loads only (the vector memory counter is in order),
    // not for the weights.
    const int row_chunks = (t1 - t0) * 32;
    const int chunks = MT * row_chunks;
    const uint32_t sink = (uint32_t)(MT * K * 2);
    constexpr int kStride = NW * 64;
    u32x4 v[4];
    auto offsets = [&](int i, uint32_t& g, uint32_t& l) {
      const int m = i / row_chunks, j = i - m * row_chunks;
      g = (uint32_t)((tok0 + m) * K * 2) + (uint32_t)(t0 * 512 + 16 * j);
      l = (uint32_t)(m * K * 2) + (uint32_t)(t0 * 512 + 16 * j);
    };
    auto fetch = [&](int base) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + u * kStride;
        uint32_t g = kOutOfRange, l;
        if (i < chunks) offsets(i, g, l);
        v[u] = bload16(src.a, g);
      }
    };
    // Every fetched value is written (a chunk past the end loaded zeros and
    // goes to the 16 spare bytes after the rows), so no load is left pending
    // with its register free for reuse: reusing one would wait for all
    // later loads.
    auto store = [&](int base) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + u * kStride;
        uint32_t g, l = sink;
        if (i < chunks) offsets(i, g, l);
        *reinterpret_cast<u32x4*>(xs + l) = v[u];
      }
    };
    fetch(threadIdx.x);
    gemv_load<NG>(ta, src, rg0, nt, t1, t, lane);
    store(threadIdx.x);
    for (int base = threadIdx.x + 4 * kStride; base < chunks; base += 4 * kStride) {
      fetch(base);
      store(base);
    }
  }
  __syncthreads();

  // One tile in flight per wave (measured faster here than two: fewer
  // outstanding requests stream better). The scheduling barriers keep the
  // arithmetic after the wait for its tile and the next tile's loads after
  // the arithmetic. A tile past the range is never computed.
  while (t < t1) {
    gemv_compute<NG, MT>(acc, ta, xs, nt, t, lane);
    __builtin_amdgcn_sched_barrier(0);
    t += NW;
    gemv_load<NG>(ta, src, rg0, nt, t1, t, lane);
    __builtin_amdgcn_sched_barrier(0);
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
  const int64_t token = tok0 + tl;
  if constexpr (EpiTraits<EPI>::swiglu) {
    store_swiglu<EPI>(res[0], res[1], alpha, g2i, lvalid, token, (int64_t)blockIdx.x * kTileRows,
                      lane, args.N / 2, args.out, args.out_scales, args.h_prescale);
  } else {
    store_dense<EPI>(res[0], alpha, lvalid, token, rg0 * kTileRows + 4 * q, args.N, args.out);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int EPI, int MT, int NW>
static hipError_t launch_mt_nw(const GemmArgs& a, hipStream_t s) {
  constexpr int NG = EpiTraits<EPI>::swiglu ? 2 : 1;
  dim3 grid((unsigned)(a.N / kTileRows / NG), (unsigned)((a.M + MT - 1) / MT));
  k_valu_gemv<EPI, MT, NW><<<grid, NW * 64, (size_t)MT * a.K * 2 + 16, s>>>(a);
  return hipGetLastError();
}

// Waves per workgroup: 8 (measured best at the decode shapes, 320 to 1088
// workgroups), 16 for grids too small to spread over the CUs otherwise.
static int valu_waves(int64_t wgs) { return wgs < 128 ? 16 : 8; }

template <int EPI, int MT>
static hipError_t launch_mt(const GemmArgs& a, hipStream_t s) {
  constexpr int NG = EpiTraits<EPI>::swiglu ? 2 : 1;
  const int64_t wgs = a.N / kTileRows / NG * ((a.M + MT - 1) / MT);
  if (valu_waves(wgs) == 16) return launch_mt_nw<EPI, MT, 16>(a, s);
  return launch_mt_nw<EPI, MT, 8>(a, s);
}

// Token rows per workgroup: up to 4, as many as fit the LDS budget.
static int valu_rows(int64_t M, int64_t K) {
  if (M >= 3 && 4 * K * 2 + 16 <= kValuGemvLdsBytes) return 4;
  if (M >= 2 && 2 * K * 2 + 16 <= kValuGemvLdsBytes) return 2;
  return 1;
}

template <int EPI>
static hipError_t launch_me(const GemmArgs& a, hipStream_t s) {
  const int mt = valu_rows(a.M, a.K);
  if (mt == 4) return launch_mt<EPI, 4>(a, s);
  if (mt == 2) return launch_mt<EPI, 2>(a, s);
  return launch_mt<EPI, 1>(a, s);
}

// W4A16 only. Needs the packed weight and the activations below 2^31 bytes
// (32-bit buffer offsets) and one bf16 token row within the LDS budget
// (K * 2 + 16 <= kValuGemvLdsBytes); the caller checks.
hipError_t launch_valu_gemv(int mode, int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (mode != kW4A16 || a.K * 2 + 16 > kValuGemvLdsBytes || a.ksplit != 1) return hipErrorInvalidValue;
  switch (epi) {
    case kOutF32: return launch_me<kOutF32>(a, s);
    case kOutBF16: return launch_me<kOutBF16>(a, s);
    case kSwigluBF16: return launch_me<kSwigluBF16>(a, s);
    case kSwigluF32: return launch_me<kSwigluF32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
