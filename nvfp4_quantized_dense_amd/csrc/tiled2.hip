// tiled2.hip -- 256 x 256 W4A4 GEMM for prefill-sized token counts.
//
// A workgroup computes 256 weight rows x 256 tokens with NWR x NWT waves;
// each wave owns GR row groups x TG token groups of MFMA 16x16x32 f16 tiles.
// Both operands stay in their 4-bit form all the way into LDS: per
// 256-column K tile the packed weight tiles (16 row groups) and the
// activation codes (rearranged into the same lane order) are copied with
// buffer_load ... lds, which writes LDS without passing through VGPRs,
// double-buffered so the next K tile streams in while the current one is
// multiplied. Token rows past M lie past the end of the activation buffers
// and load as zeros (the raw buffer range check covers the per-lane offset);
// row groups past N are clamped to the last group. Fragments are
// dequantized in registers right before the MFMA (exact f16: E2M1 convert +
// packed f16 multiply by the E4M3 scale).
//
// Tile order is XCD-aware: workgroup ids are dealt round-robin to the 8 XCDs,
// so XCD x is given a contiguous run of output tiles, in bands of 4 weight
// tiles swept token-tile-major: the 32 workgroups resident on one XCD cover
// 4 weight tiles x 8 token tiles and read 12 operand panels through its L2
// per round of tiles, not 1 weight panel and all 32 activation panels (all
// of x at 8192 tokens) as a weight-tile-major order does.
//
// One workgroup fits a CU (two 72 KB stages of LDS), so output tiles run in
// rounds of one per CU. When the last round would be at most half full (the
// down projection at 8192 tokens, hidden 7168: 896 tiles, 3.5 rounds), a
// GEMM given split-K buffers runs the whole rounds in one launch and the
// tail tiles in a second one with K split over ks workgroups each, so the
// tail takes 1 / ks of a round (the partials are combined by the last
// workgroup of each tile, in split order, before the epilogue).
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int kG = 16;                               // row groups per workgroup
constexpr int kTG = 16;                              // token groups per workgroup
constexpr int kWBytes = kG * kTileBytes;             // packed weight tiles
constexpr int kACodeBytes = kTG * 2 * 1024;          // activation codes, lane order
constexpr int kAScaleBytes = kTG * 16 * 16;          // 16 scale bytes per token
constexpr int kStageBytes = kWBytes + kACodeBytes + kAScaleBytes;
constexpr int64_t kBandWeightTiles = 4;              // tile order: weight tiles per band

// The buffer-resource type exists only for the device; the host pass sees the
// kernel's signature alone (for its launch stub).
#if defined(__HIP_DEVICE_COMPILE__)
namespace {


typedef __attribute__((address_space(3))) void lds_t;

// Raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor word 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// One wave-wide buffer load into LDS: lane l's SIZE bytes from
// base + soff + voff + IMM land at lds + IMM + SIZE * l (the instruction
// offset moves the LDS address too, so callers keep IMM = 0 and put their
// offsets into soff). SIZE and IMM are literals.
#define NVFP4_DMA(r, SIZE, IMM, voff, soff, lds) \
  __builtin_amdgcn_raw_ptr_buffer_load_lds((r), (lds_t*)(lds), SIZE, (int)(voff), (int)(soff), IMM, 0)

template <int NW>
struct StageSrc {
  static constexpr int kTGPerWave = kTG / NW;  // token groups each wave copies
  __amdgpu_buffer_rsrc_t w, a, s;              // packed weight, activation codes, scales
  uint32_t a_off[kTGPerWave];                  // lane offsets of those token rows
  uint32_t s_off;                              // lane offset of this lane's scale row
};

template <int NW>
__device__ __forceinline__ StageSrc<NW> stage_src(const GemmArgs& a, int64_t M, int64_t tok0, int wave, int lane) {
  StageSrc<NW> o;
  const int64_t T = a.K / kTileK;
  o.w = make_rsrc(a.w, (uint32_t)((a.N / kTileRows) * T * kTileBytes));
  o.a = make_rsrc(a.a, (uint32_t)(M * (a.K / 2)));
  o.s = make_rsrc(a.a_scales, (uint32_t)(M * (a.K / 16)));
  const int q = lane >> 4, tl = lane & 15;
#pragma unroll
  for (int i = 0; i < StageSrc<NW>::kTGPerWave; ++i)
    o.a_off[i] = (uint32_t)((tok0 + 16 * (wave + NW * i) + tl) * (a.K / 2) + q * 16);
  // 256 tokens x 16 scale bytes = 4 wave-wide loads, made by waves 0..3
  o.s_off = (uint32_t)((tok0 + 64 * (wave & 3) + lane) * (a.K / 16));
  return o;
}

// Copy K tile t into one LDS stage. `wave` is wave-uniform, so every scalar
// offset stays in SGPRs.
template <int NW>
__device__ __forceinline__ void issue_stage(const StageSrc<NW>& src, uint8_t* buf, int64_t t, int64_t T,
                                            int64_t rg0, int64_t ngroups, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < kG / NW; ++i) {
    const int g = wave + NW * i;
    // Groups past N are clamped to the last one: the scalar offset is not
    // covered by the buffer range check. Their results are never stored.
    const int64_t grp = min(rg0 + g, ngroups - 1);
    const uint32_t soff = (uint32_t)((grp * T + t) * kTileBytes);
    uint8_t* dst = buf + g * kTileBytes;
    NVFP4_DMA(src.w, 16, 0, 16 * lane, soff, dst);
    NVFP4_DMA(src.w, 16, 0, 16 * lane, soff + 1024, dst + 1024);
    NVFP4_DMA(src.w, 4, 0, 4 * lane, soff + kTileCodeBytes, dst + kTileCodeBytes);
  }
#pragma unroll
  for (int i = 0; i < StageSrc<NW>::kTGPerWave; ++i) {
    uint8_t* dst = buf + kWBytes + (wave + NW * i) * 2048;
    NVFP4_DMA(src.a, 16, 0, src.a_off[i], t * 128, dst);
    NVFP4_DMA(src.a, 16, 0, src.a_off[i], t * 128 + 64, dst + 1024);
  }
  if (wave < 4)
    NVFP4_DMA(src.s, 16, 0, src.s_off, t * 16, buf + kWBytes + kACodeBytes + 64 * wave * 16);
}

// 8 E2M1 codes times an f16 scale pair {s, s}: an MFMA f16 operand.
__device__ __forceinline__ f16x8 deq8_f16x2(uint32_t w, f16x2 s2) {
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  f16x8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

// E4M3 scale bytes 2 HI and 2 HI + 1 of a word as f16 {s0, s1}, one
// instruction for both (E4M3 values are exact in f16).
template <bool HI>
__device__ __forceinline__ f16x2 scale_f16x2(uint32_t sdw) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sdw, 1.0f, HI);
}

// One 128-column chunk (C = 0, 1) of a staged K tile: 4 MFMA K-steps of 32.
// Per step the token fragments are dequantized once, then each weight
// fragment in turn feeds its TG MFMAs.
template <int C, int GR, int TG>
__device__ __forceinline__ void compute_chunk(f32x4 (&acc)[GR][TG], const uint8_t* buf, int g0, int j0,
                                              int lane, const uint32_t* wsd, const uint32_t* xsd) {
  const uint8_t* W = buf;
  const uint8_t* Ac = buf + kWBytes;
  // Scales of this chunk's two 16-blocks (bytes 2C, 2C + 1 of each word),
  // each multiplied as the pair {s, s} (a half-select the multiply encodes).
  f16x2 xsp[TG], wsp[GR];
#pragma unroll
  for (int j = 0; j < TG; ++j) xsp[j] = scale_f16x2<C == 1>(xsd[j]);
#pragma unroll
  for (int g = 0; g < GR; ++g) wsp[g] = scale_f16x2<C == 1>(wsd[g]);
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    // This 16-block's code words (8 bytes per lane of each fragment),
    // read per block rather than per chunk (measured 0.5% faster).
    u32x2 xh[TG], wh[GR];
#pragma unroll
    for (int j = 0; j < TG; ++j)
      xh[j] = *reinterpret_cast<const u32x2*>(Ac + (j0 + j) * 2048 + C * 1024 + 16 * lane + 8 * blk);
#pragma unroll
    for (int g = 0; g < GR; ++g)
      wh[g] = *reinterpret_cast<const u32x2*>(W + (g0 + g) * kTileBytes + C * 1024 + 16 * lane + 8 * blk);
    f16x2 xs[TG], ws[GR];
#pragma unroll
    for (int j = 0; j < TG; ++j) xs[j] = blk ? f16x2{xsp[j].y, xsp[j].y} : f16x2{xsp[j].x, xsp[j].x};
#pragma unroll
    for (int g = 0; g < GR; ++g) ws[g] = blk ? f16x2{wsp[g].y, wsp[g].y} : f16x2{wsp[g].x, wsp[g].x};
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      f16x8 B[TG];
#pragma unroll
      for (int j = 0; j < TG; ++j) B[j] = deq8_f16x2(xh[j][uu], xs[j]);
#pragma unroll
      for (int g = 0; g < GR; ++g) {
        const f16x8 A = deq8_f16x2(wh[g][uu], ws[g]);
#pragma unroll
        for (int j = 0; j < TG; ++j) acc[g][j] = mfma16x16x32(A, B[j], acc[g][j]);
      }
    }
  }
}

}  // namespace
#endif  // __HIP_DEVICE_COMPILE__

// NWR x NWT waves; wave (wr, wt) owns row groups GR*wr.. and token groups TG*wt..
// This launch covers output tiles [tile0, tile0 + count); with SPLIT (dense
// epilogues, args.ksplit > 1) each of them as args.ksplit K splits.
template <int EPI, int NWR, int NWT, bool SPLIT>
__global__ __launch_bounds__(NWR * NWT * 64, 1) void k_tiled2(GemmArgs args_in, int64_t m_tiles, int64_t per_xcd,
                                                              int64_t tile0, int64_t count) {
#if defined(__HIP_DEVICE_COMPILE__)
  GemmArgs args = args_in;
  if (args.experts > 1) expert_slice(args, blockIdx.y);  // grouped GEMM: grid y walks the experts
  constexpr int NW = NWR * NWT;
  constexpr int GR = kG / NWR;
  constexpr int TG = kTG / NWT;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];
  __shared__ uint32_t arrived;
  clear_words(args.zero_ptr, args.zero_n);
  const int ks = SPLIT ? args.ksplit : 1;
  const int64_t id = blockIdx.x;
  const int64_t f = (id & 7) * per_xcd + (id >> 3);
  if (f >= count * ks) return;
  const int64_t local = f / ks;
  const int split = (int)(f - local * ks);
  const int64_t tile = tile0 + local;
  int64_t n_tile, m_tile;
  banded_tile(tile, (args.N / kTileRows + kG - 1) / kG, m_tiles, kBandWeightTiles, n_tile, m_tile);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave / NWT, wt = wave % NWT;
  const int q = lane >> 4, tl = lane & 15;
  const int64_t M = valid_rows(args), N = args.N, T = args.K / kTileK;
  const int64_t ngroups = N / kTileRows;
  const int64_t rg0 = n_tile * kG;
  const int64_t tok0 = m_tile * (kTG * 16);

  f32x4 acc[GR][TG];
#pragma unroll
  for (int g = 0; g < GR; ++g)
#pragma unroll
    for (int j = 0; j < TG; ++j) acc[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K tiles [t0, t1) of this split (all of them without a split).
  const int64_t per = (T + ks - 1) / ks, t0 = split * per, t1 = min(T, t0 + per);
  if (args.m_dev != nullptr && tok0 >= M) return;  // no valid row (grouped GEMMs run unsplit)
  const StageSrc<NW> src = stage_src<NW>(args, M, tok0, wave, lane);
  issue_stage<NW>(src, smem, t0, T, rg0, ngroups, wave, lane);
  for (int64_t t = t0; t < t1; ++t) {
    uint8_t* buf = smem + ((t - t0) & 1) * kStageBytes;
    // This wave's loads of stage t are the only ones outstanding: wait for
    // them, then for every wave's (and for everyone to be done reading the
    // buffer the next stage overwrites).
    __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0), other counters unchanged
    __builtin_amdgcn_s_barrier();
    if (t + 1 < t1) issue_stage<NW>(src, smem + ((t + 1 - t0) & 1) * kStageBytes, t + 1, T, rg0, ngroups, wave, lane);
    uint32_t wsd[GR], xsd[TG];
    const uint8_t* As = buf + kWBytes + kACodeBytes;
#pragma unroll
    for (int g = 0; g < GR; ++g)
      wsd[g] = *reinterpret_cast<const uint32_t*>(buf + (GR * wr + g) * kTileBytes + kTileCodeBytes + 4 * lane);
#pragma unroll
    for (int j = 0; j < TG; ++j) {
      const uint8_t* srow = As + (16 * (TG * wt + j) + tl) * 16;
      xsd[j] = (uint32_t)*reinterpret_cast<const uint16_t*>(srow + 2 * q) |
               ((uint32_t)*reinterpret_cast<const uint16_t*>(srow + 8 + 2 * q) << 16);
    }
    // Raised wave priority over the dequant + MFMA section (measured +1%:
    // a wave that has its stage's operands keeps the matrix core fed ahead
    // of waves still issuing their copies).
    __builtin_amdgcn_s_setprio(1);
    compute_chunk<0, GR, TG>(acc, buf, GR * wr, TG * wt, lane, wsd, xsd);
    compute_chunk<1, GR, TG>(acc, buf, GR * wr, TG * wt, lane, wsd, xsd);
    __builtin_amdgcn_s_setprio(0);
  }

  if constexpr (SPLIT) {
    if (!wg_splitk_last<GR, TG, NW * 64>(acc, args.part, args.counters, ks, local, split, (int)threadIdx.x,
                                         &arrived))
      return;
  }
  const float alpha = *args.alpha;
#pragma unroll
  for (int j = 0; j < TG; ++j) {
    const int64_t token = tok0 + 16 * (TG * wt + j) + tl;
    const bool tv = token < M;
    const float at = row_alpha(alpha, args.row_scale, tv, token);  // per-token factor, if any
    if constexpr (EpiTraits<EPI>::swiglu) {
      const float g2i = (EPI == kSwigluNvfp4) ? *args.g2_inv : 0.0f;
#pragma unroll
      for (int g = 0; g < GR; g += 2) {
        const int64_t grp = rg0 + GR * wr + g;  // gate group (even), up group grp + 1
        store_swiglu<EPI>(acc[g][j], acc[g + 1][j], at, g2i, tv && grp < ngroups, token,
                          (grp >> 1) * kTileRows, lane, N / 2, args.out, args.out_scales);
      }
    } else {
#pragma unroll
      for (int g = 0; g < GR; ++g) {
        const int64_t grp = rg0 + GR * wr + g;
        store_dense<EPI>(acc[g][j], at, tv && grp < ngroups, token, grp * kTileRows + 4 * q, N,
                         args.out);
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int EPI, bool SPLIT>
static hipError_t launch_range(const GemmArgs& a, int64_t m_tiles, int64_t tile0, int64_t count, int ks,
                               hipStream_t s) {
  constexpr int NWR = 2, NWT = 4;
  const int64_t per_xcd = (count * ks + 7) / 8;
  const dim3 grid((unsigned)(8 * per_xcd), (unsigned)(a.experts > 1 ? a.experts : 1));
  k_tiled2<EPI, NWR, NWT, SPLIT><<<grid, NWR * NWT * 64, 0, s>>>(a, m_tiles, per_xcd, tile0, count);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_e(const GemmArgs& a, hipStream_t s) {
  const TileShape ts = tiled2_shape(a.M, a.N);
  const int64_t m_tiles = (a.M + kTG * 16 - 1) / (kTG * 16);
  if (a.ksplit > 1) {
    // Less than a round (dense epilogues): every tile split. More: the whole
    // rounds unsplit, then the tail tiles split.
    if (ts.units < kTiledSlots) {
      if constexpr (EpiTraits<EPI>::swiglu) return hipErrorInvalidValue;
      return launch_range<EPI, true>(a, m_tiles, 0, ts.units, a.ksplit, s);
    }
    const int64_t tail = tiled_tail(ts.units), whole = ts.units - tail;
    if (tail == 0) return hipErrorInvalidValue;  // the split buffers are sized for the tail tiles
    hipError_t e = launch_range<EPI, false>(a, m_tiles, 0, whole, 1, s);
    if (e != hipSuccess) return e;
    GemmArgs t = a;  // counters to clear are cleared by the first launch only
    t.zero_ptr = nullptr;
    t.zero_n = 0;
    return launch_range<EPI, true>(t, m_tiles, whole, tail, a.ksplit, s);
  }
  return launch_range<EPI, false>(a, m_tiles, 0, ts.units, 1, s);
}

TileShape tiled2_shape(int64_t M, int64_t N) {
  const int64_t n_tiles = (N / kTileRows + kG - 1) / kG;
  const int64_t m_tiles = (M + kTG * 16 - 1) / (kTG * 16);
  return TileShape{n_tiles * m_tiles, kG * 16 * kTG * 16, 8};
}

// W4A4 only. Needs the packed weight, codes and scales below 2^31 bytes each
// (32-bit buffer offsets); the caller checks.
hipError_t launch_tiled2_gemm(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (a.experts > 1 && (a.ksplit != 1 || a.experts > 65535)) return hipErrorInvalidValue;
  if (!splitk_valid(a, epi, true)) return hipErrorInvalidValue;
  switch (epi) {
    case kOutF32: return launch_e<kOutF32>(a, s);
    case kOutBF16: return launch_e<kOutBF16>(a, s);
    case kSwigluNvfp4: return launch_e<kSwigluNvfp4>(a, s);
    case kSwigluBF16: return launch_e<kSwigluBF16>(a, s);
    case kSwigluF32: return launch_e<kSwigluF32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
