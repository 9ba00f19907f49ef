// mid.hip -- GEMM for mid token counts (tens to hundreds of tokens), with
// the activation brought into LDS once per workgroup.
//
// In the weight-streaming kernel every wave loads (and, for W4A4,
// dequantizes) the activation fragments of its own K tiles for just the 16
// or 32 weight rows of its workgroup; at 64 tokens that is two thirds of
// its VALU (W4A4), or bf16 slices of more bytes than the weight (W4A16).
// Here a workgroup of 4 waves owns 128 weight rows (8 row groups; wave w:
// groups 2 w and 2 w + 1, a gate/up pair for the SwiGLU epilogues) x 64
// tokens, and all its waves step through the K tiles together:
//
//  * each wave streams its own two weight tiles per K tile into registers
//    (16-byte loads, one K tile ahead) and dequantizes them, as the
//    streaming kernel does (f16 for W4A4, bf16 for W4A16);
//  * each wave also loads one of the 4 token groups' slice of the next K
//    tile and writes it into an LDS image of the 64 tokens x 256 columns
//    (W4A4: dequantized from NVFP4, exact f16; W4A16: the bf16 values as
//    they are), double-buffered, so one barrier per K tile separates
//    writing the next image from reading the current one;
//  * the token fragments of every MFMA are read back from the image.
//
// Token rows past M lie past the end of the activation buffers and load as
// zeros; row groups past N are clamped to the last one and never stored. A
// grouped GEMM runs all its experts in one launch (grid y). With a dense
// epilogue the K tiles of an output tile may be split over several
// workgroups (GemmArgs.ksplit, partial sums in the caller's workspace, added
// in split order by the last workgroup of the tile): mlp_forward's down
// projection, whose few output row tiles (hidden / 128) would otherwise
// leave most CUs idle.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int kMidWaves = 4;
constexpr int kMidRowBytes = 512;           // one token's 256 f16 or bf16 columns

#if defined(__HIP_DEVICE_COMPILE__)
namespace {

// One K tile of one wave: its two weight tiles and its token group's slice
// (W4A4: 16 code bytes and 2 scale bytes per lane and half tile; W4A16: the
// lane's four 16-byte chunks of bf16 per half tile).
template <int MODE>
struct MidLoad {
  u32x4 wc[2][2];
  uint32_t wsd[2];
  u32x4 xc[MODE == kW4A4 ? 2 : 8];
  uint32_t xs[2];
};

// Image offset of 16-byte chunk `chunk` (8 columns, 0..31) of token row r:
// within each 128-column half the chunks sit at (chunk % 16) ^ key(r % 16),
// key swapping the two 2-bit halves of its argument, so that a fragment read
// (lane l: row l % 16, chunk 16 c + 4 (l / 16) + u) by a quarter-wave, and
// by the 16 lanes of equal l % 4, hits 16 distinct 16-byte slots.
__device__ __forceinline__ int mid_key(int r) { return ((r >> 2) & 3) ^ ((r & 3) << 2); }

template <int MODE>
__device__ __forceinline__ void mid_load(MidLoad<MODE>& d, Rsrc w, Rsrc a, Rsrc s, const uint32_t (&gbase)[2],
                                         uint32_t a_lane, uint32_t s_lane, int64_t t, int64_t T, int lane) {
  const bool in = t < T;
  const uint32_t tw = in ? (uint32_t)(t * kTileBytes) : kOutOfRange;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    d.wc[g][0] = bload16_nt(w, tw + 16 * lane, gbase[g]);
    d.wc[g][1] = bload16_nt(w, tw + 1024 + 16 * lane, gbase[g]);
    d.wsd[g] = bload4_nt(w, tw + kTileCodeBytes + 4 * lane, gbase[g]);
  }
  if constexpr (MODE == kW4A4) {
    const uint32_t ta = in ? a_lane + (uint32_t)(t * 128) : kOutOfRange;
    const uint32_t ts = in ? s_lane + (uint32_t)(t * 16) : kOutOfRange;
    d.xc[0] = bload16(a, ta);
    d.xc[1] = bload16(a, ta + 64);
    d.xs[0] = bload2(s, ts);
    d.xs[1] = bload2(s, ts + 8);
  } else {
    // chunks 16 c + 4 q + u of the token row: bytes 256 c + 64 q + 16 u
    const uint32_t ta = in ? a_lane + (uint32_t)(t * 512) : kOutOfRange;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int u = 0; u < 4; ++u) d.xc[4 * c + u] = bload16(a, ta + 256 * c + 16 * u);
  }
}

// This wave's token group (16 rows of the image) from the loaded slice.
template <int MODE>
__device__ __forceinline__ void mid_put(uint8_t* img, const MidLoad<MODE>& d, int wave, int lane) {
  const int q = lane >> 4, tl = lane & 15;
  const int key = mid_key(tl);
  uint8_t* row = img + (16 * wave + tl) * kMidRowBytes;
  if constexpr (MODE == kW4A16) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *reinterpret_cast<u32x4*>(row + 256 * c + 16 * ((4 * q + u) ^ key)) = d.xc[4 * c + u];
    return;
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const f16x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d.xs[c], 1.0f, false);  // blocks 8 c + 2 q, + 1
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const _Float16 sv = (u >> 1) ? sc.y : sc.x;
      *reinterpret_cast<f16x8*>(row + 256 * c + 16 * ((4 * q + u) ^ key)) = deq8_f16(d.xc[c][u], sv);
    }
  }
}

// One K tile: the wave's two weight tiles dequantized in registers, the 4
// token groups' fragments read from the image.
template <int MODE, int TG>
__device__ __forceinline__ void mid_compute(f32x4 (&acc)[2][TG], const MidLoad<MODE>& d, const uint8_t* img,
                                            int lane) {
  const int q = lane >> 4, tl = lane & 15;
  const int key = mid_key(tl);
  if constexpr (MODE == kW4A16) {
    float ws[2][4];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      ws[g][0] = e4m3_to_f32<0>(d.wsd[g]); ws[g][1] = e4m3_to_f32<1>(d.wsd[g]);
      ws[g][2] = e4m3_to_f32<2>(d.wsd[g]); ws[g][3] = e4m3_to_f32<3>(d.wsd[g]);
    }
    const uint8_t* row = img + tl * kMidRowBytes;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sb = 2 * c + (u >> 1);
        const int off = 256 * c + 16 * ((4 * q + u) ^ key);
        bf16x8 B[TG];
#pragma unroll
        for (int j = 0; j < TG; ++j) B[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(row + j * 16 * kMidRowBytes + off));
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const bf16x8 A = deq8_bf16(d.wc[g][c][u], ws[g][sb]);
#pragma unroll
          for (int j = 0; j < TG; ++j) acc[g][j] = mfma16x16x32(A, B[j], acc[g][j]);
        }
      }
    return;
  }
  _Float16 ws[2][4];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d.wsd[g], 1.0f, false);
    const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d.wsd[g], 1.0f, true);
    ws[g][0] = lo.x; ws[g][1] = lo.y; ws[g][2] = hi.x; ws[g][3] = hi.y;
  }
  const uint8_t* row = img + tl * kMidRowBytes;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sb = 2 * c + (u >> 1);
      const int off = 256 * c + 16 * ((4 * q + u) ^ key);
      f16x8 B[TG];
#pragma unroll
      for (int j = 0; j < TG; ++j) B[j] = *reinterpret_cast<const f16x8*>(row + j * 16 * kMidRowBytes + off);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const f16x8 A = deq8_f16(d.wc[g][c][u], ws[g][sb]);
#pragma unroll
        for (int j = 0; j < TG; ++j) acc[g][j] = mfma16x16x32(A, B[j], acc[g][j]);
      }
    }
}

}  // namespace
#endif  // __HIP_DEVICE_COMPILE__

// Grid: 8 * per_xcd workgroups over n_tiles x m_tiles output tiles (128
// rows x 16 TG tokens), times the K splits. Workgroup ids are dealt
// round-robin to the 8 XCDs, so logical workgroup f = (id % 8) * per_xcd +
// id / 8 takes token tile f % m_tiles of its weight tile and split: the
// token tiles of one weight tile run side by side on one XCD and read its
// weight through the same L2; f >= tiles * splits exits. (8-wave workgroups whose two
// halves take alternate K tiles, adding their partial sums in LDS at the
// end, measured slower: gate_up at 64 tokens, hidden 7168, 68.9 against
// 67.2 us.)
template <int MODE, int EPI, int TG>
__global__ __launch_bounds__(kMidWaves * 64, 2) void k_mid(GemmArgs args_in, int64_t m_tiles, int64_t tiles,
                                                           int64_t per_xcd) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(16))) uint8_t img[2][TG * 16 * kMidRowBytes];
  GemmArgs args = args_in;
  clear_words(args.zero_ptr, args.zero_n);
  // Dense epilogues may split K over ks workgroups per output tile; logical
  // workgroup f takes token tile f % m_tiles of split (f / m_tiles) % ks of
  // weight tile f / (m_tiles * ks), so the token tiles that read the same
  // weight bytes stay neighbours.
  const int ks = EpiTraits<EPI>::swiglu ? 1 : args.ksplit;
  const int64_t id = blockIdx.x;
  const int64_t f = (id & 7) * per_xcd + (id >> 3);
  if (f >= tiles * ks) return;
  if (args.experts > 1) expert_slice(args, blockIdx.y);  // grouped GEMM: grid y walks the experts
  const int64_t m_tile = f % m_tiles, rest = f / m_tiles;
  const int split = (int)(rest % ks);
  const int64_t n_tile = rest / ks;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4, tl = lane & 15;
  // Valid token rows: M, or an expert's masked_m (rows past it read as
  // zeros and are not stored; a token tile wholly past it has no work).
  const int64_t M = valid_rows(args), N = args.N, K = args.K, T = K / kTileK;
  const int64_t per = (T + ks - 1) / ks, t0 = split * per, t1 = t0 + per < T ? t0 + per : T;  // this split's K tiles
  const int64_t ngroups = N / kTileRows;
  const int64_t rg = n_tile * 8 + 2 * wave;  // this wave's first row group
  const int64_t tok0 = m_tile * 16 * TG;
  if (tok0 >= M) return;

  const Rsrc w = make_rsrc(args.w, (uint32_t)(ngroups * T * kTileBytes));
  const Rsrc a = make_rsrc(args.a, (uint32_t)(M * (MODE == kW4A4 ? K / 2 : K * 2)));
  const Rsrc s = MODE == kW4A4 ? make_rsrc(args.a_scales, (uint32_t)(M * (K / 16))) : a;
  uint32_t gbase[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int64_t grp = rg + g < ngroups ? rg + g : ngroups - 1;
    gbase[g] = __builtin_amdgcn_readfirstlane((uint32_t)(grp * T * kTileBytes));
  }
  // This wave's token group of the image: rows tok0 + 16 wave + l % 16 (past
  // M: out of range, zeros). With fewer token groups than waves the other
  // waves load no slice (out of range) and put none.
  const int64_t trow = tok0 + 16 * wave + tl;
  const bool puts = wave < TG;
  const uint32_t a_lane = !puts ? kOutOfRange
                          : MODE == kW4A4 ? (uint32_t)(trow * (K / 2) + 16 * q) : (uint32_t)(trow * K * 2 + 64 * q);
  const uint32_t s_lane = puts ? (uint32_t)(trow * (K / 16) + 2 * q) : kOutOfRange;
  const float alpha = uniform_now(args.alpha);
  const float g2i = EPI == kSwigluNvfp4 ? uniform_now(args.g2_inv) : 0.0f;

  f32x4 acc[2][TG];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int j = 0; j < TG; ++j) acc[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K tile t is multiplied from cur (weights) and image t % 2; nxt holds
  // K tile t + 1, whose token slice goes into the other image once the tile
  // t arithmetic is issued; the barrier then publishes it (and frees image
  // t % 2 for K tile t + 2). (Loads two K tiles ahead, in three register
  // sets, measured slower: 242 against 176 VGPRs.)
  MidLoad<MODE> cur, nxt;
  mid_load(cur, w, a, s, gbase, a_lane, s_lane, t0, t1, lane);
  mid_load(nxt, w, a, s, gbase, a_lane, s_lane, t0 + 1, t1, lane);
  if (puts) mid_put(img[0], cur, wave, lane);
  __syncthreads();
  for (int64_t t = t0; t < t1; ++t) {
    const int b = (int)((t - t0) & 1);
    mid_compute<MODE, TG>(acc, cur, img[b], lane);
    if (puts && t + 1 < t1) mid_put(img[b ^ 1], nxt, wave, lane);
    cur = nxt;
    mid_load(nxt, w, a, s, gbase, a_lane, s_lane, t + 2, t1, lane);
    __syncthreads();
  }

  if constexpr (!EpiTraits<EPI>::swiglu) {
    if (ks > 1) {
      __shared__ uint32_t arrived;
      if (!wg_splitk_last<2, TG, kMidWaves * 64>(acc, args.part, args.counters, ks, n_tile * m_tiles + m_tile,
                                                 split, (int)threadIdx.x, &arrived))
        return;
    }
  }

#pragma unroll
  for (int j = 0; j < TG; ++j) {
    const int64_t token = tok0 + 16 * j + tl;
    const bool tv = token < M;
    const float at = row_alpha(alpha, args.row_scale, tv, token);
    if constexpr (EpiTraits<EPI>::swiglu) {
      store_swiglu<EPI>(acc[0][j], acc[1][j], at, g2i, tv && rg < ngroups, token, (rg >> 1) * kTileRows, lane,
                        N / 2, args.out, args.out_scales, args.h_prescale);
    } else {
#pragma unroll
      for (int g = 0; g < 2; ++g)
        store_dense<EPI>(acc[g][j], at, tv && rg + g < ngroups, token, (rg + g) * kTileRows + 4 * q, N, args.out);
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// 128-token tiles (W4A4, dense epilogues): the layout of k_mid with 8 token
// groups, the activation staged per 128-column half of a K tile so that an
// image of 128 tokens fits 32 KB and two of them (double buffer) keep two
// workgroups per CU; each wave puts two token groups and multiplies its two
// weight fragments against 8 token fragments per step. It serves the K-split
// down projection of mlp_forward where 48- or 64-token tiles would leave
// more output tiles than two per CU and no room to split K.
// (As the gate_up kernel it measured slower than 64-token tiles at every
// token count: 177.3 against 151.4 us at 256 tokens, 268.9 against 260.2 at
// 512, hidden 7168.)
#if defined(__HIP_DEVICE_COMPILE__)
namespace {
constexpr int kHalfRowBytes = 256;  // one token's 128 f16 columns

struct MidLoad8 {
  u32x4 wc[2];     // this half of the wave's two weight tiles
  uint32_t wsd[2];
  u32x4 xc[2];     // this half of the wave's two token groups
  uint32_t xs[2];
};

// Half h of the K range (K tile h / 2, columns 128 (h % 2)..); h >= h_end:
// out of range (zeros, no memory access).
__device__ __forceinline__ void mid8_load(MidLoad8& d, Rsrc w, Rsrc a, Rsrc s, const uint32_t (&gbase)[2],
                                          const uint32_t (&a_lane)[2], const uint32_t (&s_lane)[2], int64_t h,
                                          int64_t h_end, int lane) {
  const bool in = h < h_end;
  const int64_t t = h >> 1;
  const int c = (int)(h & 1);
  const uint32_t tw = in ? (uint32_t)(t * kTileBytes) : kOutOfRange;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    d.wc[g] = bload16_nt(w, tw + 1024 * c + 16 * lane, gbase[g]);
    d.wsd[g] = bload4_nt(w, tw + kTileCodeBytes + 4 * lane, gbase[g]);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    d.xc[i] = bload16(a, in ? a_lane[i] + (uint32_t)(t * 128 + 64 * c) : kOutOfRange);
    d.xs[i] = bload2(s, in ? s_lane[i] + (uint32_t)(t * 16 + 8 * c) : kOutOfRange);
  }
}

__device__ __forceinline__ void mid8_put(uint8_t* img, const MidLoad8& d, int wave, int lane) {
  const int q = lane >> 4, tl = lane & 15;
  const int key = mid_key(tl);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint8_t* row = img + (16 * (2 * wave + i) + tl) * kHalfRowBytes;
    const f16x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d.xs[i], 1.0f, false);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const _Float16 sv = (u >> 1) ? sc.y : sc.x;
      *reinterpret_cast<f16x8*>(row + 16 * ((4 * q + u) ^ key)) = deq8_f16(d.xc[i][u], sv);
    }
  }
}

__device__ __forceinline__ void mid8_compute(f32x4 (&acc)[2][8], const MidLoad8& d, const uint8_t* img, int c,
                                             int lane) {
  const int q = lane >> 4, tl = lane & 15;
  const int key = mid_key(tl);
  _Float16 ws[2][2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const f16x2 v = c ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d.wsd[g], 1.0f, true)
                      : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d.wsd[g], 1.0f, false);
    ws[g][0] = v.x; ws[g][1] = v.y;
  }
  const uint8_t* row = img + tl * kHalfRowBytes;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int off = 16 * ((4 * q + u) ^ key);
    f16x8 B[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) B[j] = *reinterpret_cast<const f16x8*>(row + j * 16 * kHalfRowBytes + off);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const f16x8 A = deq8_f16(d.wc[g][u], ws[g][u >> 1]);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[g][j] = mfma16x16x32(A, B[j], acc[g][j]);
    }
  }
}
}  // namespace
#endif  // __HIP_DEVICE_COMPILE__

template <int EPI>
__global__ __launch_bounds__(kMidWaves * 64, 2) void k_mid8(GemmArgs args_in, int64_t m_tiles, int64_t tiles,
                                                            int64_t per_xcd) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(16))) uint8_t img[2][128 * kHalfRowBytes];
  GemmArgs args = args_in;
  clear_words(args.zero_ptr, args.zero_n);
  const int ks = EpiTraits<EPI>::swiglu ? 1 : args.ksplit;
  const int64_t id = blockIdx.x;
  const int64_t f = (id & 7) * per_xcd + (id >> 3);
  if (f >= tiles * ks) return;
  if (args.experts > 1) expert_slice(args, blockIdx.y);
  const int64_t m_tile = f % m_tiles, rest = f / m_tiles;
  const int split = (int)(rest % ks);
  const int64_t n_tile = rest / ks;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4, tl = lane & 15;
  const int64_t M = valid_rows(args), N = args.N, K = args.K, T = K / kTileK;
  const int64_t per = (T + ks - 1) / ks, t0 = split * per, t1 = t0 + per < T ? t0 + per : T;
  const int64_t ngroups = N / kTileRows;
  const int64_t rg = n_tile * 8 + 2 * wave;
  const int64_t tok0 = m_tile * 128;
  if (tok0 >= M) return;

  const Rsrc w = make_rsrc(args.w, (uint32_t)(ngroups * T * kTileBytes));
  const Rsrc a = make_rsrc(args.a, (uint32_t)(M * (K / 2)));
  const Rsrc s = make_rsrc(args.a_scales, (uint32_t)(M * (K / 16)));
  uint32_t gbase[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int64_t grp = rg + g < ngroups ? rg + g : ngroups - 1;
    gbase[g] = __builtin_amdgcn_readfirstlane((uint32_t)(grp * T * kTileBytes));
  }
  uint32_t a_lane[2], s_lane[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t trow = tok0 + 16 * (2 * wave + i) + tl;
    a_lane[i] = (uint32_t)(trow * (K / 2) + 16 * q);
    s_lane[i] = (uint32_t)(trow * (K / 16) + 2 * q);
  }
  const float alpha = uniform_now(args.alpha);
  const float g2i = EPI == kSwigluNvfp4 ? uniform_now(args.g2_inv) : 0.0f;

  f32x4 acc[2][8];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t h0 = 2 * t0, h1 = 2 * t1;
  MidLoad8 cur, nxt;
  mid8_load(cur, w, a, s, gbase, a_lane, s_lane, h0, h1, lane);
  mid8_load(nxt, w, a, s, gbase, a_lane, s_lane, h0 + 1, h1, lane);
  mid8_put(img[0], cur, wave, lane);
  __syncthreads();
  for (int64_t h = h0; h < h1; ++h) {
    const int b = (int)((h - h0) & 1);
    mid8_compute(acc, cur, img[b], (int)(h & 1), lane);
    if (h + 1 < h1) mid8_put(img[b ^ 1], nxt, wave, lane);
    cur = nxt;
    mid8_load(nxt, w, a, s, gbase, a_lane, s_lane, h + 2, h1, lane);
    __syncthreads();
  }

  if constexpr (!EpiTraits<EPI>::swiglu) {
    if (ks > 1) {
      __shared__ uint32_t arrived;
      if (!wg_splitk_last<2, 8, kMidWaves * 64>(acc, args.part, args.counters, ks, n_tile * m_tiles + m_tile,
                                                split, (int)threadIdx.x, &arrived))
        return;
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t token = tok0 + 16 * j + tl;
    const bool tv = token < M;
    const float at = row_alpha(alpha, args.row_scale, tv, token);
    if constexpr (EpiTraits<EPI>::swiglu) {
      store_swiglu<EPI>(acc[0][j], acc[1][j], at, g2i, tv && rg < ngroups, token, (rg >> 1) * kTileRows, lane,
                        N / 2, args.out, args.out_scales, args.h_prescale);
    } else {
#pragma unroll
      for (int g = 0; g < 2; ++g)
        store_dense<EPI>(acc[g][j], at, tv && rg + g < ngroups, token, (rg + g) * kTileRows + 4 * q, N, args.out);
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int EPI>
static hipError_t mid8_launch(const GemmArgs& a, hipStream_t s) {
  const int64_t m_tiles = (a.M + 127) / 128;
  const int64_t tiles = (a.N / kTileRows + 7) / 8 * m_tiles;
  const int64_t per_xcd = (tiles * (a.ksplit > 1 ? a.ksplit : 1) + 7) / 8;
  const unsigned ex = a.experts > 1 ? (unsigned)a.experts : 1u;
  k_mid8<EPI><<<dim3((unsigned)(8 * per_xcd), ex), kMidWaves * 64, 0, s>>>(a, m_tiles, tiles, per_xcd);
  return hipGetLastError();
}

template <int MODE, int EPI, int TG>
static hipError_t mid_launch_tg(const GemmArgs& a, hipStream_t s) {
  const int64_t m_tiles = (a.M + 16 * TG - 1) / (16 * TG);
  const int64_t tiles = (a.N / kTileRows + 7) / 8 * m_tiles;
  const int64_t per_xcd = (tiles * (a.ksplit > 1 ? a.ksplit : 1) + 7) / 8;
  const unsigned ex = a.experts > 1 ? (unsigned)a.experts : 1u;
  k_mid<MODE, EPI, TG><<<dim3((unsigned)(8 * per_xcd), ex), kMidWaves * 64, 0, s>>>(a, m_tiles, tiles, per_xcd);
  return hipGetLastError();
}

// Token tiles of 48 where they pad M no more than tiles of 64 do (48-token
// workgroups also fit three to a CU against two): W4A4 gate_up at 96 / 144 /
// 192 tokens, hidden 7168, 97.0 / 119.9 / 121.8 us with 64-token tiles
// against 71.2 / 98.1 / 113.9; at 64 / 256 / 512 tokens the 64-token tiles
// win (64.4 / 152.0 / 274.4 against 71.0 / 163.2 / 293.0 us).
// Token groups per tile: 3 or 4 as above, except for one-expert W4A4 GEMMs
// with a dense epilogue whose 48- or 64-token grid has more than 256 tiles
// (two per CU, so no room for a K split): 8 (k_mid8). The forward at hidden
// 7168 / 5120 (same box, same run): 257 tokens 306.6 -> 274.6 us (7168),
// 320: 329.6 -> 294.2 (7168), 384: 357.1 / 262.6 -> 326.6 / 233.7, 512:
// 424.9 / 314.2 -> 422.0 / 299.1; where the smaller tiles still split, they
// win (257 tokens at 5120: 187.8 against 198.8 us).
static int mid_tg(int mode, bool dense, int64_t M, int64_t N, int experts) {
  const int64_t pad48 = (M + 47) / 48 * 48, pad64 = (M + 63) / 64 * 64;
  const int tg = pad48 <= pad64 ? 3 : 4;
  if (mode == kW4A4 && dense && experts <= 1 &&
      (N / kTileRows + 7) / 8 * ((M + 16 * tg - 1) / (16 * tg)) > 256)
    return 8;
  return tg;
}

template <int MODE, int EPI>
static hipError_t mid_launch(const GemmArgs& a, hipStream_t s) {
  const int tg = mid_tg(MODE, !EpiTraits<EPI>::swiglu, a.M, a.N, a.experts);
  if constexpr (MODE == kW4A4 && !EpiTraits<EPI>::swiglu) {
    if (tg == 8) return mid8_launch<EPI>(a, s);
  }
  return tg == 3 ? mid_launch_tg<MODE, EPI, 3>(a, s) : mid_launch_tg<MODE, EPI, 4>(a, s);
}

// Output tiles of a one-expert dense GEMM on the mid-size kernels and the
// floats of one tile's partial sums in a K split (256 threads x 2 row
// groups x TG token groups x 4).
TileShape mid_shape(int mode, int64_t M, int64_t N) {
  const int tg = mid_tg(mode, true, M, N, 1);
  return TileShape{(N / kTileRows + 7) / 8 * ((M + 16 * tg - 1) / (16 * tg)), 2048 * tg, kMidWaves};
}

// K splits run for dense epilogues of one-expert GEMMs only.
bool mid_supported(const GemmArgs& a) { return a.ksplit == 1 || a.experts <= 1; }

template <int MODE>
static hipError_t mid_launch_m(int epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case kOutF32: return mid_launch<MODE, kOutF32>(a, s);
    case kOutBF16: return mid_launch<MODE, kOutBF16>(a, s);
    case kSwigluNvfp4: return mid_launch<MODE, kSwigluNvfp4>(a, s);
    case kSwigluBF16: return mid_launch<MODE, kSwigluBF16>(a, s);
    case kSwigluF32: return mid_launch<MODE, kSwigluF32>(a, s);
  }
  return hipErrorInvalidValue;
}

// Unsplit; several experts (grid y, dense epilogues, each expert's valid
// rows from masked_m) or one. Needs each expert's packed weight and
// activation rows below 2^31 bytes (32-bit buffer offsets); the caller
// checks.
hipError_t launch_mid_gemm(int mode, int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (!mid_supported(a)) return hipErrorInvalidValue;
  if (a.ksplit > 1 && (epi != kOutF32 && epi != kOutBF16)) return hipErrorInvalidValue;
  if (a.ksplit > 1 && (a.part == nullptr || a.counters == nullptr)) return hipErrorInvalidValue;
  return mode == kW4A4 ? mid_launch_m<kW4A4>(epi, a, s) : mid_launch_m<kW4A16>(epi, a, s);
}

}  // namespace nvfp4
