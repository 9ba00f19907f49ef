// tiled16.hip -- 256 x 128 W4A16 GEMM for prefill-sized token counts.
//
// W4A16 multiplies bf16 activations by NVFP4 weights (the pages' W4A16
// path: PR #35120 report, implementation breakdown items 2 and 3), so only
// the weights need dequantizing: the activation fragments go to the bf16
// MFMA as loaded. A workgroup computes 256 weight rows (16 row groups) x 128
// tokens (8 token groups) with 8 waves; wave w owns row groups 2 w, 2 w + 1
// and all 8 token groups: 16 MFMA 16x16x32 tiles. The dequantization of a
// weight fragment (16 VALU instructions per 8 codes: convert to f32,
// multiply by the E4M3 scale, pack to bf16; exact, q * s has at most 6
// significant bits) is shared by the 8 MFMAs of its row group, 2 VALU per
// MFMA; measured against 4 per MFMA with 4 x 4 wave tiles (38% of the bf16
// peak against 45-47% here at 4096 tokens) and against 1 wave per SIMD
// with 4 x 8 tiles (33%).
//
// K is staged in halves of a packed K tile (128 columns): the 16 weight
// tiles' code halves and scale blocks, and the 128 tokens x 128 bf16
// columns of activations, copied by buffer_load ... lds (no VGPRs) into one
// of two LDS stages (52 KB each) while the other is multiplied (three
// stages measured slower). Token rows past M lie past the end of the
// activation buffer and load as zeros; row groups past N are clamped to the
// last group and never stored. Output tiles are dealt to each XCD in bands
// of 4 token tiles swept weight-tile-major, so the XCD's 32 resident
// workgroups cover 4 token tiles x 8 weight tiles and read 12 operand
// panels through its L2 per round, not 1 activation panel and 32 weight
// panels (the bf16 activation tile is 3.6x the bytes of a weight tile per K
// column).
//
// Activation layout in LDS: token row r takes 256 bytes, its sixteen 16-byte
// chunks (8 columns each) stored at slot chunk ^ key(r % 16), where key swaps
// the two 2-bit halves of its argument. A fragment read has lane l read row
// l % 16 at chunk 4 (l / 16) + u: the 16 lanes of each quarter-wave, and also
// the 16 lanes of equal l % 4, then hit 16 distinct slots (all banks once).
// Measured with rocprofv3's LDS bank-conflict counter: with key(r) = r (only
// the first grouping conflict-free) 48% of LDS cycles were conflicts and the
// kernel ran at 45% of the bf16 peak; with this key, none, and 50%. The copy
// assigns each lane the chunk that lands in its slot.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

namespace {
constexpr int kG16 = 16;                         // row groups per workgroup
constexpr int kTG16 = 8;                         // token groups per workgroup
constexpr int kNW16 = 8;                         // waves: wave w has row groups 2 w, 2 w + 1
constexpr int kW16Bytes = kG16 * 1024;           // code halves of the weight tiles
constexpr int kS16Bytes = kG16 * 256;            // scale blocks of the weight tiles
constexpr int kA16Bytes = kTG16 * 16 * 256;      // 128 tokens x 128 bf16
constexpr int kStage16 = kW16Bytes + kS16Bytes + kA16Bytes;
constexpr int64_t kBandTokenTiles = 4;           // tile order: token tiles per band
}  // namespace

#if defined(__HIP_DEVICE_COMPILE__)
namespace {

typedef __attribute__((address_space(3))) void lds16_t;

// One wave-wide buffer load into LDS (lane l's SIZE bytes land at
// lds + SIZE * l).
#define NVFP4_DMA16(r, SIZE, voff, soff, lds) \
  __builtin_amdgcn_raw_ptr_buffer_load_lds((r), (lds16_t*)(lds), SIZE, (int)(voff), (int)(soff), 0, 0)

struct Stage16Src {
  Rsrc w, a;
  uint32_t a_voff[4];  // lane offset of this lane's activation chunk, by copy index % 4
};

__device__ __forceinline__ Stage16Src stage16_src(const GemmArgs& a, int64_t M, int lane) {
  Stage16Src o;
  const int64_t T = a.K / kTileK;
  o.w = make_rsrc(a.w, (uint32_t)((a.N / kTileRows) * T * kTileBytes));
  o.a = make_rsrc(a.a, (uint32_t)(M * a.K * 2));
  // Copy i of a wave moves 4 token rows (4 (4 w + i) + lane / 16); lane l
  // fills slot l % 16 of its row, i.e. chunk (l % 16) ^ key(row % 16), and
  // row % 16 = 4 i + l / 16, so key = i ^ 4 (l / 16).
  const int rsub = lane >> 4, slot = lane & 15;
#pragma unroll
  for (int m = 0; m < 4; ++m)
    o.a_voff[m] = (uint32_t)(rsub * a.K * 2 + 16 * (slot ^ m ^ (rsub << 2)));
  return o;
}

// Copy stage s (K tile s / 2, half s % 2) into buf. Wave w copies weight
// groups w and w + 8 and token rows [16 w, 16 w + 16).
__device__ __forceinline__ void issue_stage16(const Stage16Src& src, uint8_t* buf, int64_t s, int64_t T,
                                              int64_t K, int64_t rg0, int64_t ngroups, int64_t tok0, int wave,
                                              int lane) {
  const int64_t t = s >> 1, c = s & 1;
#pragma unroll
  for (int i = 0; i < kG16 / kNW16; ++i) {
    const int g = wave + kNW16 * i;
    const int64_t grp = min(rg0 + g, ngroups - 1);
    const uint32_t tb = (uint32_t)((grp * T + t) * kTileBytes);
    NVFP4_DMA16(src.w, 16, 16 * lane, tb + (uint32_t)(c * 1024), buf + g * 1024);
    NVFP4_DMA16(src.w, 4, 4 * lane, tb + kTileCodeBytes, buf + kW16Bytes + g * 256);
  }
  uint8_t* abuf = buf + kW16Bytes + kS16Bytes;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = 4 * wave + i;  // rows 4 blk .. 4 blk + 3 of the tile
    // The whole offset, token row included, goes into the per-lane offset,
    // which the buffer range check covers: rows past the valid ones read
    // zeros and nothing past the end of the activations is touched.
    const uint32_t voff = src.a_voff[i & 3] + (uint32_t)((tok0 + 4 * blk) * K * 2 + t * 512 + c * 256);
    NVFP4_DMA16(src.a, 16, voff, 0u, abuf + blk * 1024);
  }
}

// The 4 K steps of one staged half (C = 0, 1). Per step: the 8 activation
// fragments (lane l: token 16 j + l % 16, chunk 4 q + u), then per row group
// its dequantized weight fragment and 8 MFMAs.
template <int C>
__device__ __forceinline__ void compute_stage16(f32x4 (&acc)[2][8], const uint8_t* buf, int wave, int lane) {
  const int q = lane >> 4, tl = lane & 15;
  u32x4 wc[2];
  uint32_t wsd[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    wc[g] = *reinterpret_cast<const u32x4*>(buf + (2 * wave + g) * 1024 + 16 * lane);
    wsd[g] = *reinterpret_cast<const uint32_t*>(buf + kW16Bytes + (2 * wave + g) * 256 + 4 * lane);
  }
  const uint8_t* arow = buf + kW16Bytes + kS16Bytes + tl * 256;
  const int key = (tl >> 2) ^ ((tl & 3) << 2);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint8_t* ap = arow + 16 * ((4 * q + u) ^ key);
    bf16x8 B[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) B[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(ap + j * 4096));
    float ws[2];
#pragma unroll
    for (int g = 0; g < 2; ++g)
      ws[g] = (u >> 1) ? e4m3_to_f32<2 * C + 1>(wsd[g]) : e4m3_to_f32<2 * C>(wsd[g]);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const bf16x8 A = deq8_bf16(wc[g][u], ws[g]);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[g][j] = mfma16x16x32(A, B[j], acc[g][j]);
    }
  }
}


}  // namespace
#endif  // __HIP_DEVICE_COMPILE__

// SPLIT: compiled with the K-split combine (ksplit > 1). A separate
// instantiation: with the combine merely present, the main loop of the
// unsplit down projection compiled 23% slower (861 against 699 us at 4096
// tokens, hidden 5120). This launch covers output tiles [tile0, tile0 +
// count); with SPLIT each of them as args.ksplit K splits.
template <int EPI, bool SPLIT>
__global__ __launch_bounds__(kNW16 * 64, 1) void k_tiled16(GemmArgs args_in, int64_t n_tiles, int64_t per_xcd,
                                                           int64_t tile0, int64_t count) {
#if defined(__HIP_DEVICE_COMPILE__)
  GemmArgs args = args_in;
  if (args.experts > 1) expert_slice(args, blockIdx.y);  // grouped GEMM: grid y walks the experts
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage16];
  __shared__ uint32_t arrived;
  clear_words(args.zero_ptr, args.zero_n);
  // XCD-aware order: workgroup ids are dealt round-robin to the 8 XCDs, so
  // XCD x takes a contiguous run of output tiles, in bands of 4 token tiles
  // (banded_tile). With a K split, the ks splits of an output tile are
  // consecutive.
  const int ks = SPLIT ? args.ksplit : 1;
  const int64_t id = blockIdx.x;
  const int64_t f = (id & 7) * per_xcd + (id >> 3);
  if (f >= count * ks) return;
  const int64_t local = f / ks;
  const int split = (int)(f - local * ks);
  const int64_t tile = tile0 + local;
  int64_t m_tile, n_tile;
  banded_tile(tile, (args.M + kTG16 * 16 - 1) / (kTG16 * 16), n_tiles, kBandTokenTiles, m_tile, n_tile);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4, tl = lane & 15;
  const int64_t M = valid_rows(args), N = args.N, K = args.K, T = K / kTileK;
  const int64_t ngroups = N / kTileRows;
  const int64_t rg0 = n_tile * kG16;
  const int64_t tok0 = m_tile * (kTG16 * 16);
  const float alpha = uniform_now(args.alpha);
  const float g2i = EPI == kSwigluNvfp4 ? uniform_now(args.g2_inv) : 0.0f;

  f32x4 acc[2][8];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K tiles [t0, t1) of this split (all of them without a split).
  const int64_t per = (T + ks - 1) / ks, t0 = split * per, t1 = min(T, t0 + per);
  if (args.m_dev != nullptr && tok0 >= M) return;  // no valid row (grouped GEMMs run unsplit)
  const Stage16Src src = stage16_src(args, M, lane);
  issue_stage16(src, smem, 2 * t0, T, K, rg0, ngroups, tok0, wave, lane);
  for (int64_t s = 2 * t0; s < 2 * t1; s += 2) {
    // Two halves per trip (C = 0 in stage buffer 0, C = 1 in buffer 1).
    __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): this wave's copies of stage s
    __builtin_amdgcn_s_barrier();
    issue_stage16(src, smem + kStage16, s + 1, T, K, rg0, ngroups, tok0, wave, lane);
    __builtin_amdgcn_s_setprio(1);
    compute_stage16<0>(acc, smem, wave, lane);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0x3F70);
    __builtin_amdgcn_s_barrier();
    if (s + 2 < 2 * t1) issue_stage16(src, smem, s + 2, T, K, rg0, ngroups, tok0, wave, lane);
    __builtin_amdgcn_s_setprio(1);
    compute_stage16<1>(acc, smem + kStage16, wave, lane);
    __builtin_amdgcn_s_setprio(0);
  }
  if constexpr (SPLIT) {
    if (!wg_splitk_last<2, 8, kNW16 * 64>(acc, args.part, args.counters, ks, local, split, (int)threadIdx.x, &arrived))
      return;
  }

#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t token = tok0 + 16 * j + tl;
    const bool tv = token < M;
    if constexpr (EpiTraits<EPI>::swiglu) {
      const int64_t grp = rg0 + 2 * wave;  // gate group (even), up group grp + 1
      store_swiglu<EPI>(acc[0][j], acc[1][j], alpha, g2i, tv && grp < ngroups, token,
                        (grp >> 1) * kTileRows, lane, N / 2, args.out, args.out_scales, args.h_prescale);
    } else {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int64_t grp = rg0 + 2 * wave + g;
        store_dense<EPI>(acc[g][j], alpha, tv && grp < ngroups, token, grp * kTileRows + 4 * q, N, args.out);
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

TileShape tiled16_shape(int64_t M, int64_t N) {
  const int64_t n_tiles = (N / kTileRows + kG16 - 1) / kG16;
  const int64_t m_tiles = (M + kTG16 * 16 - 1) / (kTG16 * 16);
  return TileShape{n_tiles * m_tiles, kG16 * 16 * kTG16 * 16, kNW16};
}

template <int EPI, bool SPLIT>
static hipError_t launch16_range(const GemmArgs& a, int64_t n_tiles, int64_t tile0, int64_t count, int ks,
                                 hipStream_t s) {
  const int64_t per_xcd = (count * ks + 7) / 8;
  const dim3 grid((unsigned)(8 * per_xcd), (unsigned)(a.experts > 1 ? a.experts : 1));
  k_tiled16<EPI, SPLIT><<<grid, kNW16 * 64, 0, s>>>(a, n_tiles, per_xcd, tile0, count);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch16_e(const GemmArgs& a, hipStream_t s) {
  const int64_t n_tiles = (a.N / kTileRows + kG16 - 1) / kG16;
  const int64_t units = tiled16_shape(a.M, a.N).units;
  if (a.ksplit > 1) {
    // Less than a round (dense epilogues): every tile split. More: the whole
    // rounds unsplit, then the tail tiles split.
    if (units < kTiledSlots) {
      if constexpr (EpiTraits<EPI>::swiglu) return hipErrorInvalidValue;
      return launch16_range<EPI, true>(a, n_tiles, 0, units, a.ksplit, s);
    }
    const int64_t tail = tiled_tail(units), whole = units - tail;
    if (tail == 0) return hipErrorInvalidValue;  // the split buffers are sized for the tail tiles
    hipError_t e = launch16_range<EPI, false>(a, n_tiles, 0, whole, 1, s);
    if (e != hipSuccess) return e;
    GemmArgs t = a;  // counters to clear are cleared by the first launch only
    t.zero_ptr = nullptr;
    t.zero_n = 0;
    return launch16_range<EPI, true>(t, n_tiles, whole, tail, a.ksplit, s);
  }
  return launch16_range<EPI, false>(a, n_tiles, 0, units, 1, s);
}

// W4A16 only. Needs the packed weight below 2^31 bytes and the activation
// rows, with 256 rows of padding past M, below 2^31 bytes (32-bit buffer
// offsets); the caller checks.
hipError_t launch_tiled16_gemm(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (a.experts > 1 && (a.ksplit != 1 || a.experts > 65535)) return hipErrorInvalidValue;
  if (!splitk_valid(a, epi, true)) return hipErrorInvalidValue;
  switch (epi) {
    case kOutF32: return launch16_e<kOutF32>(a, s);
    case kOutBF16: return launch16_e<kOutBF16>(a, s);
    case kSwigluNvfp4: return launch16_e<kSwigluNvfp4>(a, s);
    case kSwigluBF16: return launch16_e<kSwigluBF16>(a, s);
    case kSwigluF32: return launch16_e<kSwigluF32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
