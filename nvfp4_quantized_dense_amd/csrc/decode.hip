// decode.hip -- the W4A4 MLP forward of one token in a single launch:
// NVFP4 quantization of x, gate_up GEMV + SiLU(gate) * up + NVFP4
// re-quantization of h, and the down projection GEMV (the quantized
// DeepseekV2MLP.forward of the sglang PR #26626 digest, key source
// snippets; the NVFP4 encoding is the one nvfp4_quantize documents), with no
// kernel boundary between the two GEMVs: the down projection's weight loads
// start while the gate_up GEMV is still streaming its own.
//
// Two kinds of workgroup, by index:
//   * gate_up units, workgroups [0, I / 16): unit i is the FP4 GEMV of gate
//     rows 16 i.. and up rows 16 i.. over all of H (x quantized as it is
//     staged). It writes the 16 elements of h it owns to the workspace's h
//     (plain stores, as the two-launch path leaves it) and as tagged records
//     for the down units (below), and exits without waiting.
//   * down units, the next (H / 16) * S workgroups: unit (r, s) is the FP4
//     GEMV of output rows 16 r.. over the K tiles of split s. It issues the
//     loads of its weight tiles first, then polls the records of its part of
//     h until every one carries this launch's tag, writing each into its LDS
//     image as it arrives, and runs the GEMV. Units of splits below S - 1
//     store their 16 partial sums as tagged records; the unit of split S - 1
//     polls those, adds the S partials in split order and writes the output.
//
// The records are the tagged 64-bit words of decode_records.h: 32 bits of
// data and the low 32 bits of the launch's epoch, which the host makes new
// for every launch, so a record left by an earlier launch (whose tag differs,
// until 2^32 launches later) is never mistaken for a current one.
//
// Every wait is on workgroups of smaller index, or on gate_up units that
// never wait: each XCD starts its workgroups in index order, so the awaited
// workgroups are running or done whatever the number of resident ones. The
// waits are bounded all the same: one that runs out (which no schedule of
// the hardware produces) writes NaN for the rows of that unit instead of
// hanging, and sets kDecodeWaitExpired in the status word for the host.
#include <algorithm>

#include "decode_records.h"
#include "fp4_tile.h"

namespace nvfp4 {

namespace {
constexpr int kDecodeWaves = 4;
constexpr int kDownSets = 4;         // weight tiles per wave in flight in a down unit
constexpr int kPollWords = 8;        // record words per thread a down unit can poll
// K tiles per down split aimed at: all of a split's weight tiles in the
// wave's registers (kDownSets per wave) before the wait for h.
constexpr int kSplitTiles = kDownSets * kDecodeWaves;
// Down units cover at most this many K tiles (48 record words per tile).
constexpr int kMaxSplitTiles = kPollWords * kDecodeWaves * 64 / 48;

}  // namespace

template <int EPI>
__global__ __launch_bounds__(kDecodeWaves * 64) void k_decode_mlp(DecodeArgs d) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = kDecodeWaves;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = (int)threadIdx.x;
  const int q = lane >> 4;
  extern __shared__ __attribute__((aligned(16))) uint8_t xl[];
  __shared__ float red[NW * 2 * 16];
  const int64_t nA = d.I / kTileRows;
  const bool lvalid = (lane & 15) == 0;  // lanes holding token 0
  const uint32_t tag = (uint32_t)d.epoch;  // the tag every wait looks for
  const uint32_t ptag = tag ^ d.tag_skew;  // the tag records are written with
  // Records: h codes as 32-bit words (unit u: words 2 u, 2 u + 1 = code
  // bytes 0..3 and 4..7 of its block), then h scales (word u: the scale
  // byte), then the down units' partial sums (unit j, row k: word j * 16 + k).
  uint64_t* rec_codes = d.records;
  uint64_t* rec_scales = d.records + 2 * nA;
  uint64_t* rec_part = d.records + 3 * nA;

  if ((int64_t)blockIdx.x < nA) {
    // ---- gate_up unit i: rows [16 i, 16 i + 16) of gate and of up ----
    GemmArgs g{d.x, nullptr, d.w_gu, 1, 2 * d.I, d.H, d.alpha_gu, d.g2_inv, d.h_codes, d.h_scales};
    g.a_g_inv = d.g1_inv;
    const float alpha = uniform_now(d.alpha_gu), g2i = uniform_now(d.g2_inv);
    f32x4 acc[2][1];
    f4_gemv_acc<2, 1, NW, true>(g, 2 * (int64_t)blockIdx.x, 0, xl, lane, wave, acc);
    f32x4 res[2];
    if (!f4_reduce<2, 1, NW>(acc, red, wave, lane, lvalid, res)) return;
    const SwigluBlock b = swiglu_nvfp4(res[0], res[1], alpha, g2i);
    // Lanes 0, 16, 32, 48 hold the codes of elements 4 q .. 4 q + 3 (code
    // bytes 2 q, 2 q + 1 of the block).
    const uint32_t c16 = (uint32_t)__shfl((int)b.codes, 16), c32 = (uint32_t)__shfl((int)b.codes, 32),
                   c48 = (uint32_t)__shfl((int)b.codes, 48);
    if (lane == 0) {
      const uint32_t lo = (b.codes & 0xFFFFu) | (c16 << 16), hi = (c32 & 0xFFFFu) | (c48 << 16);
      const int64_t i = blockIdx.x;
      put_record(rec_codes + 2 * i, lo, ptag);
      put_record(rec_codes + 2 * i + 1, hi, ptag);
      put_record(rec_scales + i, b.scale, ptag);
      reinterpret_cast<uint32_t*>(d.h_codes)[2 * i] = lo;
      reinterpret_cast<uint32_t*>(d.h_codes)[2 * i + 1] = hi;
      d.h_scales[i] = (uint8_t)b.scale;
    }
    return;
  }

  // ---- down unit (r, s): output rows [16 r, 16 r + 16), K split s ----
  const int64_t j = (int64_t)blockIdx.x - nA;
  const int64_t RG = d.H / kTileRows;
  const int64_t r = j % RG;
  const int s = (int)(j / RG);
  const int T = (int)(d.I / kTileK);
  const int per = (T + d.ksplit - 1) / d.ksplit;
  const int t0 = s * per, t1 = min(T, t0 + per), nts = t1 - t0;
  const int Kl = nts * kTileK;  // columns of the LDS image (this split's part of h)

  const float alpha = uniform_now(d.alpha_d);
  F4Src<1> src;
  src.w = make_rsrc(d.w_d, (uint32_t)(RG * T * kTileBytes));
  f4_slots<1>(src, lane, Kl);
  F4Tile<1, 1> tw[kDownSets];
#pragma unroll
  for (int u = 0; u < kDownSets; ++u) f4_load_w<1, 1>(tw[u], src, r, T, t1, t0 + wave + u * NW, lane);

  // h of tiles [t0, t1): 32 nts code words and 16 nts scale words, word
  // tid + 256 k of them polled by this thread until its tag is current, its
  // data written to the image: codes [0, Kl / 2), zeros [Kl / 2, Kl),
  // scales [Kl, Kl + Kl / 16).
  bool timed_out = false;
  {
    const int ncw = 32 * nts, nw = 48 * nts;
    const uint64_t* cw = rec_codes + 32 * (int64_t)t0;
    const uint64_t* sw = rec_scales + 16 * (int64_t)t0;
    uint32_t pending = 0;
#pragma unroll
    for (int k = 0; k < kPollWords; ++k)
      if (tid + NW * 64 * k < nw) pending |= 1u << k;
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < nts * 8; i += NW * 64)
      *reinterpret_cast<u32x4*>(xl + lds_zero_off(1, Kl) + 16 * i) = z;
    for (int spin = 0;; ++spin) {
#pragma unroll
      for (int k = 0; k < kPollWords; ++k) {
        const int w = tid + NW * 64 * k;
        if (pending & (1u << k)) {
          const uint64_t v = get_record(w < ncw ? cw + w : sw + (w - ncw));
          if ((uint32_t)(v >> 32) == tag) {
            pending &= ~(1u << k);
            if (w < ncw) *reinterpret_cast<uint32_t*>(xl + 4 * w) = (uint32_t)v;
            else xl[Kl + (w - ncw)] = (uint8_t)v;
          }
        }
      }
      if (!__syncthreads_or(pending != 0)) break;
      if (spin >= d.spin_limit) {
        timed_out = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();

  // kDownSets register sets per wave, one tile each, refilled kDownSets * NW
  // tiles ahead (tiles past the split load zeros without memory access).
  f32x4 acc[1][1] = {{f32x4{0.0f, 0.0f, 0.0f, 0.0f}}};
  for (int base = 0; base < nts; base += kDownSets * NW) {
#pragma unroll
    for (int u = 0; u < kDownSets; ++u) {
      const int tl = base + wave + u * NW;  // tile index within the split
      f4_load_x<1, 1>(tw[u], src, xl, nts, tl);
      f4_compute<1, 1>(acc, tw[u]);
      __builtin_amdgcn_sched_barrier(0);
      f4_load_w<1, 1>(tw[u], src, r, T, t1, t0 + tl + kDownSets * NW, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  f32x4 res[1];
  if (!f4_reduce<1, 1, NW>(acc, red, wave, lane, lvalid, res)) return;
  // timed_out is uniform (every thread took the same exit of the poll).
  if (timed_out) {
    res[0] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    if (tid == 0) report_expired(d.status);
  }
  const int64_t row0 = r * kTileRows + 4 * q;
  if (s < d.ksplit - 1) {
    if (lvalid) {
#pragma unroll
      for (int k = 0; k < 4; ++k) put_record(rec_part + j * 16 + 4 * q + k, __float_as_uint(res[0][k]), ptag);
    }
    return;
  }
  if (d.ksplit > 1) {
    // The last split adds the S partials of rows 16 r.. in split order.
    const f32x4 sum = sum_split_partials(rec_part, RG, r, d.ksplit, tag, d.spin_limit, d.status, lane);
#pragma unroll
    for (int k = 0; k < 4; ++k) res[0][k] = sum[k] + res[0][k];
  }
  store_dense<EPI>(res[0], alpha, lvalid, 0, row0, d.H, d.out);
#endif  // __HIP_DEVICE_COMPILE__
}

// K splits of the down projection: the fewest whose splits fit a down
// unit's weight registers (kDownSets tiles per wave, all loaded before the
// wait for h), every split non-empty.
int decode_splits(int64_t H, int64_t I) {
  (void)H;
  const int64_t T = I / kTileK;
  int64_t ks = (T + kSplitTiles - 1) / kSplitTiles;
  ks = ks < 1 ? 1 : (ks > kDecodeMaxSplits ? kDecodeMaxSplits : ks);
  while (ks > 1 && (ks - 1) * ((T + ks - 1) / ks) >= T) --ks;
  return (int)ks;
}

static bool split_ok(int64_t I, int ks) {
  if (ks < 1 || ks > kDecodeMaxSplits) return false;
  const int64_t T = I / kTileK, per = (T + ks - 1) / ks;
  return (ks - 1) * per < T && per <= kMaxSplitTiles;
}

bool decode_supported(int64_t H, int64_t I) {
  if (H % kTileK != 0 || I % kTileK != 0 || H <= 0 || I <= 0) return false;
  // 32-bit buffer offsets: both packed weights below 2^31 bytes.
  const int64_t lim = int64_t(1) << 31;
  if (2 * I * H / 16 * 9 >= lim) return false;
  if (!split_ok(I, decode_splits(H, I))) return false;
  // LDS: the quantized x (H columns) and the largest split of h.
  return fp4_lds_bytes(1, H) <= kFp4GemvLdsBytes && fp4_lds_bytes(1, I) <= kFp4GemvLdsBytes;
}

int64_t decode_record_words(int64_t H, int64_t I) { return 3 * (I / kTileRows) + H * kDecodeMaxSplits; }

hipError_t launch_decode_mlp(int epi, const DecodeArgs& d, hipStream_t s) {
  if (!decode_supported(d.H, d.I) || !split_ok(d.I, d.ksplit) || (uint32_t)d.epoch == 0u || !d.records ||
      !d.status || d.spin_limit < 1)
    return hipErrorInvalidValue;
  const int T = (int)(d.I / kTileK), per = (T + d.ksplit - 1) / d.ksplit;
  const int64_t grid = d.I / kTileRows + d.H / kTileRows * d.ksplit;
  const size_t lds = (size_t)std::max(fp4_lds_bytes(1, d.H), fp4_lds_bytes(1, (int64_t)per * kTileK));
  if (epi == kOutF32) {
    k_decode_mlp<kOutF32><<<dim3((unsigned)grid), kDecodeWaves * 64, lds, s>>>(d);
  } else if (epi == kOutBF16) {
    k_decode_mlp<kOutBF16><<<dim3((unsigned)grid), kDecodeWaves * 64, lds, s>>>(d);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nvfp4
