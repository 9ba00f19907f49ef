// decode16.hip -- the W4A16 MLP forward of one token in a single launch:
// gate_up GEMV + SiLU(gate) * up to a bf16 h, then the down projection GEMV
// on that h (the W4A16 dense path of the sglang PR #35120 report,
// implementation breakdown items 2 and 3, at one token), with no kernel
// boundary between the two GEMVs: the down projection's weight loads start
// while the gate_up GEMV still streams its own.
//
// The structure is the W4A4 single-launch decode's (decode.hip) with the
// VALU GEMV of gemv_tile.h (the two-launch W4A16 path's arithmetic, same
// wave count and order) in place of the FP4 one:
//   * gate_up units, workgroups [0, I / 16): unit i is the GEMV of gate rows
//     16 i.. and up rows 16 i.. over all of H with x (bf16) staged in LDS;
//     it forms h = bf16(SiLU(gate) * up) for its 16 elements, stores them to
//     the workspace's h (as the two-launch path leaves it) and as 8 tagged
//     records of two bf16 each (decode_records.h), and exits without waiting.
//   * down units, the next (H / 16) * S workgroups: unit (r, s) is the GEMV
//     of output rows 16 r.. over the K tiles of split s. It issues the loads
//     of its weight tiles first, then polls the records of its part of h
//     until each carries this launch's tag, writing them into its LDS image
//     as they arrive, and runs the GEMV. Units of splits below S - 1 store
//     their 16 partial sums as tagged records; the unit of split S - 1 polls
//     those, adds the S partials in split order and writes the output.
//
// Every wait is on workgroups of smaller index, or on gate_up units, which
// never wait: each XCD starts its workgroups in index order, so the awaited
// ones are running or done whatever the number of resident workgroups. Each
// wait is still bounded; one that gives up writes NaN for that unit's rows
// and sets kDecodeWaitExpired in the status word.
#include <algorithm>

#include "decode_records.h"
#include "gemv_tile.h"

namespace nvfp4 {

namespace {
constexpr int kD16Waves = 8;       // waves per workgroup, as the two-launch VALU GEMV at these grids
constexpr int kD16Sets = 2;        // weight tiles per wave a down unit holds before the wait for h
constexpr int kD16PollWords = 4;   // record words per thread a down unit can poll
constexpr int kD16SplitTiles = kD16Sets * kD16Waves;
// Down units cover at most this many K tiles (128 record words of h per tile).
constexpr int kD16MaxSplitTiles = kD16PollWords * kD16Waves * 64 / 128;
}  // namespace

template <int EPI>
__global__ __launch_bounds__(kD16Waves * 64) void k_decode_mlp16(Decode16Args d) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = kD16Waves;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = (int)threadIdx.x;
  const int q = lane >> 4;
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  __shared__ float red[NW][2][16];
  const int64_t nA = d.I / kTileRows;
  const bool lvalid = (lane & 15) == 0;  // lanes holding token 0
  const uint32_t tag = (uint32_t)d.epoch;  // the tag every wait looks for
  const uint32_t ptag = tag ^ d.tag_skew;  // the tag records are written with
  // Records: h as I / 2 words (word w: elements 2 w, 2 w + 1 as bf16 in the
  // low and high half), then the down units' partial sums (unit j, row k:
  // word j * 16 + k).
  uint64_t* rec_h = d.records;
  uint64_t* rec_part = d.records + d.I / 2;

  if ((int64_t)blockIdx.x < nA) {
    // ---- gate_up unit i: rows [16 i, 16 i + 16) of gate and of up ----
    const int64_t K = d.H;
    const int nt = (int)(K / kTileK);
    GemvSrc src;
    src.w = make_rsrc(d.w_gu, (uint32_t)(2 * nA * nt * kTileBytes));
    src.a = make_rsrc(d.x, (uint32_t)(K * 2));
    const float alpha = uniform_now(d.alpha_gu);
    const int64_t rg0 = 2 * (int64_t)blockIdx.x;
    float acc[2][1] = {{0.0f}, {0.0f}};
    int t = wave;
    GemvTile<2> ta;
    {
      // Staging of x in 16-byte chunks, the first four per thread requested
      // before the first weight tile (as in k_valu_gemv); a chunk past the
      // row goes to the 16 spare bytes after it, so no load stays pending.
      const int chunks = nt * 32;
      const uint32_t sink = (uint32_t)(K * 2);
      constexpr int kStride = NW * 64;
      u32x4 v[4];
      auto fetch = [&](int base) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = base + u * kStride;
          v[u] = bload16(src.a, i < chunks ? (uint32_t)(16 * i) : kOutOfRange);
        }
      };
      auto store = [&](int base) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = base + u * kStride;
          *reinterpret_cast<u32x4*>(xs + (i < chunks ? (uint32_t)(16 * i) : sink)) = v[u];
        }
      };
      fetch(tid);
      gemv_load<2>(ta, src, rg0, nt, nt, t, lane);
      store(tid);
      for (int base = tid + 4 * kStride; base < chunks; base += 4 * kStride) {
        fetch(base);
        store(base);
      }
    }
    __syncthreads();
    while (t < nt) {
      gemv_compute<2, 1>(acc, ta, xs, nt, t, lane);
      __builtin_amdgcn_sched_barrier(0);
      t += NW;
      gemv_load<2>(ta, src, rg0, nt, nt, t, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Sum the four lanes of each row, then the waves in order (as k_valu_gemv).
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      acc[g][0] += __shfl_xor(acc[g][0], 16);
      acc[g][0] += __shfl_xor(acc[g][0], 32);
    }
    if (q == 0) {
      red[wave][0][lane] = acc[0][0];
      red[wave][1][lane] = acc[1][0];
    }
    __syncthreads();
    if (wave > 0) return;
    float h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float sg = 0.0f, su = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        sg += red[w][0][4 * q + r];
        su += red[w][1][4 * q + r];
      }
      h[r] = silu_mul(alpha * sg, alpha * su);
    }
    if (lvalid) {
      // Elements 16 i + 4 q + r, r = 0..3: two words of bf16 pairs.
      const uint32_t b0 = __builtin_bit_cast(uint16_t, (__bf16)h[0]), b1 = __builtin_bit_cast(uint16_t, (__bf16)h[1]);
      const uint32_t b2 = __builtin_bit_cast(uint16_t, (__bf16)h[2]), b3 = __builtin_bit_cast(uint16_t, (__bf16)h[3]);
      const uint32_t w0 = b0 | (b1 << 16), w1 = b2 | (b3 << 16);
      const int64_t e0 = 16 * (int64_t)blockIdx.x + 4 * q;
      put_record(rec_h + e0 / 2, w0, ptag);
      put_record(rec_h + e0 / 2 + 1, w1, ptag);
      uint2 hv;
      hv.x = w0;
      hv.y = w1;
      *reinterpret_cast<uint2*>(d.h + e0) = hv;
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

  const float alpha = uniform_now(d.alpha_d);
  GemvSrc src;
  src.w = make_rsrc(d.w_d, (uint32_t)(RG * T * kTileBytes));
  src.a = src.w;
  GemvTile<1> tw[kD16Sets];
#pragma unroll
  for (int u = 0; u < kD16Sets; ++u) gemv_load<1>(tw[u], src, r, T, t1, t0 + wave + u * NW, lane);

  // h of tiles [t0, t1): 128 nts words, word tid + 512 k of them polled by
  // this thread until its tag is current, its two bf16 written to the image
  // (the split's part of h as one bf16 row of nts tiles).
  bool timed_out = false;
  {
    const int nw = 128 * nts;
    const uint64_t* hw = rec_h + 128 * (int64_t)t0;
    uint32_t pending = 0;
#pragma unroll
    for (int k = 0; k < kD16PollWords; ++k)
      if (tid + NW * 64 * k < nw) pending |= 1u << k;
    for (int spin = 0;; ++spin) {
#pragma unroll
      for (int k = 0; k < kD16PollWords; ++k) {
        const int w = tid + NW * 64 * k;
        if (pending & (1u << k)) {
          const uint64_t v = get_record(hw + w);
          if ((uint32_t)(v >> 32) == tag) {
            pending &= ~(1u << k);
            *reinterpret_cast<uint32_t*>(xs + 4 * w) = (uint32_t)v;
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

  // kD16Sets register sets per wave, one tile each, refilled kD16Sets * NW
  // tiles ahead (tiles past the split load zeros and are not computed).
  float acc[1][1] = {{0.0f}};
  for (int base = 0; base < nts; base += kD16Sets * NW) {
#pragma unroll
    for (int u = 0; u < kD16Sets; ++u) {
      const int tl = base + wave + u * NW;  // tile index within the split
      if (tl < nts) gemv_compute<1, 1>(acc, tw[u], xs, nts, tl, lane);
      __builtin_amdgcn_sched_barrier(0);
      gemv_load<1>(tw[u], src, r, T, t1, t0 + tl + kD16Sets * NW, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  acc[0][0] += __shfl_xor(acc[0][0], 16);
  acc[0][0] += __shfl_xor(acc[0][0], 32);
  if (q == 0) red[wave][0][lane] = acc[0][0];
  __syncthreads();
  if (wave > 0) return;
  f32x4 res;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += red[w][0][4 * q + k];
    res[k] = lvalid ? sum : 0.0f;
  }
  // timed_out is uniform (every thread took the same exit of the poll).
  if (timed_out) {
    res = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    if (lane == 0) report_expired(d.status);
  }
  const int64_t row0 = r * kTileRows + 4 * q;
  if (s < d.ksplit - 1) {
    if (lvalid) {
#pragma unroll
      for (int k = 0; k < 4; ++k) put_record(rec_part + j * 16 + 4 * q + k, __float_as_uint(res[k]), ptag);
    }
    return;
  }
  if (d.ksplit > 1) {
    // The last split adds the S partials of rows 16 r.. in split order.
    const f32x4 sum = sum_split_partials(rec_part, RG, r, d.ksplit, tag, d.spin_limit, d.status, lane);
#pragma unroll
    for (int k = 0; k < 4; ++k) res[k] = sum[k] + res[k];
  }
  store_dense<EPI>(res, alpha, lvalid, 0, row0, d.H, d.out);
#endif  // __HIP_DEVICE_COMPILE__
}

// K splits of the down projection: the fewest whose splits fit a down unit's
// weight registers (kD16Sets tiles per wave, all loaded before the wait for
// h), every split non-empty.
int decode16_splits(int64_t H, int64_t I) {
  (void)H;
  const int64_t T = I / kTileK;
  int64_t ks = (T + kD16SplitTiles - 1) / kD16SplitTiles;
  ks = ks < 1 ? 1 : (ks > kDecodeMaxSplits ? kDecodeMaxSplits : ks);
  while (ks > 1 && (ks - 1) * ((T + ks - 1) / ks) >= T) --ks;
  return (int)ks;
}

static bool split16_ok(int64_t I, int ks) {
  if (ks < 1 || ks > kDecodeMaxSplits) return false;
  const int64_t T = I / kTileK, per = (T + ks - 1) / ks;
  return (ks - 1) * per < T && per <= kD16MaxSplitTiles;
}

bool decode16_supported(int64_t H, int64_t I) {
  if (H % kTileK != 0 || I % kTileK != 0 || H <= 0 || I <= 0) return false;
  // 32-bit buffer offsets: both packed weights below 2^31 bytes.
  const int64_t lim = int64_t(1) << 31;
  if (2 * I * H / 16 * 9 >= lim) return false;
  const int ks = decode16_splits(H, I);
  if (!split16_ok(I, ks)) return false;
  // LDS: x (H bf16 and 16 spare bytes) and the largest split of h.
  const int64_t per = (I / kTileK + ks - 1) / ks;
  return H * 2 + 16 <= kValuGemvLdsBytes && per * kTileK * 2 <= kValuGemvLdsBytes;
}

int64_t decode16_record_words(int64_t H, int64_t I) { return I / 2 + H * kDecodeMaxSplits; }

hipError_t launch_decode_mlp16(int epi, const Decode16Args& d, hipStream_t s) {
  if (!decode16_supported(d.H, d.I) || !split16_ok(d.I, d.ksplit) || (uint32_t)d.epoch == 0u || !d.records ||
      !d.status || d.spin_limit < 1)
    return hipErrorInvalidValue;
  const int T = (int)(d.I / kTileK), per = (T + d.ksplit - 1) / d.ksplit;
  const int64_t grid = d.I / kTileRows + d.H / kTileRows * d.ksplit;
  const size_t lds = (size_t)std::max<int64_t>(d.H * 2 + 16, (int64_t)per * kTileK * 2);
  if (epi == kOutF32) {
    k_decode_mlp16<kOutF32><<<dim3((unsigned)grid), kD16Waves * 64, lds, s>>>(d);
  } else if (epi == kOutBF16) {
    k_decode_mlp16<kOutBF16><<<dim3((unsigned)grid), kD16Waves * 64, lds, s>>>(d);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nvfp4
