// fp4_tile.h -- building blocks of the W4A4 decode GEMV on the FP4 matrix
// core, with the per-16 E4M3 scales applied exactly (used by fp4gemv.hip and
// by the single-launch decode MLP in decode.hip).
//
// The 16x16x128 FP4 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4 with both E8M0
// scales at 2^0) takes E2M1 codes straight from memory: lane l supplies 32
// codes of A row l % 16 and 32 codes of B column l % 16, at the same 32 K
// positions for both operands, and the products of grid values and their
// sums are exact. It cannot apply the NVFP4 block scales itself (those are
// E4M3 per 16 elements, its own are powers of two per 32), so the blocks are
// kept apart instead of scaled inside the instruction:
//
//   * B is the packed weight tile as it is loaded: lane l holds row
//     n = l % 16 and, in half tile c, columns 128 c + 32 q + [0, 32) with
//     q = l / 16, i.e. the two 16-element blocks 8 c + 2 q + b, b = 0, 1.
//   * A is the token's activation codes with one block per output row:
//     row rho = 4 q' + 2 c' + b' holds block 8 c' + 2 q' + b' (and zeros
//     elsewhere). In the half-c instruction, lane (rho, q) carries that block
//     at the nibbles where the weight lane (n, q) keeps the same block, when
//     q == q' and c == c', and zeros otherwise.
//
// Two instructions (c = 0, 1) fill all 16 rows, so C[rho][n] is the exact,
// unscaled dot product of weight row n and the activation over block
// 8 c' + 2 q' + b'. Lane l of the 16x16 result holds rows 4 q + r, r = 0..3,
// of column n = l % 16: exactly the blocks whose weight scales the same lane
// loaded (byte r of its scale dword is block c = r / 2, b = r % 2) and whose
// activation scales it loads. Each block sum is then scaled once by
// s_w * s_a (a product of two E4M3 values, exact in fp32) and accumulated
// in fp32, the same arithmetic per block as the VALU formulation.
#pragma once
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

#if defined(__HIP_DEVICE_COMPILE__)

typedef int i32x8 __attribute__((ext_vector_type(8)));

// C + A * B over 128 E2M1 codes per row and column (unit E8M0 scales).
__device__ __forceinline__ f32x4 mfma_fp4(const u32x4& a, const u32x4& b, const f32x4& c) {
  const i32x8 a8 = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8 b8 = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 4, 0, 127, 0, 127);
}

// LDS image of a workgroup's activations over K columns: the MT token rows
// of codes, then K / 2 zero bytes (read by the slots a lane does not carry),
// then the MT rows of scales.
__device__ __forceinline__ int lds_zero_off(int MT, int K) { return MT * K / 2; }
__device__ __forceinline__ int lds_scale_off(int MT, int K) { return MT * K / 2 + K / 2; }

template <int MT>
struct F4Src {
  Rsrc w;
  // LDS offset, in tile 0, of this lane's activation block for token m,
  // half c and block parity b; the zero region where the lane carries no
  // block in that slot.
  uint32_t slot[MT][2][2];
  uint32_t s_row[MT];  // LDS offset of the token's scales + 2 q
};

// A-operand slots of this lane for an image of K columns: row rho = lane % 16
// carries block 8 c' + 2 q' + b' with q' = rho / 4, c' = (rho / 2) % 2,
// b' = rho % 2, in the lanes of K chunk q == q' of the half-c' instruction.
template <int MT>
__device__ __forceinline__ void f4_slots(F4Src<MT>& src, int lane, int K) {
  const int q = lane >> 4, rho = lane & 15;
  const int cp = (rho >> 1) & 1, bp = rho & 1;
  const bool carrier = q == (rho >> 2);
  const uint32_t blk_off = (uint32_t)(8 * (8 * cp + 2 * q + bp));
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        src.slot[m][c][b] = (carrier && c == cp && b == bp) ? (uint32_t)(m * K / 2) + blk_off
                                                            : (uint32_t)lds_zero_off(MT, K);
    src.s_row[m] = (uint32_t)(lds_scale_off(MT, K) + m * K / 16 + 2 * q);
  }
}

template <int NG, int MT>
struct F4Tile {
  u32x4 wc[NG][2];
  uint32_t wsd[NG];
  u32x2 xa[MT][2][2];
  uint32_t xsd[MT][2];  // activation scales of blocks 2 q + {0, 1} and 8 + 2 q + {0, 1}
};

// Weight loads of tile t of row groups of T tiles (out of range from tile
// t_end on: zeros, no memory access).
template <int NG, int MT>
__device__ __forceinline__ void f4_load_w(F4Tile<NG, MT>& d, const F4Src<MT>& src, int64_t rg0, int T,
                                          int t_end, int t, int lane) {
  const uint32_t tw = t < t_end ? (uint32_t)(t * kTileBytes) : kOutOfRange;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint32_t gbase = (uint32_t)((rg0 + g) * T * kTileBytes);
    d.wc[g][0] = bload16_nt(src.w, tw + 16 * lane, gbase);
    d.wc[g][1] = bload16_nt(src.w, tw + 1024 + 16 * lane, gbase);
    d.wsd[g] = bload4_nt(src.w, tw + kTileCodeBytes + 4 * lane, gbase);
  }
}

// The activation slots of image tile t from LDS (from tile t_end - 1 when t
// is past the image: valid addresses, values multiplied by zero weights).
template <int NG, int MT>
__device__ __forceinline__ void f4_load_x(F4Tile<NG, MT>& d, const F4Src<MT>& src, const uint8_t* xl,
                                          int t_end, int t) {
  const uint32_t tc = (uint32_t)((t < t_end ? t : t_end - 1));
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        d.xa[m][c][b] = *reinterpret_cast<const u32x2*>(xl + src.slot[m][c][b] + tc * 128);
    const uint8_t* sp = xl + src.s_row[m] + tc * 16;
    d.xsd[m][0] = *reinterpret_cast<const uint16_t*>(sp);
    d.xsd[m][1] = *reinterpret_cast<const uint16_t*>(sp + 8);
  }
}

// The half-c instruction fills only rows 4 q + 2 c + {0, 1} of each lane
// (r = 2 c + b), so the two halves accumulate into separate results and
// each row takes its value from the one that wrote it.
template <int NG, int MT>
__device__ __forceinline__ void f4_compute(f32x4 (&acc)[NG][MT], const F4Tile<NG, MT>& d) {
  float xs[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    xs[m][0] = e4m3_to_f32<0>(d.xsd[m][0]); xs[m][1] = e4m3_to_f32<1>(d.xsd[m][0]);
    xs[m][2] = e4m3_to_f32<0>(d.xsd[m][1]); xs[m][3] = e4m3_to_f32<1>(d.xsd[m][1]);
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float ws[4];
    ws[0] = e4m3_to_f32<0>(d.wsd[g]); ws[1] = e4m3_to_f32<1>(d.wsd[g]);
    ws[2] = e4m3_to_f32<2>(d.wsd[g]); ws[3] = e4m3_to_f32<3>(d.wsd[g]);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const u32x4 a0 = {d.xa[m][0][0][0], d.xa[m][0][0][1], d.xa[m][0][1][0], d.xa[m][0][1][1]};
      const u32x4 a1 = {d.xa[m][1][0][0], d.xa[m][1][0][1], d.xa[m][1][1][0], d.xa[m][1][1][1]};
      const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
      const f32x4 c0 = mfma_fp4(a0, d.wc[g][0], zero);
      const f32x4 c1 = mfma_fp4(a1, d.wc[g][1], zero);
      acc[g][m][0] = __builtin_fmaf(c0[0], ws[0] * xs[m][0], acc[g][m][0]);
      acc[g][m][1] = __builtin_fmaf(c0[1], ws[1] * xs[m][1], acc[g][m][1]);
      acc[g][m][2] = __builtin_fmaf(c1[2], ws[2] * xs[m][2], acc[g][m][2]);
      acc[g][m][3] = __builtin_fmaf(c1[3], ws[3] * xs[m][3], acc[g][m][3]);
    }
  }
}

// The GEMV of one workgroup over all K tiles: NG row groups from rg0 (gate
// and up for SwiGLU), MT token rows from tok0, NW waves dividing the tiles.
// Stages the token rows in LDS at xl (QX: bf16 rows quantized to NVFP4 on the
// way in with args.a_g_inv, the same arithmetic as launch_quantize) and
// leaves each lane's per-block sums in acc (zero-initialised here).
template <int NG, int MT, int NW, bool QX>
__device__ __forceinline__ void f4_gemv_acc(const GemmArgs& args, int64_t rg0, int64_t tok0, uint8_t* xl,
                                            int lane, int wave, f32x4 (&acc)[NG][MT]) {
  const int64_t K = args.K, T = K / kTileK;
  const int Ki = (int)K;
  F4Src<MT> src;
  src.w = make_rsrc(args.w, (uint32_t)(args.N / kTileRows * T * kTileBytes));
  f4_slots<MT>(src, lane, Ki);
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[g][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // K tiles [t0, t1): all of them (the staging and loop are written for a
  // tile range).
  const int nt = (int)T;
  const int t0 = 0, t1 = nt, tlast = nt;
  int t = t0 + wave;
  F4Tile<NG, MT> ta, tb;
  {
    // Staging of tiles [t0, t1) of the MT token rows, codes and scales, in
    // 16-byte chunks (rows past M are past the end of the buffers and read
    // as zeros). The first four chunks per thread are requested before the
    // first two weight tiles, so that writing them to LDS waits for these
    // loads only (the vector memory counter is in order), not for the
    // weights.
    const Rsrc ra = make_rsrc(args.a, (uint32_t)(args.M * (K / 2)));
    const Rsrc rs = make_rsrc(args.a_scales, (uint32_t)(args.M * (K / 16)));
    const int nts = t1 > t0 ? t1 - t0 : 0;
    const int code_row = nts * 8, code_chunks = MT * code_row, chunks = code_chunks + MT * nts;
    constexpr int kStride = NW * 64;
    const int tid = (int)threadIdx.x;
    u32x4 v[4];
    // Byte offsets in the buffers (code or scale) and in LDS of chunk i.
    auto offsets = [&](int i, uint32_t& g, uint32_t& l) {
      if (i < code_chunks) {
        const int m = i / code_row, j = i - m * code_row;
        g = (uint32_t)((tok0 + m) * (K / 2)) + (uint32_t)(t0 * 128 + 16 * j);
        l = (uint32_t)(m * Ki / 2 + t0 * 128 + 16 * j);
      } else {
        const int i2 = i - code_chunks, m = i2 / (nts > 0 ? nts : 1), j = i2 - m * nts;
        g = (uint32_t)((tok0 + m) * (K / 16)) + (uint32_t)((t0 + j) * 16);
        l = (uint32_t)(lds_scale_off(MT, Ki) + m * Ki / 16 + (t0 + j) * 16);
      }
    };
    auto fetch = [&](int base) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + u * kStride;
        uint32_t g = kOutOfRange, l = 0;
        if (i < chunks) offsets(i, g, l);
        v[u] = bload16(i < code_chunks ? ra : rs, g);
      }
    };
    // Every fetched value is written (a chunk past the end loaded zeros and
    // goes to the zero region), so no load is left pending with its
    // register free for reuse: reusing one would wait for all later loads.
    auto store = [&](int base) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + u * kStride;
        uint32_t g, l = (uint32_t)(lds_zero_off(MT, Ki) + t0 * 128);
        if (i < chunks) offsets(i, g, l);
        *reinterpret_cast<u32x4*>(xl + l) = v[u];
      }
    };
    if constexpr (QX) {
      // bf16 token rows quantized on the way in: chunk i holds 8 elements,
      // chunks 2b and 2b + 1 of a row (neighbouring lanes) form block b and
      // exchange their amax, exactly as in the standalone quantizer.
      const Rsrc rx = make_rsrc(args.a, (uint32_t)(args.M * K * 2));
      const float gi = *args.a_g_inv;
      const int row8 = nts * 32, xchunks = MT * row8;
      auto xfetch = [&](int base) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = base + u * kStride;
          const int m = i / row8, j = i - m * row8;
          v[u] = bload16(rx, i < xchunks ? (uint32_t)((tok0 + m) * K * 2) + (uint32_t)(t0 * 512 + 16 * j)
                                         : kOutOfRange);
        }
      };
      auto xstore = [&](int base) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = base + u * kStride;
          float e[8];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            e[2 * k] = __uint_as_float(v[u][k] << 16);
            e[2 * k + 1] = __uint_as_float(v[u][k] & 0xFFFF0000u);
          }
          uint32_t mx = 0;
#pragma unroll
          for (int k = 0; k < 8; ++k) mx = max(mx, __float_as_uint(e[k]) & 0x7FFFFFFFu);
          mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1));
          const BlockScale bs = block_scale(__uint_as_float(mx), gi);
          float y[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) y[k] = e[k] * bs.r;
          const uint32_t packed = e2m1_pack8(y);
          if (i < xchunks) {
            const int m = i / row8, j = i - m * row8;
            *reinterpret_cast<uint32_t*>(xl + m * Ki / 2 + t0 * 128 + 4 * j) = packed;
            if ((j & 1) == 0) xl[lds_scale_off(MT, Ki) + m * Ki / 16 + t0 * 16 + j / 2] = (uint8_t)bs.byte;
          }
        }
      };
      xfetch(tid);
      f4_load_w<NG, MT>(ta, src, rg0, nt, t1, t, lane);
      f4_load_w<NG, MT>(tb, src, rg0, nt, t1, t + NW, lane);
      xstore(tid);
      for (int base = tid + 4 * kStride; base < xchunks; base += 4 * kStride) {
        xfetch(base);
        xstore(base);
      }
    } else {
      fetch(tid);
      f4_load_w<NG, MT>(ta, src, rg0, nt, t1, t, lane);
      f4_load_w<NG, MT>(tb, src, rg0, nt, t1, t + NW, lane);
      store(tid);
      for (int base = tid + 4 * kStride; base < chunks; base += 4 * kStride) {
        fetch(base);
        store(base);
      }
    }
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < nts * 8; i += kStride)
      *reinterpret_cast<u32x4*>(xl + lds_zero_off(MT, Ki) + t0 * 128 + 16 * i) = z;
  }
  __syncthreads();
  f4_load_x<NG, MT>(ta, src, xl, tlast, t);
  f4_load_x<NG, MT>(tb, src, xl, tlast, t + NW);

  // Two register sets, two tiles per trip and no exit between them: a tile
  // past the range has all-zero weight codes and scales (out-of-range
  // loads), so its products add +0. (An exit between the halves lets the
  // compiler sink the second half's prefetch into it.) The scheduling
  // barriers keep each prefetch clear of the arithmetic before it: an
  // instruction on prefetched data pulled forward would wait for every
  // load in flight.
  while (t < t1) {
    f4_compute<NG, MT>(acc, ta);
    __builtin_amdgcn_sched_barrier(0);
    f4_load_w<NG, MT>(ta, src, rg0, nt, t1, t + 2 * NW, lane);
    f4_load_x<NG, MT>(ta, src, xl, tlast, t + 2 * NW);
    __builtin_amdgcn_sched_barrier(0);
    f4_compute<NG, MT>(acc, tb);
    __builtin_amdgcn_sched_barrier(0);
    f4_load_w<NG, MT>(tb, src, rg0, nt, t1, t + 3 * NW, lane);
    f4_load_x<NG, MT>(tb, src, xl, tlast, t + 3 * NW);
    __builtin_amdgcn_sched_barrier(0);
    t += 2 * NW;
  }
}

// Sum of a lane's per-block results (r), of the four K chunks (xor 16, then
// 32) and of the NW waves through red (NW * NG * MT * 16 floats of LDS).
// Wave 0 receives the result in the MFMA layout of the other GEMM kernels
// (lane l: token l % 16, rows 4 (l / 16) + r; zeros where !lvalid) and
// returns true; the other waves return false and have nothing left to do.
template <int NG, int MT, int NW>
__device__ __forceinline__ bool f4_reduce(const f32x4 (&acc)[NG][MT], float* red, int wave, int lane,
                                          bool lvalid, f32x4 (&res)[NG]) {
  const int q = lane >> 4;
  float v[NG][MT];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      v[g][m] = (acc[g][m][0] + acc[g][m][1]) + (acc[g][m][2] + acc[g][m][3]);
      v[g][m] += __shfl_xor(v[g][m], 16);
      v[g][m] += __shfl_xor(v[g][m], 32);
    }
  if (q == 0) {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int m = 0; m < MT; ++m) red[((wave * NG + g) * MT + m) * 16 + lane] = v[g][m];
  }
  __syncthreads();
  if (wave > 0) return false;
  const int tl = lane & 15;
  const int tm = tl < MT ? tl : 0;
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red[((w * NG + g) * MT + tm) * 16 + 4 * q + r];
      res[g][r] = lvalid ? s : 0.0f;
    }
  return true;
}

#endif  // __HIP_DEVICE_COMPILE__

// Bytes of the LDS activation image of MT token rows over K columns.
inline int64_t fp4_lds_bytes(int64_t MT, int64_t K) { return MT * K / 2 + K / 2 + MT * K / 16; }

}  // namespace nvfp4
