// device_common.h -- gfx950 device helpers shared by the NVFP4 kernels:
// the E2M1/E4M3 encoders, in-register dequantization for the MFMA operands,
// the packed-weight tile geometry and the GEMM epilogues.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace nvfp4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Packed weight tile: 16 rows x 256 columns. Lane l of a wave owns, for
// c = 0, 1, the 16 code bytes at c * 1024 + 16 l (row l % 16, columns
// 256 t + 128 c + 32 (l / 16) + [0, 32)) and 4 scale bytes at 2048 + 4 l
// (blocks 16 t + 8 c + 2 (l / 16) + {0, 1}, ordered c0b0 c0b1 c1b0 c1b1).
constexpr int kTileRows = 16;
constexpr int kTileK = 256;
constexpr int kTileCodeBytes = 2048;
constexpr int kTileBytes = 2304;

template <int E>
struct EpiTraits {
  static constexpr bool swiglu = (E == kSwigluNvfp4 || E == kSwigluBF16 || E == kSwigluF32);
};

// ---------------------------------------------------------------------------
// Encoders (round to nearest, ties to even, saturating).
// ---------------------------------------------------------------------------

// Non-negative finite fp32 -> E4M3FN byte. Normal range: round the 23-bit
// mantissa to 3 bits with the carry running into the exponent; below 2^-6 the
// quantum is 2^-9, so rint(v * 512) is the subnormal mantissa (8 = 2^-6 is
// byte 0x08 as well). Values at or above 448 saturate to 0x7E.
// Both roundings are computed and the right one selected (no branch: the
// lanes of a wave hold different blocks).
__device__ __forceinline__ uint32_t e4m3_from_f32(float v) {
  const uint32_t u = __float_as_uint(v) & 0x7FFFFFFFu;
  const uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(u) * 512.0f);  // < 2^-6
  const uint32_t un = u + 0x7FFFFu + ((u >> 20) & 1u);
  const uint32_t nrm = (((un >> 23) - 120u) << 3) | ((un >> 20) & 7u);
  return u >= 0x43E00000u ? 0x7Eu : (u < 0x3C800000u ? sub : nrm);  // >= 448 saturates
}

// E4M3FN byte (selected byte of a dword) -> fp32, hardware OCP decode.
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t dword) {
  return __builtin_amdgcn_cvt_f32_fp8((int)dword, SEL);
}

// fp32 -> 4-bit E2M1 code. The code magnitude counts the grid midpoints that
// |y| has passed; the comparison at each midpoint (strict or not) sends ties
// to the even neighbour. Bit 3 takes the sign bit of y.
__device__ __forceinline__ uint32_t e2m1_from_f32(float y) {
  float a = __builtin_fabsf(y);
  uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
               (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
               (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(y) >> 28) & 8u);
}

// Pairs of fp32 values to E2M1 codes with the hardware conversion (unit
// scale): round to nearest even, saturating at 6, sign kept, exactly the
// rules of e2m1_from_f32 (checked on the GPU against it on every tie, the
// neighbours of every tie and grid point, a dense sweep of [-8, 8], zeros,
// subnormals and values far past 6). The first of a pair goes to the low
// nibble; pair k fills byte k.
__device__ __forceinline__ uint32_t e2m1_pack8(const float (&y)[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}
__device__ __forceinline__ uint32_t e2m1_pack4(float y0, float y1, float y2, float y3) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y0, y1, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y2, y3, 1.0f, 1);
  return w;
}

// One NVFP4 block: scale byte and the per-element multiplier r = g_inv / s.
struct BlockScale {
  uint32_t byte;
  float r;
};
// x / 6 as RN(x * y) corrected by one fused multiply-add of its remainder,
// y = RN(1/6): the correctly rounded quotient for every fp32 x >= 2^-125
// (checked over every such input); below that both are under 2^-120 and
// encode to the E4M3 byte 0, so the scale byte is the one x / 6 gives.
__device__ __forceinline__ float div6(float x) {
  const float y = 0x1.555556p-3f;
  const float q0 = x * y;
  return __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, x), y, q0);
}

__device__ __forceinline__ BlockScale block_scale(float amax, float g_inv) {
  float sv = div6(amax * g_inv);
  BlockScale b;
  b.byte = e4m3_from_f32(sv);
  float s = __builtin_amdgcn_cvt_f32_fp8((int)b.byte, 0);
  b.r = (s != 0.0f) ? g_inv / s : 0.0f;
  return b;
}

// ---------------------------------------------------------------------------
// Dequantization of 8 E2M1 codes (one dword) into an MFMA operand.
// The fp4 conversion instructions scale by a power of two only (the exponent
// of their f32 scale operand), so the E4M3 block scale is applied separately:
//  * f16: q converts exactly, then a packed f16 multiply by s; q * s has at
//    most 6 significant bits and lies in [2^-10, 2688], so it is exact.
//  * bf16: q * s through f32 (exact) and a round-to-nearest pack that keeps
//    the exact value.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f16x8 deq8_f16(uint32_t w, _Float16 s) {
  f16x2 s2 = {s, s};
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  f16x8 r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

__device__ __forceinline__ bf16x8 deq8_bf16(uint32_t w, float s) {
  f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  bf16x8 r = {(__bf16)(p0[0] * s), (__bf16)(p0[1] * s), (__bf16)(p1[0] * s),
              (__bf16)(p1[1] * s), (__bf16)(p2[0] * s), (__bf16)(p2[1] * s),
              (__bf16)(p3[0] * s), (__bf16)(p3[1] * s)};
  return r;
}

// Scale byte k (0..3) of a lane's scale dword as f16 / f32.
template <int K>
__device__ __forceinline__ _Float16 scale_f16(uint32_t sdw) {
  return (_Float16)e4m3_to_f32<K>(sdw);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------------------
// Raw buffer loads (device pass only: the resource type is a GPU type). The
// per-lane offset is range-checked against the resource's byte count and an
// out-of-range load returns zeros without touching memory, so ragged token
// rows and the "no next tile" case of a software pipeline need no branch.
// ---------------------------------------------------------------------------
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOutOfRange = 0x80000000u;  // a lane offset past any buffer used here

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// `nt`: streamed once (the packed weights), with a wave-uniform scalar base
// `soff`; plain: re-read data, keep cached.
__device__ __forceinline__ u32x4 bload16_nt(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2);
}
__device__ __forceinline__ uint32_t bload4_nt(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 2);
}
__device__ __forceinline__ u32x4 bload16(Rsrc r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}
// Device-scope (sc1) load: sees stores of other workgroups made with
// device-scope stores, whichever XCD they ran on.
__device__ __forceinline__ u32x4 bload16_dev(Rsrc r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 16);
}
// Device-scope (sc1) 16-byte store: completed (vmcnt), visible to
// device-scope loads of other workgroups on any XCD.
__device__ __forceinline__ void bstore16_dev(Rsrc r, uint32_t voff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, 0, 16);
}
__device__ __forceinline__ uint32_t bload2(Rsrc r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, 0, 0);
}
#endif

// ---------------------------------------------------------------------------
// Split-K combine, run by the one wave that holds a workgroup's result tile
// (NT token groups, one f32x4 per lane each). Everything the workgroups of a
// tile exchange goes through device-scope (sc1) atomic loads and stores,
// which are coherent across the XCDs' separate L2 caches without the
// whole-L2 write-back and invalidate of a device-scope fence (that costs
// microseconds per workgroup here). The partial is stored, the wave waits
// until those stores have completed (vmcnt(0)), then counts its arrival;
// the workgroup that arrives last (of ks) reads the ks partials, adds them
// in split order (so the result does not depend on which workgroup
// finished last), resets the count for the next launch and returns true.
// The others return false and have nothing left to do. Only vector-memory
// instructions are used.
// ---------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ bool splitk_last(f32x4 (&res)[NT], float* part, uint32_t* counters, int ks,
                                            int64_t unit, int s, int lane) {
  float* mine = part + ((unit * ks + s) * NT) * 256;
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      __hip_atomic_store(mine + (j * 64 + lane) * 4 + r, res[j][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): the partial has reached device scope
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  uint32_t arrived = 0;
  if (lane == 0) arrived = __hip_atomic_fetch_add(counters + unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  arrived = __shfl(arrived, 0);
  if (arrived != (uint32_t)(ks - 1)) return false;
#pragma unroll
  for (int j = 0; j < NT; ++j) res[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int sp = 0; sp < ks; ++sp) {
    const float* p = part + ((unit * ks + sp) * NT) * 256;
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        res[j][r] += __hip_atomic_load(p + (j * 64 + lane) * 4 + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (lane == 0) __hip_atomic_store(counters + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// K-split combine of a workgroup's output tile (NT threads, acc[A][B] per
// thread). Each thread stores its partial of split `split` of tile `unit`
// (device scope), every wave waits for its stores to complete, then one
// thread counts the workgroup's arrival. The workgroup that arrives last (of
// ks) adds the ks partials in split order (the result does not depend on
// arrival order), resets the count and returns true; the others return
// false. part holds ks * A * B * 4 * NT floats per tile.
#if defined(__HIP_DEVICE_COMPILE__)
template <int A, int B, int NT>
__device__ __forceinline__ bool wg_splitk_last(f32x4 (&acc)[A][B], float* part, uint32_t* counters, int ks,
                                               int64_t unit, int split, int tid, uint32_t* arrived_lds) {
  constexpr int kTileFloats = A * B * 4 * NT;
  const Rsrc rp = make_rsrc(part + unit * ks * kTileFloats, (uint32_t)(ks * kTileFloats * 4));
#pragma unroll
  for (int g = 0; g < A; ++g)
#pragma unroll
    for (int j = 0; j < B; ++j)
      bstore16_dev(rp, (uint32_t)(((split * A * B + B * g + j) * NT + tid) * 16), __builtin_bit_cast(u32x4, acc[g][j]));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): this wave's partial is at device scope
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (tid == 0)
    *arrived_lds = __hip_atomic_fetch_add(counters + unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (*arrived_lds != (uint32_t)(ks - 1)) return false;
#pragma unroll
  for (int g = 0; g < A; ++g)
#pragma unroll
    for (int j = 0; j < B; ++j) acc[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < ks; ++sp) {
#pragma unroll
    for (int g = 0; g < A; ++g)
#pragma unroll
      for (int j = 0; j < B; ++j)
        acc[g][j] += __builtin_bit_cast(f32x4, bload16_dev(rp, (uint32_t)(((sp * A * B + B * g + j) * NT + tid) * 16)));
  }
  if (tid == 0) __hip_atomic_store(counters + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}
#endif  // __HIP_DEVICE_COMPILE__

// A kernel-uniform scalar read at this point of the program: the scalar load
// is issued here and kept in a register, not sunk to its use (an epilogue
// reading it after the main loop would wait there for a memory round trip).
__device__ __forceinline__ float uniform_now(const float* p) {
  int v = __builtin_amdgcn_readfirstlane(__float_as_int(*p));
  asm volatile("" : "+s"(v));
  return __int_as_float(v);
}

// A grouped GEMM launched once for all experts (GemmArgs.experts > 1):
// the operands of expert e.
__device__ __forceinline__ void expert_slice(GemmArgs& a, int64_t e) {
  a.a = static_cast<const uint8_t*>(a.a) + e * a.e_a;
  if (a.a_scales != nullptr) a.a_scales += e * a.e_as;
  a.w += e * a.e_w;
  a.out = static_cast<uint8_t*>(a.out) + e * a.e_out;
  a.alpha += e;
  if (a.m_dev != nullptr) a.m_dev += e;
}

// Valid token rows of a GEMM (the device-side masked row count of a grouped
// GEMM, else M).
__device__ __forceinline__ int64_t valid_rows(const GemmArgs& a) {
  if (a.m_dev == nullptr) return a.M;
  const int64_t r = (int64_t)__builtin_amdgcn_readfirstlane(*a.m_dev);
  return r < 0 ? 0 : (r > a.M ? a.M : r);
}

// Output tile `tile` of a grid of outer_n x inner_n tiles in bands of
// `band` outer tiles: within a band the tiles run inner-major with the
// band's outer tiles fastest (the last band may be narrower), a bijection
// onto [0, outer_n) x [0, inner_n). A run of consecutive tiles (one XCD's
// resident workgroups) then spans about band outer tiles by run / band inner
// tiles, so it reads that many operand panels of each kind instead of one
// of the first kind and a whole operand of the second.
__device__ __forceinline__ void banded_tile(int64_t tile, int64_t outer_n, int64_t inner_n, int64_t band,
                                            int64_t& outer, int64_t& inner) {
  const int64_t span = band * inner_n;
  const int64_t b = tile / span, within = tile - b * span;
  const int64_t rest = outer_n - b * band;
  const int64_t bw = rest < band ? rest : band;
  outer = b * band + within % bw;
  inner = within / bw;
}

// Workgroup (0, 0, 0) clears n words at p (the next GEMM's split-K counters).
__device__ __forceinline__ void clear_words(uint32_t* p, int n) {
  if (p != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Epilogues. The MFMA 16x16x32 result tile of a lane holds rows 4(l/16)+r,
// r = 0..3, of one token column l % 16.
// ---------------------------------------------------------------------------

// Output scale of a token: alpha, times the token's own factor when the
// activation has per-token dynamic scales (row_scale[token] = the token's
// global scale; the product is one fp32 multiply, as alpha itself is).
__device__ __forceinline__ float row_alpha(float alpha, const float* row_scale, bool valid, int64_t token) {
  return (row_scale != nullptr && valid) ? alpha * row_scale[token] : alpha;
}

// Dense output: out[token, row0 + r] = alpha * acc[r].
template <int E>
__device__ __forceinline__ void store_dense(const f32x4& acc, float alpha, bool valid,
                                            int64_t token, int64_t row0, int64_t N, void* out) {
  if (!valid) return;
  f32x4 v = {alpha * acc[0], alpha * acc[1], alpha * acc[2], alpha * acc[3]};
  if constexpr (E == kOutF32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + token * N + row0) = v;
  } else {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 b = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(out) + token * N + row0) = b;
  }
}

// SiLU(g) * u = g / (1 + e^-g) * u, with the hardware base-2 exponential
// and reciprocal (about 1 ulp each): h lands within a few ulp of the exactly
// rounded value, far inside the re-quantization tie window, for about a
// quarter of the instructions of expf and an IEEE division (the SiLU was the
// bulk of the standalone SiLU * mul + quantize kernel's arithmetic).
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  const float s = g * __builtin_amdgcn_rcpf(1.0f + e);
  return s * u;
}

// max(v, v of lane l ^ 16) and max(v, v of lane l ^ 32) on the VALU (no LDS
// round trip): a permlane swap of v with itself leaves v and its partner's v
// in the two results, in either order depending on the lane.
__device__ __forceinline__ float max_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// SwiGLU of matching gate/up tiles re-quantized to NVFP4. Lane l holds
// outputs j0 + 4(l/16) + r of token l % 16 (j0 a multiple of 16), so the 64
// lanes of the wave hold whole 16-element blocks of h, one per token column.
// Returns the lane's 4 codes (16 bits, element 4(l/16) + r in bits 4r..) and
// the block's scale byte. All lanes of the wave must call this (the block
// amax is a cross-lane reduction).
struct SwigluBlock {
  uint32_t codes;  // 16 bits
  uint32_t scale;  // E4M3 byte
};
__device__ __forceinline__ SwigluBlock swiglu_nvfp4(const f32x4& gate, const f32x4& up, float alpha,
                                                    float g2_inv) {
  float h[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) h[r] = silu_mul(alpha * gate[r], alpha * up[r]);
  float amax = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(h[0]), __builtin_fabsf(h[1])),
                               __builtin_fmaxf(__builtin_fabsf(h[2]), __builtin_fabsf(h[3])));
  amax = max_xor16(amax);
  amax = max_xor32(amax);
  BlockScale bs = block_scale(amax, g2_inv);
  SwigluBlock b;
  b.codes = e2m1_pack4(h[0] * bs.r, h[1] * bs.r, h[2] * bs.r, h[3] * bs.r);
  b.scale = bs.byte;
  return b;
}

// SwiGLU of matching gate/up tiles, stored. Lane layout as swiglu_nvfp4; all
// lanes of the wave must call this for the NVFP4 output.
template <int E>
__device__ __forceinline__ void store_swiglu(const f32x4& gate, const f32x4& up, float alpha,
                                             float g2_inv, bool valid, int64_t token, int64_t j0,
                                             int lane, int64_t I, void* out, uint8_t* out_scales,
                                             const uint16_t* h_scale = nullptr) {
  const int q = lane >> 4;
  const int64_t j = j0 + 4 * q;
  if constexpr (E == kSwigluF32 || E == kSwigluBF16) {
    float h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = silu_mul(alpha * gate[r], alpha * up[r]);
    if (valid) {
      if constexpr (E == kSwigluF32) {
        f32x4 v = {h[0], h[1], h[2], h[3]};
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + token * I + j) = v;
      } else {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 b = {(__bf16)h[0], (__bf16)h[1], (__bf16)h[2], (__bf16)h[3]};
        if (h_scale != nullptr) {
          // The next layer's AWQ pre-quant scale: bf16(bf16(h) * s).
          const uint2 sw = *reinterpret_cast<const uint2*>(h_scale + j);
          const float s4[4] = {__uint_as_float(sw.x << 16), __uint_as_float(sw.x & 0xFFFF0000u),
                               __uint_as_float(sw.y << 16), __uint_as_float(sw.y & 0xFFFF0000u)};
#pragma unroll
          for (int r = 0; r < 4; ++r) b[r] = (__bf16)((float)b[r] * s4[r]);
        }
        *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(out) + token * I + j) = b;
      }
    }
  } else {
    const SwigluBlock b = swiglu_nvfp4(gate, up, alpha, g2_inv);
    if (valid) {
      uint8_t* codes = reinterpret_cast<uint8_t*>(out);
      *reinterpret_cast<uint16_t*>(codes + token * (I / 2) + j / 2) = (uint16_t)b.codes;
      if (q == 0) out_scales[token * (I / 16) + j0 / 16] = (uint8_t)b.scale;
    }
  }
}

}  // namespace nvfp4
