// api.cpp -- the extern "C" entry points declared in include/nvfp4.h:
// argument validation (always before any HIP call), the gfx950 device check,
// the choice of kernel class by token count, and the launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <random>

#include "../../include/nvfp4.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";
thread_local int g_path = NVFP4_PATH_AUTO;  // nvfp4_set_path, per calling thread
// nvfp4_set_decode_wait_test, per calling thread: withhold the single-launch
// decode's records and bound its waits by this many polls (0: off).
thread_local int g_decode_test_spins = 0;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest GEMM dimension accepted: keeps every index of the 32-bit grid
// arithmetic and the 64-bit byte offsets far from overflow.
constexpr int64_t kMaxDim = int64_t(1) << 24;

bool dim_ok(int64_t v) { return v >= 0 && v <= kMaxDim; }

// gfx950 check, cached per device.
int check_device() {
  static std::mutex mu;
  static int cached[64];
  static bool init = false;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(NVFP4_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(NVFP4_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!init) {
    for (int& c : cached) c = -1;
    init = true;
  }
  if (cached[dev] < 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(NVFP4_ERR_HIP, "hipGetDeviceProperties failed");
    cached[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 0;
    if (!cached[dev]) {
      fail(NVFP4_ERR_UNSUPPORTED, "device %d is %s; this library runs on gfx950 (MI355X) only", dev,
           prop.gcnArchName);
    }
  }
  if (cached[dev] != 1)
    return fail(NVFP4_ERR_UNSUPPORTED, "device %d is not gfx950 (MI355X); no other path exists", dev);
  return NVFP4_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return NVFP4_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Epochs of the single-launch decode kernel's records: a new value for every
// launch, counting up from a random start drawn once per process (records
// are tagged with the low 32 bits, which are never 0, the tag of no record).
uint64_t next_epoch() {
  static std::atomic<uint64_t> epoch{0};
  static std::once_flag once;
  std::call_once(once, [] {
    std::random_device rd;
    const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    epoch.store((((uint64_t)rd() << 32) | rd()) ^ (t * 0x9E3779B97F4A7C15ull));
  });
  for (;;) {
    const uint64_t e = epoch.fetch_add(1) + 1;
    if ((uint32_t)e != 0u) return e;
  }
}

// The decode kernel needs a fresh epoch per launch, which a replayed graph
// would not give: under stream capture the two-kernel path runs.
bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) return true;
  return cs != hipStreamCaptureStatusNone;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Largest token count the weight-streaming kernel takes under the
// automatic path, from the forward measured on both paths (hidden 5120 and
// 7168): W4A4 streaming beats the 256-token tiled kernel up to 128 tokens
// (80: 233 against 274 us, hidden 7168; 128: 206 against 228 us, hidden
// 5120, a tie at 7168) and loses from 144 (349 against 279 us); W4A16
// streaming wins up to 48 (117 against 122 us) and loses at 56 (148 against
// 124 us) to the 128-token tiled kernel. W4A16 dense GEMMs, whose
// streaming grids fill one round with 5, 7 or 8 row groups per workgroup
// (stream_groups), stream up to 96 tokens: the forward at 49 / 64 / 72 / 96
// tokens, hidden 5120, 116.5 / 118.3 / 122.2 / 123.6 us with a tiled down
// projection against 95.3 / 96.3 / 119.7 / 121.5 streaming.
int64_t stream_max_m(int mode, bool swiglu) { return mode == NVFP4_MODE_W4A4 ? 128 : swiglu ? 48 : 96; }

// Largest tokens per expert a grouped GEMM runs as one streaming launch
// over all experts under the automatic path.
constexpr int64_t kGroupedStreamMaxM = 256;
constexpr int64_t kGroupedMidMinM = 64, kGroupedMidMaxM = 512;

// Token counts at which a W4A4 GEMM with a SwiGLU epilogue (the gate_up of
// the MLP) runs the mid-size kernel under the automatic path. Gate_up alone
// (hidden 7168 / 5120): 64 tokens 78.9 / 61.0 us streaming against 69.0 /
// 51.8; 128: 138.0 / 103.6 against 106.9 / 78.3; 256: 183.1 / 135.0 tiled
// against 161.5 / 121.1; up to 48 tokens the 48-token tile: 40 / 48 tokens
// 56.5 / 62.1 and 42.3 / 46.6 streaming against 52.2 / 53.2 and 39.4 /
// 40.2, a tie at 33 (51.9 / 39.0 against 51.6 / 39.2) and streaming ahead
// at 32 (41.9 / 32.2 against 51.3 / 38.6). Whole forward, tiled gate_up (with its K-split tail)
// against mid-size: 384 tokens 439.4 / 345.4 against 374.7 / 276.4 us, 512:
// 463.7 / 362.9 against 441.9 / 322.9; 768: 608.7 / 442.7 against 633.9 /
// 443.3, and the tiled kernel wins above. Dense GEMMs (the down projection,
// 5120 / 7168 rows: 40 / 56 mid-size workgroups per 64 tokens) keep the
// streaming and tiled kernels, whose split-K fills the CUs.
constexpr int64_t kMidMinM = 33, kMidMaxM = 512;

// W4A16 SwiGLU GEMMs take the mid-size kernel from 33 to 64 tokens, where
// its 48- and 64-token tiles beat the streaming kernel and the 128-token
// tiled one. Gate_up alone, hidden 5120: 33 / 40 / 48 / 64 tokens 62.7 /
// 64.9 / 67.3 / 64.8 us (streaming up to 48, then tiled) against 50.5 /
// 51.6 / 54.0 / 61.1; whole forward at 40 / 48 / 64 tokens 96.2 / 98.9 /
// 121.6 against 83.4 / 85.0 / 118.6 us. It loses at 32 (50.0 against
// 56.5 with the 64-token tile) and from 65 to 128 (65.9 against 96.6 at
// 128: one tiled token tile). From 129 to 192 tokens it
// beats the tiled gate_up alone (113.8 against 128.9 at 192) but not the
// forward's, whose tail tiles are K-split (184.9 against 168.7 us).
bool mid_w4a16(int64_t M) { return M >= 33 && M <= 64; }

// Kernel class for a GEMM of M tokens: the decode GEMV up to M = 2 (W4A4,
// whose FP4 GEMV carries two tokens per workgroup) or M = 1 (W4A16), the
// mid-size kernel for the SwiGLU GEMMs of kMidMinM..kMidMaxM tokens (W4A4)
// or mid_w4a16 (W4A16), the weight-streaming MFMA kernel up to
// stream_max_m, the LDS-tiled kernel above.
int choose_path(int mode, int64_t M, bool swiglu) {
  int p = g_path;
  if (p != NVFP4_PATH_AUTO) return p;
  if (M <= (mode == NVFP4_MODE_W4A4 ? 2 : 1)) return NVFP4_PATH_GEMV;
  if (mode == NVFP4_MODE_W4A4 && swiglu && M >= kMidMinM && M <= kMidMaxM) return NVFP4_PATH_MID;
  if (mode != NVFP4_MODE_W4A4 && swiglu && mid_w4a16(M)) return NVFP4_PATH_MID;
  if (M <= stream_max_m(mode, swiglu)) return NVFP4_PATH_STREAM;
  return NVFP4_PATH_TILED;
}

// K splits of a dense GEMM on the mid-size kernels: as many as bring the
// grid to about two workgroups per CU (their occupancy), at most 8, every
// split non-empty and at least 8 K tiles long.
int64_t mid_ways(int mode, int64_t M, int64_t N, int64_t K) {
  const int64_t units = nvfp4::mid_shape(mode, M, N).units, T = K / 256;
  int64_t ks = std::min<int64_t>(2 * nvfp4::kTiledSlots / std::max<int64_t>(units, 1), 8);
  while (ks > 1 && ((ks - 1) * ((T + ks - 1) / ks) >= T || (T + ks - 1) / ks < 8)) --ks;
  return std::max<int64_t>(ks, 1);
}

// Path of mlp_forward's down projection (a dense GEMM that can split K
// through the workspace): the mid-size kernels wherever they K-split (at
// most 256 output tiles of 128 rows x 48 or 64 tokens, or W4A4 x 128
// tokens where the smaller tiles are more), W4A4 from 17 tokens and W4A16
// from 65 to 192, else as choose_path. The W4A4 forward
// at hidden 7168 / 5120 (same box, same run): 17 tokens 69.1 / 57.7 -> 67.3
// / 56.4 us, 64: 109.4 / 90.1 -> 102.6 / 83.8, 96: 144.2 -> 118.6 (7168),
// 128: 179.0 / 148.3 -> 153.6 / 114.9, 256: 258.7 / 213.8 -> 246.8 / 177.3,
// 320: 246.1 -> 216.5 (5120); unsplit it lost at 320 (7168), 384 (5120),
// 448 and 512 (both). W4A16, hidden 5120: 80 / 96 / 128 / 192 tokens
// 119.9 / 121.3 / 125.9 / 169.4 -> 105.2 / 106.4 / 113.5 / 164.1 us; at
// 49-64 tokens the streaming kernel's one-round grid wins (95.2 against
// 98.4 us at 49), at 256-320 the tiled kernel (174.2 against 177.2 at 256).
int choose_path_down(int mode, int64_t M, int64_t H, int64_t I) {
  const bool mid = mode == NVFP4_MODE_W4A4 ? M >= 17 : (M >= 65 && M <= 192);
  if (g_path == NVFP4_PATH_AUTO && mid && mid_ways(mode, M, H, I) > 1) return NVFP4_PATH_MID;
  return choose_path(mode, M, false);
}

// Kernels that address their operands with 32-bit buffer offsets: the packed
// weight and the activation rows (including one tile of padding past M) must
// stay below 2^31 bytes.
bool fits_buffers(const nvfp4::GemmArgs& a, int mode) {
  const int64_t lim = int64_t(1) << 31;
  const int64_t row = mode == NVFP4_MODE_W4A4 ? a.K / 2 : a.K * 2;
  return a.N * a.K / 16 * 9 < lim && (a.M + 256) * row < lim;
}

// The kernel a GEMM runs on, from the path and what the operands allow.
enum Kernel { kFp4Gemv, kValuGemv, kStream, kTiled2, kTiled16, kTiled, kMid };

Kernel select_kernel(int path, int mode, const nvfp4::GemmArgs& a) {
  if (path != NVFP4_PATH_TILED64 && fits_buffers(a, mode)) {
    if (path == NVFP4_PATH_GEMV) {
      if (mode == NVFP4_MODE_W4A4 && nvfp4::fp4_gemv_supported(a.M, a.K)) return kFp4Gemv;
      if (mode == NVFP4_MODE_W4A16 && a.K * 2 + 16 <= nvfp4::kValuGemvLdsBytes) return kValuGemv;
      return kStream;
    }
    if (path == NVFP4_PATH_STREAM) return kStream;
    if (path == NVFP4_PATH_MID) return nvfp4::mid_supported(a) ? kMid : kStream;
    return mode == NVFP4_MODE_W4A4 ? kTiled2 : kTiled16;
  }
  // Beyond 2^31-byte operands only the 64-bit-addressed tiled kernel runs
  // (and under the override that forces it at any size).
  return kTiled;
}

hipError_t run_gemm(int path, int mode, int epi, const nvfp4::GemmArgs& a, hipStream_t s) {
  switch (select_kernel(path, mode, a)) {
    case kFp4Gemv: return nvfp4::launch_fp4_gemv(epi, a, s);
    case kValuGemv: return nvfp4::launch_valu_gemv(mode, epi, a, s);
    case kStream: return nvfp4::launch_stream_gemm(mode, epi, a, s);
    case kTiled2: return nvfp4::launch_tiled2_gemm(epi, a, s);
    case kTiled16: return nvfp4::launch_tiled16_gemm(epi, a, s);
    case kMid: return nvfp4::launch_mid_gemm(mode, epi, a, s);
    default: return nvfp4::launch_tiled_gemm(mode, epi, a, s);
  }
}

// Split-K of a dense GEMM on the weight-streaming kernel: only a grid of
// fewer output tiles than a quarter of the CUs is split, into at most as
// many ways as keep one workgroup per CU, at least 4 K tiles per split.
// Larger grids run unsplit: with 2 row groups x 8 waves per workgroup the
// down projection at 4 and 16 tokens (160 tiles at hidden 5120, 224 at
// 7168) measured 14.4 / 16.0 us unsplit against 16.4 / 19.0 (2 ways),
// 14.7 / 16.4 (3 ways) and 19.9 / 21.3 (7 ways), and 17.5 against 24.5 us
// at 16 tokens on hidden 7168: the dense kernel's register use leaves 2
// such workgroups per CU, and the partial-sum exchange adds three
// dependent memory round trips to every tile. (The decode GEMVs do not
// split either.)
constexpr int64_t kStreamSplitMaxUnits = 64;
constexpr int64_t kStreamSplitTargetWgs = 256;

struct SplitPlan {
  int ways = 1;
  int64_t units = 0;
  size_t part_bytes = 0, counter_bytes = 0;
};

// Tail split of a tiled kernel's grid: when its last round of one
// workgroup per CU is at most half full, the tail tiles are K-split into as
// many splits as fill that round (at most 8, at least min_tiles K tiles
// each).
// K splits that put `units` tiles into one round of the tiled kernels (at
// most 8, every split non-empty and at least min_tiles of the T K tiles).
static int64_t round_ways(int64_t units, int64_t T, int64_t min_tiles) {
  int64_t ks = std::min<int64_t>(nvfp4::kTiledSlots / units, 8);
  while (ks > 1 && ((ks - 1) * ((T + ks - 1) / ks) >= T || (T + ks - 1) / ks < min_tiles)) --ks;
  return std::max<int64_t>(ks, 1);
}

static SplitPlan tail_split(const nvfp4::TileShape& ts, int64_t K, int64_t min_tiles) {
  SplitPlan p;
  const int64_t tail = nvfp4::tiled_tail(ts.units);
  if (tail == 0 || 2 * tail > nvfp4::kTiledSlots) return p;
  const int64_t ks = round_ways(tail, K / 256, min_tiles);
  if (ks <= 1) return p;
  p.ways = (int)ks;
  p.units = tail;
  p.part_bytes = align256((size_t)(tail * ks * ts.tile_floats) * sizeof(float));
  p.counter_bytes = align256((size_t)tail * sizeof(uint32_t));
  return p;
}

// Split-K plan of a GEMM of mlp_forward (swiglu: the gate_up GEMM).
SplitPlan split_plan(Kernel k, int mode, int64_t M, int64_t N, int64_t K, bool swiglu) {
  SplitPlan p;
  if (M <= 0) return p;
  // The W4A4 tiled kernel: a grid of less than one round (dense epilogues:
  // the down projection at a few hundred tokens) into as many K splits as
  // fill one round, else the tail tiles; at least 8 K tiles per split.
  if (k == kTiled2) {
    const nvfp4::TileShape ts = nvfp4::tiled2_shape(M, N);
    if (ts.units >= nvfp4::kTiledSlots) return tail_split(ts, K, 8);
    if (swiglu) return p;
    p.ways = (int)round_ways(ts.units, K / 256, 8);
    if (p.ways > 1) {
      p.units = ts.units;
      p.part_bytes = align256((size_t)(ts.units * p.ways * ts.tile_floats) * sizeof(float));
      p.counter_bytes = align256((size_t)ts.units * sizeof(uint32_t));
    }
    return p;
  }
  if (k == kTiled16) {
    // The W4A16 tiled kernel (one 8-wave workgroup per CU): a grid of less
    // than one round (dense epilogues: the down projection at a few hundred
    // tokens) into as many K splits as fill one round, at least 4 K tiles
    // each (forward at 256 tokens, hidden 5120: 216 -> 183 us against
    // splitting to about two rounds); a larger grid in its tail tiles (the
    // gate_up at 256 tokens: 272 tiles).
    const nvfp4::TileShape ts = nvfp4::tiled16_shape(M, N);
    if (ts.units >= nvfp4::kTiledSlots) return tail_split(ts, K, 4);
    if (swiglu) return p;
    p.ways = (int)round_ways(ts.units, K / 256, 4);
    if (p.ways > 1) {
      p.units = ts.units;
      p.part_bytes = align256((size_t)(ts.units * p.ways * ts.tile_floats) * sizeof(float));
      p.counter_bytes = align256((size_t)ts.units * sizeof(uint32_t));
    }
    return p;
  }
  if (k == kMid) {
    // Dense epilogues only (mid_ways).
    if (swiglu) return p;
    const nvfp4::TileShape ts = nvfp4::mid_shape(mode, M, N);
    const int64_t ks = mid_ways(mode, M, N, K);
    if (ks > 1) {
      p.ways = (int)ks;
      p.units = ts.units;
      p.part_bytes = align256((size_t)(ts.units * ks * ts.tile_floats) * sizeof(float));
      p.counter_bytes = align256((size_t)ts.units * sizeof(uint32_t));
    }
    return p;
  }
  if (k != kStream || swiglu) return p;
  const nvfp4::TileShape ts = nvfp4::stream_shape(mode, M, N);
  if (ts.units >= kStreamSplitMaxUnits) return p;
  p.ways = nvfp4::splitk_ways(ts.units, K / 256, kStreamSplitTargetWgs, 4);
  if (p.ways > 1) {
    p.units = ts.units;
    p.part_bytes = align256((size_t)(ts.units * p.ways * ts.tile_floats) * sizeof(float));
    p.counter_bytes = align256((size_t)ts.units * sizeof(uint32_t));
  }
  return p;
}

// Kernel of an mlp_forward GEMM (the activation buffers do not matter for
// the choice beyond their size, which depends on M and K only).
Kernel mlp_kernel(int path, int mode, int64_t M, int64_t N, int64_t K) {
  nvfp4::GemmArgs a{};
  a.M = M;
  a.N = N;
  a.K = K;
  return select_kernel(path, mode, a);
}

// The kernels that clear the split-K counters of the GEMM after them.
bool clears_counters(Kernel k) {
  return k == kFp4Gemv || k == kValuGemv || k == kStream || k == kTiled2 || k == kTiled16 || k == kMid;
}

// Shared checks of the GEMM entry points. N is the packed row count.
int check_gemm(int mode, const void* a, const uint8_t* a_scales, const void* w, int64_t M,
               int64_t N, int64_t K, const float* alpha, const void* out) {
  if (mode != NVFP4_MODE_W4A4 && mode != NVFP4_MODE_W4A16)
    return fail(NVFP4_ERR_INVALID_ARG, "unsupported quant mode %d (W4A4=0, W4A16=1)", mode);
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K)) return fail(NVFP4_ERR_INVALID_ARG, "dimension out of range");
  if (K <= 0 || K % 256 != 0) return fail(NVFP4_ERR_INVALID_ARG, "K=%lld must be a positive multiple of 256", (long long)K);
  if (N <= 0 || N % 16 != 0) return fail(NVFP4_ERR_INVALID_ARG, "N=%lld must be a positive multiple of 16", (long long)N);
  if (M > 0) {
    if (!a || !w || !alpha || !out) return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(a) || !aligned16(w) || !aligned16(out))
      return fail(NVFP4_ERR_INVALID_ARG, "activation, weight and output must be 16-byte aligned");
    if (mode == NVFP4_MODE_W4A4 && !a_scales)
      return fail(NVFP4_ERR_INVALID_ARG, "W4A4 needs activation scales");
    if (mode == NVFP4_MODE_W4A4 && !aligned16(a_scales))
      return fail(NVFP4_ERR_INVALID_ARG, "activation scales must be 16-byte aligned");
  }
  if (mode == NVFP4_MODE_W4A16 && a_scales)
    return fail(NVFP4_ERR_INVALID_ARG, "W4A16 takes bf16 activations: a_scales must be NULL");
  return NVFP4_OK;
}

}  // namespace

extern "C" {

const char* nvfp4_last_error(void) { return g_err; }

int nvfp4_set_path(int path) {
  if (path < NVFP4_PATH_AUTO || path > NVFP4_PATH_MID)
    return fail(NVFP4_ERR_INVALID_ARG, "unknown path %d", path);
  const int prev = g_path;
  g_path = path;
  return prev;
}

int nvfp4_calibrate(const void* x, int x_dtype, int64_t n, float* g, float* g_inv, void* stream) {
  if (x_dtype != NVFP4_DTYPE_BF16 && x_dtype != NVFP4_DTYPE_F32)
    return fail(NVFP4_ERR_INVALID_ARG, "x_dtype must be BF16 or F32");
  if (n <= 0 || n > (int64_t(1) << 40)) return fail(NVFP4_ERR_INVALID_ARG, "n must be positive");
  if (!x || !g || !g_inv) return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
  if (reinterpret_cast<uintptr_t>(g) % 4 || reinterpret_cast<uintptr_t>(g_inv) % 4)
    return fail(NVFP4_ERR_INVALID_ARG, "g and g_inv must be 4-byte aligned");
  if (g == g_inv) return fail(NVFP4_ERR_INVALID_ARG, "g and g_inv must differ");
  int st = check_device();
  if (st) return st;
  return hip_status(nvfp4::launch_calibrate(x, x_dtype == NVFP4_DTYPE_F32, n, g, g_inv, as_stream(stream)),
                    "calibrate launch");
}

int nvfp4_quantize(const void* x, int x_dtype, int64_t M, int64_t K, const float* g_inv,
                   uint8_t* codes, uint8_t* scales, void* stream) {
  if (x_dtype != NVFP4_DTYPE_BF16 && x_dtype != NVFP4_DTYPE_F32)
    return fail(NVFP4_ERR_INVALID_ARG, "x_dtype must be BF16 or F32");
  if (!dim_ok(M) || K < 0 || K > (int64_t(1) << 30) || K % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "need 0 <= M <= 2^24 and 0 <= K <= 2^30 a multiple of 16 (M=%lld K=%lld)",
                (long long)M, (long long)K);
  if (M * K == 0) { g_err[0] = '\0'; return NVFP4_OK; }
  if (!x || !g_inv || !codes || !scales) return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(x) || !aligned16(codes))
    return fail(NVFP4_ERR_INVALID_ARG, "x and codes must be 16-byte aligned");
  int st = check_device();
  if (st) return st;
  return hip_status(nvfp4::launch_quantize(x, x_dtype == NVFP4_DTYPE_F32, M, K, g_inv, codes, scales,
                                           as_stream(stream)),
                    "quantize launch");
}

int nvfp4_quantize_per_token(const void* x, int x_dtype, int64_t M, int64_t K, uint8_t* codes,
                             uint8_t* scales, float* row_g, void* stream) {
  if (x_dtype != NVFP4_DTYPE_BF16 && x_dtype != NVFP4_DTYPE_F32)
    return fail(NVFP4_ERR_INVALID_ARG, "x_dtype must be BF16 or F32");
  if (!dim_ok(M) || K < 0 || K > (int64_t(1) << 30) || K % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "need 0 <= M <= 2^24 and 0 <= K <= 2^30 a multiple of 16 (M=%lld K=%lld)",
                (long long)M, (long long)K);
  if (M * K == 0) { g_err[0] = '\0'; return NVFP4_OK; }
  if (!x || !codes || !scales || !row_g) return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(x) || !aligned16(codes) || reinterpret_cast<uintptr_t>(row_g) % 4)
    return fail(NVFP4_ERR_INVALID_ARG, "x and codes must be 16-byte aligned, row_g 4-byte aligned");
  int st = check_device();
  if (st) return st;
  return hip_status(nvfp4::launch_quantize_per_token(x, x_dtype == NVFP4_DTYPE_F32, M, K, codes, scales, row_g,
                                                     as_stream(stream)),
                    "quantize_per_token launch");
}

int silu_mul_nvfp4_quant(const void* gate_up, int64_t E, int64_t M, int64_t I, const int32_t* masked_m,
                         const float* g_inv, uint8_t* codes, uint8_t* scales, void* stream) {
  if (E < 0 || M < 0 || E >= 65536 || M >= 65536 || !dim_ok(I) || I < 0 || I % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "need 0 <= E, M < 65536 and I a multiple of 16 (E=%lld M=%lld I=%lld)",
                (long long)E, (long long)M, (long long)I);
  if (E * M * I == 0) { g_err[0] = '\0'; return NVFP4_OK; }
  if (!gate_up || !g_inv || !codes || !scales) return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(gate_up) || !aligned16(codes) || reinterpret_cast<uintptr_t>(g_inv) % 4 ||
      reinterpret_cast<uintptr_t>(masked_m) % 4)
    return fail(NVFP4_ERR_INVALID_ARG, "gate_up and codes must be 16-byte aligned, g_inv and masked_m 4-byte");
  int st = check_device();
  if (st) return st;
  return hip_status(nvfp4::launch_silu_mul_quant(gate_up, E, M, I, masked_m, g_inv, codes, scales,
                                                 as_stream(stream)),
                    "silu_mul_nvfp4_quant launch");
}

size_t nvfp4_repack_bytes(int kind, int64_t R, int64_t C) {
  if (kind != NVFP4_REPACK_PLAIN && kind != NVFP4_REPACK_SWIGLU) return 0;
  if (R <= 0 || C <= 0 || R % 16 != 0 || C % 256 != 0 || R > kMaxDim || C > kMaxDim) return 0;
  if (kind == NVFP4_REPACK_SWIGLU && (R / 2) % 16 != 0) return 0;
  return static_cast<size_t>(R) * static_cast<size_t>(C) / 16 * 9;
}

size_t nvfp4_packed_bytes(int kind, int64_t R, int64_t C) { return nvfp4_repack_bytes(kind, R, C); }

static int repack_common(int kind, const uint8_t* codes, const uint8_t* scales, int64_t R, int64_t C,
                         const void* packed, bool unpack, uint8_t* oc, uint8_t* os, void* stream) {
  if (nvfp4_repack_bytes(kind, R, C) == 0)
    return fail(NVFP4_ERR_INVALID_ARG,
                "repack needs kind PLAIN/SWIGLU, R %% 16 == 0 (SWIGLU: R/2 %% 16 == 0), C %% 256 == 0 "
                "(kind=%d R=%lld C=%lld)", kind, (long long)R, (long long)C);
  if (!packed) return fail(NVFP4_ERR_INVALID_ARG, "null packed pointer");
  if (unpack ? (!oc || !os) : (!codes || !scales)) return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(packed) || !aligned16(unpack ? oc : codes))
    return fail(NVFP4_ERR_INVALID_ARG, "packed and codes must be 16-byte aligned");
  int st = check_device();
  if (st) return st;
  return hip_status(nvfp4::launch_repack(kind, codes, scales, R, C,
                                         const_cast<uint8_t*>(static_cast<const uint8_t*>(packed)), unpack,
                                         oc, os, as_stream(stream)),
                    "repack launch");
}

int nvfp4_repack_weight(int kind, const uint8_t* codes, const uint8_t* scales, int64_t R, int64_t C,
                        void* packed, void* stream) {
  return repack_common(kind, codes, scales, R, C, packed, false, nullptr, nullptr, stream);
}

int nvfp4_unpack_weight(int kind, const void* packed, int64_t R, int64_t C, uint8_t* codes,
                        uint8_t* scales, void* stream) {
  return repack_common(kind, nullptr, nullptr, R, C, packed, true, codes, scales, stream);
}

int nvfp4_gemm(int mode, const void* a, const uint8_t* a_scales, const void* w_packed, int64_t M,
               int64_t N, int64_t K, const float* alpha, void* out, int out_dtype, void* stream) {
  int st = check_gemm(mode, a, a_scales, w_packed, M, N, K, alpha, out);
  if (st) return st;
  if (out_dtype != NVFP4_DTYPE_F32 && out_dtype != NVFP4_DTYPE_BF16)
    return fail(NVFP4_ERR_INVALID_ARG, "out_dtype must be F32 or BF16");
  if (M == 0) { g_err[0] = '\0'; return NVFP4_OK; }
  st = check_device();
  if (st) return st;
  nvfp4::GemmArgs ga{a, a_scales, static_cast<const uint8_t*>(w_packed), M, N, K, alpha, nullptr, out, nullptr};
  const int epi = out_dtype == NVFP4_DTYPE_F32 ? nvfp4::kOutF32 : nvfp4::kOutBF16;
  return hip_status(run_gemm(choose_path(mode, M, false), mode, epi, ga, as_stream(stream)), "gemm launch");
}

int gemm_swiglu_nvfp4_quant(const uint8_t* a_codes, const uint8_t* a_scales, const void* w_gu_packed,
                            int64_t M, int64_t I, int64_t K, const float* alpha, const float* g2_inv,
                            uint8_t* h_codes, uint8_t* h_scales, void* stream) {
  if (!dim_ok(I) || I <= 0 || I % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "I=%lld must be a positive multiple of 16", (long long)I);
  int st = check_gemm(NVFP4_MODE_W4A4, a_codes, a_scales, w_gu_packed, M, 2 * I, K, alpha, h_codes);
  if (st) return st;
  if (M > 0 && (!g2_inv || !h_scales)) return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
  if (M == 0) { g_err[0] = '\0'; return NVFP4_OK; }
  st = check_device();
  if (st) return st;
  nvfp4::GemmArgs ga{a_codes, a_scales, static_cast<const uint8_t*>(w_gu_packed), M, 2 * I, K, alpha, g2_inv,
                     h_codes, h_scales};
  return hip_status(run_gemm(choose_path(NVFP4_MODE_W4A4, M, true), NVFP4_MODE_W4A4, nvfp4::kSwigluNvfp4, ga, as_stream(stream)),
                    "gemm_swiglu_nvfp4_quant launch");
}

int nvfp4_gemm_rowscale(const uint8_t* a_codes, const uint8_t* a_scales, const float* row_g,
                        const void* w_packed, int64_t M, int64_t N, int64_t K, const float* g_w,
                        void* out, int out_dtype, void* stream) {
  int st = check_gemm(NVFP4_MODE_W4A4, a_codes, a_scales, w_packed, M, N, K, g_w, out);
  if (st) return st;
  if (out_dtype != NVFP4_DTYPE_F32 && out_dtype != NVFP4_DTYPE_BF16)
    return fail(NVFP4_ERR_INVALID_ARG, "out_dtype must be F32 or BF16");
  if (M > 0 && !row_g) return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
  if (M == 0) { g_err[0] = '\0'; return NVFP4_OK; }
  st = check_device();
  if (st) return st;
  nvfp4::GemmArgs ga{a_codes, a_scales, static_cast<const uint8_t*>(w_packed), M, N, K, g_w, nullptr, out, nullptr};
  ga.row_scale = row_g;
  const int epi = out_dtype == NVFP4_DTYPE_F32 ? nvfp4::kOutF32 : nvfp4::kOutBF16;
  return hip_status(run_gemm(choose_path(NVFP4_MODE_W4A4, M, false), NVFP4_MODE_W4A4, epi, ga, as_stream(stream)),
                    "gemm_rowscale launch");
}

int gemm_swiglu_nvfp4_quant_rowscale(const uint8_t* a_codes, const uint8_t* a_scales, const float* row_g,
                                     const void* w_gu_packed, int64_t M, int64_t I, int64_t K,
                                     const float* g_w, const float* g2_inv, uint8_t* h_codes,
                                     uint8_t* h_scales, void* stream) {
  if (!dim_ok(I) || I <= 0 || I % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "I=%lld must be a positive multiple of 16", (long long)I);
  int st = check_gemm(NVFP4_MODE_W4A4, a_codes, a_scales, w_gu_packed, M, 2 * I, K, g_w, h_codes);
  if (st) return st;
  if (M > 0 && (!g2_inv || !h_scales || !row_g)) return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
  if (M == 0) { g_err[0] = '\0'; return NVFP4_OK; }
  st = check_device();
  if (st) return st;
  nvfp4::GemmArgs ga{a_codes, a_scales, static_cast<const uint8_t*>(w_gu_packed), M, 2 * I, K, g_w, g2_inv,
                     h_codes, h_scales};
  ga.row_scale = row_g;
  return hip_status(run_gemm(choose_path(NVFP4_MODE_W4A4, M, true), NVFP4_MODE_W4A4, nvfp4::kSwigluNvfp4, ga,
                             as_stream(stream)),
                    "gemm_swiglu_nvfp4_quant_rowscale launch");
}

int gemm_swiglu(int mode, const void* a, const uint8_t* a_scales, const void* w_gu_packed, int64_t M,
                int64_t I, int64_t K, const float* alpha, void* h, int h_dtype, void* stream) {
  if (!dim_ok(I) || I <= 0 || I % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "I=%lld must be a positive multiple of 16", (long long)I);
  int st = check_gemm(mode, a, a_scales, w_gu_packed, M, 2 * I, K, alpha, h);
  if (st) return st;
  if (h_dtype != NVFP4_DTYPE_F32 && h_dtype != NVFP4_DTYPE_BF16)
    return fail(NVFP4_ERR_INVALID_ARG, "h_dtype must be F32 or BF16");
  if (M == 0) { g_err[0] = '\0'; return NVFP4_OK; }
  st = check_device();
  if (st) return st;
  nvfp4::GemmArgs ga{a, a_scales, static_cast<const uint8_t*>(w_gu_packed), M, 2 * I, K, alpha, nullptr, h, nullptr};
  const int epi = h_dtype == NVFP4_DTYPE_F32 ? nvfp4::kSwigluF32 : nvfp4::kSwigluBF16;
  return hip_status(run_gemm(choose_path(mode, M, true), mode, epi, ga, as_stream(stream)), "gemm_swiglu launch");
}

// Activation part of the workspace: W4A4 x and h as NVFP4 (W4A4_DYN then
// x's per-token g), W4A16 h in bf16.
static size_t mlp_act_bytes(int mode, size_t m, int64_t H, int64_t I) {
  const size_t nvfp4 = align256(m * H / 2) + align256(m * H / 16) + align256(m * I / 2) + align256(m * I / 16);
  if (mode == NVFP4_MODE_W4A4) return nvfp4;
  if (mode == NVFP4_MODE_W4A4_DYN) return nvfp4 + align256(m * sizeof(float));
  if (mode == NVFP4_MODE_W4A16_AWQ) return align256(m * I * 2) + align256(m * H * 2);  // h, then x'
  return align256(m * I * 2);
}

// Records of the single-launch W4A4 decode kernel (0 where it cannot run).
static size_t decode_bytes(int64_t H, int64_t I) {
  if (!nvfp4::decode_supported(H, I)) return 0;
  return align256((size_t)nvfp4::decode_record_words(H, I) * sizeof(uint64_t));
}

// Records of the single-launch W4A16 decode kernel (0 where it cannot run).
static size_t decode16_bytes(int64_t H, int64_t I) {
  if (!nvfp4::decode16_supported(H, I)) return 0;
  return align256((size_t)nvfp4::decode16_record_words(H, I) * sizeof(uint64_t));
}

// The tail of every mlp_forward workspace, counted from the END of the
// buffer as the caller passes it (ws + ws_bytes): the status word in its
// last 4 bytes and, 256 bytes before it, the single-launch decode kernel's
// records. Its size is the same for every mode, token count and shape, so no
// other call on a buffer shared with the same ws_bytes writes there, and the
// records stay as the decode launches leave them. 4 MiB holds the records of
// every shape the decode kernels take (the W4A4 one's LDS bounds H and I by
// 61440 and its 31-bit offsets H * I by 1.9e9: at most 3.98 MB; the W4A16
// one's LDS bounds H by 32760 and its splits I by 32768: at most 2.3 MB)
// plus the status word and the records' alignment; decode_in_tail checks
// it per shape.
constexpr size_t kTailBytes = size_t(4) << 20;
static size_t tail_bytes(int64_t, int64_t) { return kTailBytes; }
static bool decode_in_tail(int64_t H, int64_t I) {
  return nvfp4::decode_supported(H, I) && decode_bytes(H, I) + 512 <= kTailBytes;
}
static bool decode16_in_tail(int64_t H, int64_t I) {
  return nvfp4::decode16_supported(H, I) && decode16_bytes(H, I) + 512 <= kTailBytes;
}

static uint32_t* tail_status(void* ws, size_t ws_bytes) {
  return reinterpret_cast<uint32_t*>((reinterpret_cast<uintptr_t>(ws) + ws_bytes - 4) & ~uintptr_t(3));
}

static uint64_t* tail_records(void* ws, size_t ws_bytes, size_t record_bytes) {
  const uintptr_t end = reinterpret_cast<uintptr_t>(ws) + ws_bytes;
  return reinterpret_cast<uint64_t*>((end - 256 - record_bytes) & ~uintptr_t(255));
}

// Split-K partials and counters of the largest plan over the kernels of
// every path, for either GEMM on any path (the automatic path picks the
// gate_up's and the down projection's separately), so the size does not
// depend on the path override.
static size_t mlp_split_bytes(int mode, int64_t M, int64_t H, int64_t I) {
  size_t most = 0;
  constexpr int kPaths[] = {NVFP4_PATH_GEMV, NVFP4_PATH_STREAM, NVFP4_PATH_TILED, NVFP4_PATH_TILED64, NVFP4_PATH_MID};
  for (int pg : kPaths) {
    const SplitPlan g = split_plan(mlp_kernel(pg, mode, M, 2 * I, H), mode, M, 2 * I, H, true);
    for (int pd : kPaths) {
      // The two GEMMs share the partials region (they run one after the
      // other) and have counters of their own.
      const SplitPlan d = split_plan(mlp_kernel(pd, mode, M, H, I), mode, M, H, I, false);
      most = std::max(most, std::max(d.part_bytes, g.part_bytes) + d.counter_bytes + g.counter_bytes);
    }
  }
  return most;
}

// Workspace of an mlp_forward call on one path (the size of mlp_workspace_bytes
// with the split-K plan of that path's kernels only).
static size_t mlp_path_bytes(int mode, int64_t M, int64_t H, int64_t I, int path_gu, int path_d) {
  const int kmode = (mode == NVFP4_MODE_W4A16 || mode == NVFP4_MODE_W4A16_AWQ) ? NVFP4_MODE_W4A16 : NVFP4_MODE_W4A4;
  const SplitPlan d = split_plan(mlp_kernel(path_d, kmode, M, H, I), kmode, M, H, I, false);
  const SplitPlan g = split_plan(mlp_kernel(path_gu, kmode, M, 2 * I, H), kmode, M, 2 * I, H, true);
  return mlp_act_bytes(mode, static_cast<size_t>(M), H, I) + std::max(d.part_bytes, g.part_bytes) + d.counter_bytes +
         g.counter_bytes + tail_bytes(H, I);
}

size_t mlp_workspace_bytes(int mode, int64_t M, int64_t H, int64_t I) {
  if (M < 0 || H <= 0 || I <= 0 || !dim_ok(M) || !dim_ok(H) || !dim_ok(I)) return 0;
  if (mode != NVFP4_MODE_W4A4 && mode != NVFP4_MODE_W4A16 && mode != NVFP4_MODE_W4A4_DYN &&
      mode != NVFP4_MODE_W4A16_AWQ)
    return 0;
  // W4A4_DYN runs the W4A4 GEMM kernels, never the single-launch decode
  // one; W4A16_AWQ the W4A16 ones.
  const int kmode = (mode == NVFP4_MODE_W4A16 || mode == NVFP4_MODE_W4A16_AWQ) ? NVFP4_MODE_W4A16 : NVFP4_MODE_W4A4;
  return mlp_act_bytes(mode, static_cast<size_t>(M), H, I) + mlp_split_bytes(kmode, M, H, I) + tail_bytes(H, I);
}

uint32_t* mlp_workspace_status(void* ws, size_t ws_bytes) {
  if (!ws || ws_bytes < 512) return nullptr;
  return tail_status(ws, ws_bytes);
}

int nvfp4_set_decode_wait_test(int withhold, int spin_limit) {
  if (withhold && spin_limit < 1) return fail(NVFP4_ERR_INVALID_ARG, "spin_limit must be positive");
  g_decode_test_spins = withhold ? spin_limit : 0;
  g_err[0] = '\0';
  return NVFP4_OK;
}

}  // extern "C"

// ---- the library's own workspace, for mlp_forward_noalloc -----------------
//
// One static device array per GPU (each device that loads the library holds
// its own copy until the process ends). Host code never passes the array's
// name to a kernel or copy: in host code it stands for no device address.
// The address comes from hipGetSymbolAddress, once per device with that
// device current, and is kept per device.
static __device__ __align__(256) uint8_t scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

__global__ void k_clear_words(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// The scratch address on the current device; on its first use there, the
// tail (decode records and status word) is cleared on `s` by a fill kernel
// (stream-ordered before the caller's work; no memset, so a capturing
// caller records a kernel node). nullptr (with the message set) on failure.
static uint8_t* scratch_on_current_device(hipStream_t s) {
  static std::mutex mu;
  static uint8_t* ptr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    fail(NVFP4_ERR_HIP, "hipGetDevice failed or device index out of range");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      fail(NVFP4_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return nullptr;
    }
    // The tail of the scratch (the same size for every shape).
    uint32_t* t = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(p) + NVFP4_NOALLOC_SCRATCH_BYTES - kTailBytes);
    k_clear_words<<<256, 256, 0, s>>>(t, (int64_t)(kTailBytes / 4));
    const hipError_t le = hipGetLastError();
    if (le != hipSuccess) {
      fail(NVFP4_ERR_HIP, "scratch clear launch: %s", hipGetErrorString(le));
      return nullptr;
    }
    ptr[dev] = static_cast<uint8_t*>(p);
  }
  return ptr[dev];
}

// The MLP forward of every mode; s_gu / s_d are the AWQ pre-quant scales of
// NVFP4_MODE_W4A16_AWQ (null otherwise). With use_scratch, ws and ws_bytes
// are ignored and the library's scratch array serves as the workspace.
static int mlp_forward_impl(int mode, const uint16_t* x, int64_t M, int64_t H, int64_t I, const void* w_gu_packed,
                            const float* alpha_gu, const void* w_d_packed, const float* alpha_d,
                            const float* g1_inv, const float* g2_inv, const uint16_t* s_gu, const uint16_t* s_d,
                            void* ws, size_t ws_bytes, void* out, int out_dtype, void* stream,
                            bool use_scratch = false) {
  if (mode != NVFP4_MODE_W4A4 && mode != NVFP4_MODE_W4A16 && mode != NVFP4_MODE_W4A4_DYN &&
      mode != NVFP4_MODE_W4A16_AWQ)
    return fail(NVFP4_ERR_INVALID_ARG, "unsupported quant mode %d", mode);
  if (!dim_ok(M) || !dim_ok(H) || !dim_ok(I)) return fail(NVFP4_ERR_INVALID_ARG, "dimension out of range");
  if (H <= 0 || H % 256 != 0 || I <= 0 || I % 256 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "H and I must be positive multiples of 256 (H=%lld I=%lld)",
                (long long)H, (long long)I);
  if (out_dtype != NVFP4_DTYPE_F32 && out_dtype != NVFP4_DTYPE_BF16)
    return fail(NVFP4_ERR_INVALID_ARG, "out_dtype must be F32 or BF16");
  if ((mode == NVFP4_MODE_W4A16 || mode == NVFP4_MODE_W4A16_AWQ) && (g1_inv || g2_inv))
    return fail(NVFP4_ERR_INVALID_ARG, "W4A16 takes no activation scales: g1_inv and g2_inv must be NULL");
  if (mode == NVFP4_MODE_W4A16_AWQ && M > 0 && (!s_gu || !s_d || !aligned16(s_gu) || !aligned16(s_d)))
    return fail(NVFP4_ERR_INVALID_ARG, "W4A16_AWQ needs 16-byte aligned pre-quant scales s_gu [H] and s_d [I]");
  if (M == 0) { g_err[0] = '\0'; return NVFP4_OK; }
  if (!x || !w_gu_packed || !alpha_gu || !w_d_packed || !alpha_d || !out || (!ws && !use_scratch))
    return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
  if (mode == NVFP4_MODE_W4A4 && (!g1_inv || !g2_inv))
    return fail(NVFP4_ERR_INVALID_ARG, "W4A4 needs g1_inv and g2_inv");
  if (mode == NVFP4_MODE_W4A4_DYN && (g1_inv || !g2_inv))
    return fail(NVFP4_ERR_INVALID_ARG, "W4A4_DYN computes x's scales per token: g1_inv must be NULL, g2_inv set");
  if (!aligned16(x) || !aligned16(w_gu_packed) || !aligned16(w_d_packed) || !aligned16(out) ||
      (!use_scratch && !aligned16(ws)))
    return fail(NVFP4_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
  if (use_scratch) {
    const int kmode = (mode == NVFP4_MODE_W4A16 || mode == NVFP4_MODE_W4A16_AWQ) ? NVFP4_MODE_W4A16 : NVFP4_MODE_W4A4;
    const size_t need = mlp_path_bytes(mode, M, H, I, choose_path(kmode, M, true), choose_path_down(kmode, M, H, I));
    if (need > NVFP4_NOALLOC_SCRATCH_BYTES)
      return fail(NVFP4_ERR_INVALID_ARG,
                  "mlp_forward_noalloc: M=%lld H=%lld I=%lld needs %zu bytes of workspace, more than the %zu of the "
                  "library's scratch (use mlp_forward with a workspace)",
                  (long long)M, (long long)H, (long long)I, need, (size_t)NVFP4_NOALLOC_SCRATCH_BYTES);
    ws_bytes = NVFP4_NOALLOC_SCRATCH_BYTES;
  } else {
    const size_t need = mlp_workspace_bytes(mode, M, H, I);
    if (ws_bytes < need)
      return fail(NVFP4_ERR_INVALID_ARG, "workspace %zu bytes < %zu needed", ws_bytes, need);
  }
  int st = check_device();
  if (st) return st;
  hipStream_t s = as_stream(stream);
  if (use_scratch) {
    ws = scratch_on_current_device(s);
    if (!ws) return NVFP4_ERR_HIP;
  }
  const int ws_mode = mode;
  const bool dyn = mode == NVFP4_MODE_W4A4_DYN;
  if (dyn) mode = NVFP4_MODE_W4A4;  // the W4A4 kernels, x quantized per token
  if (mode == NVFP4_MODE_W4A16_AWQ) mode = NVFP4_MODE_W4A16;  // the W4A16 kernels on pre-scaled inputs
  const int path = choose_path(mode, M, true);  // the gate_up GEMM's (and decode checks')
  const int path_d = choose_path_down(mode, M, H, I);
  const int epi_out = out_dtype == NVFP4_DTYPE_F32 ? nvfp4::kOutF32 : nvfp4::kOutBF16;
  uint8_t* base = static_cast<uint8_t*>(ws);
  const size_t m = static_cast<size_t>(M);

  // Split-K (partials, then the counters of the down projection, then those
  // of the gate_up GEMM, after the activations). The gate_up's first launch
  // clears both counter sets before it runs (a split gate_up runs its whole
  // rounds first and its K-split tail tiles in a second launch); every split
  // GEMM also leaves its counters at zero.
  const Kernel k_gu = mlp_kernel(path, mode, M, 2 * I, H);
  const Kernel k_d = mlp_kernel(path_d, mode, M, H, I);
  SplitPlan sp = split_plan(k_d, mode, M, H, I, false);
  SplitPlan sg = split_plan(k_gu, mode, M, 2 * I, H, true);
  if (!clears_counters(k_gu)) sp = sg = SplitPlan{};
  uint8_t* split_base = base + mlp_act_bytes(ws_mode, m, H, I);
  float* part = reinterpret_cast<float*>(split_base);
  uint32_t* counters = reinterpret_cast<uint32_t*>(split_base + std::max(sp.part_bytes, sg.part_bytes));
  uint32_t* counters_gu = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(counters) + sp.counter_bytes);
  auto with_split = [&](nvfp4::GemmArgs& gu, nvfp4::GemmArgs& dn) {
    if (sp.ways > 1 || sg.ways > 1) {
      gu.zero_ptr = counters;
      gu.zero_n = (int)((sp.counter_bytes + sg.counter_bytes) / sizeof(uint32_t));
    }
    if (sp.ways > 1) {
      dn.part = part;
      dn.counters = counters;
      dn.ksplit = sp.ways;
    }
    if (sg.ways > 1) {
      gu.part = part;
      gu.counters = counters_gu;
      gu.ksplit = sg.ways;
    }
  };

  hipError_t e;
  if (mode == NVFP4_MODE_W4A4) {
    uint8_t* xq = base;
    uint8_t* xs = xq + align256(m * H / 2);
    uint8_t* hq = xs + align256(m * H / 16);
    uint8_t* hs = hq + align256(m * I / 2);
    if (dyn) {
      float* row_g = reinterpret_cast<float*>(hs + align256(m * I / 16));
      e = nvfp4::launch_quantize_per_token(x, false, M, H, xq, xs, row_g, s);
      if (e != hipSuccess) return hip_status(e, "mlp_forward quantize_per_token");
      nvfp4::GemmArgs g1{xq, xs, static_cast<const uint8_t*>(w_gu_packed), M, 2 * I, H, alpha_gu, g2_inv, hq, hs};
      g1.row_scale = row_g;
      nvfp4::GemmArgs g2{hq, hs, static_cast<const uint8_t*>(w_d_packed), M, H, I, alpha_d, nullptr, out, nullptr};
      with_split(g1, g2);
      e = run_gemm(path, NVFP4_MODE_W4A4, nvfp4::kSwigluNvfp4, g1, s);
      if (e != hipSuccess) return hip_status(e, "mlp_forward gate_up");
      return hip_status(run_gemm(path_d, NVFP4_MODE_W4A4, epi_out, g2, s), "mlp_forward down");
    }
    // One token under the automatic path: the whole forward in one launch
    // (x quantized as it is staged, h handed from the gate_up workgroups to
    // the down workgroups as epoch-tagged records in the workspace).
    if (M == 1 && g_path == NVFP4_PATH_AUTO && decode_in_tail(H, I) && !stream_capturing(s)) {
      nvfp4::DecodeArgs d{x, g1_inv, static_cast<const uint8_t*>(w_gu_packed), static_cast<const uint8_t*>(w_d_packed),
                          alpha_gu, alpha_d, g2_inv, hq, hs, out, tail_records(ws, ws_bytes, decode_bytes(H, I)),
                          H, I, nvfp4::decode_splits(H, I), next_epoch(), tail_status(ws, ws_bytes),
                          nvfp4::kDecodeSpinLimit, 0u};
      if (g_decode_test_spins > 0) {
        // Test hook: producers tag with the epoch's top bit flipped, a tag
        // the epoch counter reaches only 2^31 launches later.
        d.spin_limit = g_decode_test_spins;
        d.tag_skew = 0x80000000u;
      }
      return hip_status(nvfp4::launch_decode_mlp(epi_out, d, s), "mlp_forward decode");
    }
    // At M = 1 the decode GEMV quantizes x itself as it stages it (no
    // separate launch); otherwise x is quantized by launch_quantize (with two
    // token rows per workgroup the fused variant needs more registers than
    // keep its grid resident: measured 35.5 against 26.5 + 4.8 us).
    const bool fused_quant = k_gu == kFp4Gemv && M == 1;
    if (!fused_quant) {
      e = nvfp4::launch_quantize(x, false, M, H, g1_inv, xq, xs, s);
      if (e != hipSuccess) return hip_status(e, "mlp_forward quantize");
    }
    nvfp4::GemmArgs g1{xq, xs, static_cast<const uint8_t*>(w_gu_packed), M, 2 * I, H, alpha_gu, g2_inv, hq, hs};
    if (fused_quant) {
      g1.a = x;
      g1.a_scales = nullptr;
      g1.a_g_inv = g1_inv;
    }
    nvfp4::GemmArgs g2{hq, hs, static_cast<const uint8_t*>(w_d_packed), M, H, I, alpha_d, nullptr, out, nullptr};
    with_split(g1, g2);
    e = run_gemm(path, NVFP4_MODE_W4A4, nvfp4::kSwigluNvfp4, g1, s);
    if (e != hipSuccess) return hip_status(e, "mlp_forward gate_up");
    e = run_gemm(path_d, NVFP4_MODE_W4A4, epi_out, g2, s);
    return hip_status(e, "mlp_forward down");
  }
  uint8_t* hb = base;
  // One token under the automatic path (plain W4A16, outside stream
  // capture): the whole forward in one launch, the bf16 h handed from the
  // gate_up workgroups to the down workgroups as tagged records.
  if (M == 1 && !s_gu && g_path == NVFP4_PATH_AUTO && decode16_in_tail(H, I) && !stream_capturing(s)) {
    nvfp4::Decode16Args d{x, static_cast<const uint8_t*>(w_gu_packed), static_cast<const uint8_t*>(w_d_packed),
                          alpha_gu, alpha_d, reinterpret_cast<uint16_t*>(hb), out,
                          tail_records(ws, ws_bytes, decode16_bytes(H, I)), H, I, nvfp4::decode16_splits(H, I),
                          next_epoch(), tail_status(ws, ws_bytes), nvfp4::kDecodeSpinLimit, 0u};
    if (g_decode_test_spins > 0) {
      d.spin_limit = g_decode_test_spins;
      d.tag_skew = 0x80000000u;
    }
    return hip_status(nvfp4::launch_decode_mlp16(epi_out, d, s), "mlp_forward decode (W4A16)");
  }
  const void* xin = x;
  if (s_gu) {
    // AWQ: x' = bf16(x * s_gu) into the workspace; h gets s_d in the gate_up
    // epilogue.
    uint8_t* xs = base + align256(m * I * 2);
    e = nvfp4::launch_prescale_bf16(x, s_gu, M, H, xs, s);
    if (e != hipSuccess) return hip_status(e, "mlp_forward prescale");
    xin = xs;
  }
  nvfp4::GemmArgs g1{xin, nullptr, static_cast<const uint8_t*>(w_gu_packed), M, 2 * I, H, alpha_gu, nullptr, hb, nullptr};
  g1.h_prescale = s_d;
  nvfp4::GemmArgs g2{hb, nullptr, static_cast<const uint8_t*>(w_d_packed), M, H, I, alpha_d, nullptr, out, nullptr};
  with_split(g1, g2);
  e = run_gemm(path, NVFP4_MODE_W4A16, nvfp4::kSwigluBF16, g1, s);
  if (e != hipSuccess) return hip_status(e, "mlp_forward gate_up");
  e = run_gemm(path_d, NVFP4_MODE_W4A16, epi_out, g2, s);
  return hip_status(e, "mlp_forward down");
}

extern "C" {

int mlp_forward(int mode, const uint16_t* x, int64_t M, int64_t H, int64_t I, const void* w_gu_packed,
                const float* alpha_gu, const void* w_d_packed, const float* alpha_d, const float* g1_inv,
                const float* g2_inv, void* ws, size_t ws_bytes, void* out, int out_dtype, void* stream) {
  if (mode == NVFP4_MODE_W4A16_AWQ)
    return fail(NVFP4_ERR_INVALID_ARG, "W4A16_AWQ takes its pre-quant scales: call mlp_forward_w4a16_awq");
  return mlp_forward_impl(mode, x, M, H, I, w_gu_packed, alpha_gu, w_d_packed, alpha_d, g1_inv, g2_inv, nullptr,
                          nullptr, ws, ws_bytes, out, out_dtype, stream);
}

int mlp_forward_noalloc(int mode, const uint16_t* x, int64_t M, int64_t H, int64_t I, const void* w_gu_packed,
                        const float* alpha_gu, const void* w_d_packed, const float* alpha_d, const float* g1_inv,
                        const float* g2_inv, void* out, int out_dtype, void* stream) {
  if (mode == NVFP4_MODE_W4A16_AWQ)
    return fail(NVFP4_ERR_INVALID_ARG, "W4A16_AWQ takes its pre-quant scales: call mlp_forward_w4a16_awq");
  return mlp_forward_impl(mode, x, M, H, I, w_gu_packed, alpha_gu, w_d_packed, alpha_d, g1_inv, g2_inv, nullptr,
                          nullptr, nullptr, 0, out, out_dtype, stream, true);
}

int mlp_forward_w4a16_awq(const uint16_t* x, int64_t M, int64_t H, int64_t I, const void* w_gu_packed,
                          const float* g_gu, const uint16_t* s_gu, const void* w_d_packed, const float* g_d,
                          const uint16_t* s_d, void* ws, size_t ws_bytes, void* out, int out_dtype, void* stream) {
  return mlp_forward_impl(NVFP4_MODE_W4A16_AWQ, x, M, H, I, w_gu_packed, g_gu, w_d_packed, g_d, nullptr, nullptr,
                          s_gu, s_d, ws, ws_bytes, out, out_dtype, stream);
}

int nvfp4_grouped_gemm(int mode, const void* a, const uint8_t* a_scales, const void* w_packed, int64_t E,
                       int64_t M, int64_t N, int64_t K, const int32_t* masked_m, const float* alpha, void* out,
                       int out_dtype, void* stream) {
  if (E < 0 || E > 65535) return fail(NVFP4_ERR_INVALID_ARG, "expert count %lld not in [0, 65535]", (long long)E);
  int st = check_gemm(mode, a, a_scales, w_packed, E == 0 ? 0 : M, N, K, alpha, out);
  if (st) return st;
  if (out_dtype != NVFP4_DTYPE_F32 && out_dtype != NVFP4_DTYPE_BF16)
    return fail(NVFP4_ERR_INVALID_ARG, "out_dtype must be F32 or BF16");
  if (reinterpret_cast<uintptr_t>(masked_m) % 4) return fail(NVFP4_ERR_INVALID_ARG, "masked_m must be 4-byte aligned");
  if (M == 0 || E == 0) { g_err[0] = '\0'; return NVFP4_OK; }
  const size_t wbytes = nvfp4_repack_bytes(NVFP4_REPACK_PLAIN, N, K);
  nvfp4::GemmArgs probe{};
  probe.M = M;
  probe.N = N;
  probe.K = K;
  if (!fits_buffers(probe, mode))
    return fail(NVFP4_ERR_UNSUPPORTED, "grouped GEMM needs each expert's operands below 2^31 bytes");
  st = check_device();
  if (st) return st;
  const int epi = out_dtype == NVFP4_DTYPE_F32 ? nvfp4::kOutF32 : nvfp4::kOutBF16;
  const size_t out_row = (size_t)N * (out_dtype == NVFP4_DTYPE_F32 ? 4 : 2);
  const size_t a_row = mode == NVFP4_MODE_W4A4 ? (size_t)K / 2 : (size_t)K * 2;
  hipStream_t sm = as_stream(stream);
  // Every expert in one launch (grid z of the weight-streaming kernel, grid
  // y of the tiled ones), each workgroup reading its expert's valid row
  // count from masked_m: an expert's GEMM alone is too narrow to fill the
  // CUs (4096 rows: 128 streaming workgroups, 16 x (M / 256) tiled ones).
  // W4A4 from kGroupedMidMinM to kGroupedMidMaxM tokens per expert on the
  // mid-size kernel (always under its override; 8 experts of 4096 x 7168:
  // 47 / 68 / 121 / 127 / 175 us at 64 / 128 / 256 / 384 / 512 tokens
  // against 53 / 84 / 128 / 171 / 228 streaming and 185 tiled at 512);
  // otherwise the weight-streaming kernel up to kGroupedStreamMaxM tokens
  // per expert (under the automatic path; always under the stream or GEMV
  // override), the tiled kernel above (always under the tiled override).
  const int p = g_path;
  const bool mid = mode == NVFP4_MODE_W4A4 &&
                   (p == NVFP4_PATH_AUTO ? M >= kGroupedMidMinM && M <= kGroupedMidMaxM : p == NVFP4_PATH_MID);
  const bool streaming =
      !mid && (p == NVFP4_PATH_AUTO ? M <= kGroupedStreamMaxM : (p != NVFP4_PATH_TILED && p != NVFP4_PATH_TILED64));
  nvfp4::GemmArgs g{a, a_scales, static_cast<const uint8_t*>(w_packed), M, N, K, alpha, nullptr, out, nullptr};
  g.m_dev = masked_m;
  if (E > 1) {
    g.experts = (int)E;
    g.e_a = (int64_t)(M * a_row);
    g.e_as = a_scales ? M * (K / 16) : 0;
    g.e_w = (int64_t)wbytes;
    g.e_out = (int64_t)(M * out_row);
  }
  hipError_t err = mid         ? nvfp4::launch_mid_gemm(mode, epi, g, sm)
                   : streaming ? nvfp4::launch_stream_gemm(mode, epi, g, sm)
                   : mode == NVFP4_MODE_W4A4 ? nvfp4::launch_tiled2_gemm(epi, g, sm)
                                             : nvfp4::launch_tiled16_gemm(epi, g, sm);
  if (err != hipSuccess) return hip_status(err, "grouped_gemm launch");
  g_err[0] = '\0';
  return NVFP4_OK;
}

int nvfp4_prescale_bf16(const void* x, const void* s, int64_t M, int64_t K, void* out, void* stream) {
  if (!dim_ok(M) || K < 0 || K > (int64_t(1) << 30) || K % 8 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "need 0 <= M <= 2^24 and 0 <= K <= 2^30 a multiple of 8 (M=%lld K=%lld)", (long long)M,
                (long long)K);
  if (M * K == 0) { g_err[0] = '\0'; return NVFP4_OK; }
  if (!x || !s || !out) return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(x) || !aligned16(s) || !aligned16(out))
    return fail(NVFP4_ERR_INVALID_ARG, "x, s and out must be 16-byte aligned");
  int st = check_device();
  if (st) return st;
  return hip_status(nvfp4::launch_prescale_bf16(x, s, M, K, out, as_stream(stream)), "prescale launch");
}

}  // extern "C"
