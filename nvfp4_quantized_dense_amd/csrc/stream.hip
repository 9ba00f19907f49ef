// stream.hip -- launches of the weight-streaming kernel (stream_kernel.h):
// the W4A4 2-4 token-group instantiations here, one token group (W4A4 up to
// 16 tokens, W4A16 at any count) in stream_nt1.hip.
#include "stream_kernel.h"

namespace nvfp4 {

// Token groups per workgroup: W4A16 always one (the grid's y dimension
// covers the token groups; its bf16 activation slices and register sets
// at 2-4 groups left 2-3 waves per SIMD: forward at 32 / 64 tokens, hidden
// 5120, 130.6 / 238.9 -> 92.9 / 149.9 us with one). W4A4 up to 4 (one or
// two measured no better over hidden 5120 and 7168 at 24-64 tokens).
static bool stream_one_group(int mode, int64_t M) { return M <= 16 || mode == kW4A16; }

TileShape stream_shape(int mode, int64_t M, int64_t N) {
  int64_t groups = (M + 15) / 16;
  const int64_t nt = stream_one_group(mode, M) ? 1 : (groups < 4 ? groups : 4);
  const int64_t g = nt == 1 ? stream_groups(mode, false, M, N) : ((N / kTileRows) % 2 == 0 ? 2 : 1);
  return TileShape{N / kTileRows / g * ((M + 16 * nt - 1) / (16 * nt)), 256 * nt * g, nt == 1 ? 8 : 4};
}

template <int MODE, int EPI>
static hipError_t launch_mode_epi(const GemmArgs& a, hipStream_t s) {
  const int64_t groups = (a.M + 15) / 16;
  if (groups == 2) return launch_nt<MODE, EPI, 2>(a, s);
  if (groups == 3) return launch_nt<MODE, EPI, 3>(a, s);
  return launch_nt<MODE, EPI, 4>(a, s);
}

// Needs the packed weight and the activations below 2^31 bytes (32-bit
// buffer offsets); the caller checks.
hipError_t launch_stream_gemm(int mode, int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (!splitk_valid(a, epi)) return hipErrorInvalidValue;
  if (a.experts > 1 && (a.ksplit != 1 || a.experts > 65535)) return hipErrorInvalidValue;
  if (stream_one_group(mode, a.M)) return launch_stream_nt1(mode, epi, a, s);
  if (mode != kW4A4) return hipErrorInvalidValue;  // W4A16 runs one token group at every M
  switch (epi) {
    case kOutF32: return launch_mode_epi<kW4A4, kOutF32>(a, s);
    case kOutBF16: return launch_mode_epi<kW4A4, kOutBF16>(a, s);
    case kSwigluNvfp4: return launch_mode_epi<kW4A4, kSwigluNvfp4>(a, s);
    case kSwigluBF16: return launch_mode_epi<kW4A4, kSwigluBF16>(a, s);
    case kSwigluF32: return launch_mode_epi<kW4A4, kSwigluF32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
