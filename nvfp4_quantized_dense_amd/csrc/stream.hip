// stream.hip -- launches of the weight-streaming kernel (stream_kernel.h):
// the 2-4 token-group instantiations here, one token group in
// stream_nt1.hip.
#include "stream_kernel.h"

namespace nvfp4 {

TileShape stream_shape(int mode, int64_t M, int64_t N) {
  int64_t groups = (M + 15) / 16;
  const int64_t nt = groups < 4 ? groups : 4;
  const int64_t g = nt == 1 ? stream_groups(mode, false, M, N) : 1;
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
  if (a.M <= 16) return launch_stream_nt1(mode, epi, a, s);
  if (mode == kW4A4) {
    switch (epi) {
      case kOutF32: return launch_mode_epi<kW4A4, kOutF32>(a, s);
      case kOutBF16: return launch_mode_epi<kW4A4, kOutBF16>(a, s);
      case kSwigluNvfp4: return launch_mode_epi<kW4A4, kSwigluNvfp4>(a, s);
      case kSwigluBF16: return launch_mode_epi<kW4A4, kSwigluBF16>(a, s);
      case kSwigluF32: return launch_mode_epi<kW4A4, kSwigluF32>(a, s);
    }
  } else {
    switch (epi) {
      case kOutF32: return launch_mode_epi<kW4A16, kOutF32>(a, s);
      case kOutBF16: return launch_mode_epi<kW4A16, kOutBF16>(a, s);
      case kSwigluBF16: return launch_mode_epi<kW4A16, kSwigluBF16>(a, s);
      case kSwigluF32: return launch_mode_epi<kW4A16, kSwigluF32>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
