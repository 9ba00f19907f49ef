// stream_nt1.hip -- the one-token-group instantiations of the
// weight-streaming kernel (stream_kernel.h): W4A4 up to 16 tokens, W4A16 at
// any count (token groups along the grid's y dimension). A translation unit
// of its own so that it can be scheduled differently from the 2-4
// token-group kernels (build.py).
#include "stream_kernel.h"

namespace nvfp4 {

template <int MODE>
static hipError_t nt1_mode(int epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case kOutF32: return launch_nt<MODE, kOutF32, 1>(a, s);
    case kOutBF16: return launch_nt<MODE, kOutBF16, 1>(a, s);
    case kSwigluBF16: return launch_nt<MODE, kSwigluBF16, 1>(a, s);
    case kSwigluF32: return launch_nt<MODE, kSwigluF32, 1>(a, s);
    case kSwigluNvfp4:
      if constexpr (MODE == kW4A4) return launch_nt<MODE, kSwigluNvfp4, 1>(a, s);
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_stream_nt1(int mode, int epi, const GemmArgs& a, hipStream_t s) {
  return mode == kW4A4 ? nt1_mode<kW4A4>(epi, a, s) : nt1_mode<kW4A16>(epi, a, s);
}

}  // namespace nvfp4
