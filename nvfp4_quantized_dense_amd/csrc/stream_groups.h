// stream_groups.h -- packed row groups (16 weight rows each) per workgroup of
// the weight-streaming kernel at one token group (M <= 16).
//
// SwiGLU epilogues take one gate/up pair (2 groups). Dense epilogues take 2
// groups where N / 16 is even: each activation slice then serves two weight
// tiles (MLP forward at 16 tokens: W4A4 hidden 7168 62.4 -> 59.1 us, W4A16
// hidden 5120 69.8 -> 65.8 us; 4 groups, or 2 gate/up pairs, were slower).
#pragma once
#include <stdint.h>

namespace nvfp4 {

inline int stream_groups(bool swiglu, int64_t M, int64_t N) {
  (void)M;
  if (swiglu) return 2;
  return (N / 16) % 2 == 0 ? 2 : 1;
}

}  // namespace nvfp4
