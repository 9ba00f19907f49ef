// stream_groups.h -- packed row groups (16 weight rows each) per workgroup of
// the weight-streaming kernel at one token group (M <= 16).
//
// SwiGLU epilogues take whole gate/up pairs (2 or 4 groups), dense ones 1,
// 2 or 4; the count must divide N / 16 (else it halves). More groups let
// each activation slice a workgroup loads serve more weight tiles.
// W4A4 (NVFP4 activations, a slice as many bytes as a weight tile at 16
// tokens): dense 2, SwiGLU 2 (MLP forward at 16 tokens: hidden 7168
// 62.4 -> 59.1 us with dense 2; 4 groups, or 2 gate/up pairs, were slower).
#pragma once
#include <stdint.h>

#include "kernels.h"

namespace nvfp4 {

// W4A16 (bf16 activations: at 16 tokens a slice is 3.6 times the bytes of
// the weight tile it multiplies): SwiGLU 2 pairs above 8 tokens (gate_up at
// 16 tokens, hidden 5120: 39.8 -> 35.5 us), one pair below (at 2 and 4
// tokens two pairs took 28.7 against 24.2 us); dense 4 above 16 tokens,
// where the grid has several token-group rows (down projection at 32
// tokens, intermediate 17408: 42.9 -> 29.7 us), 2 up to 16 (4 took 28.7
// against 23.1 us at 16 tokens and was slower at 2 and 4).
//
// W4A16 dense above 16 tokens with a grid of more than one workgroup per CU
// (256) at 4 groups (a W4A16 workgroup takes one token group, so the grid
// is N / 16 / g x token groups): the fewest of 5, 7 or 8 groups that divide
// N / 16 and fit one round. The down projection at 49-64 tokens, hidden
// 5120 (320 row groups x 4 token groups) runs 256 workgroups of 5 groups
// instead of 320 of 4, of which 64 CUs took two.
inline int stream_groups(int mode, bool swiglu, int64_t M, int64_t N, int64_t experts = 1) {
  int g = mode == kW4A16 && (swiglu ? M > 8 : M > 16) ? 4 : 2;
  while (g > (swiglu ? 2 : 1) && (N / 16) % g != 0) g /= 2;
  if (mode == kW4A16 && !swiglu && M > 16 && experts <= 1) {
    const int64_t rg = N / 16, tg = (M + 15) / 16;
    if (rg / g * tg > 256) {
      for (const int h : {5, 7, 8})
        if (rg % h == 0 && rg / h * tg <= 256) return h;
    }
  }
  return g;
}

}  // namespace nvfp4
