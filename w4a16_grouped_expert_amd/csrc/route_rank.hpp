// Order of the router's top-k selection: by logit descending, ties to the lower
// expert index (ExactMoE, page "Every Expert Counts: ExactMoE for
// Memory-Efficient W4A16 Inference", Abstract: the top-k routing procedure is
// unchanged), and the rank of a logit in that order.
#pragma once

#include "common.hpp"

namespace moe {

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Number of the token's E logits (row, in LDS) that beat (v, e): 16 broadcast
// reads are issued before their compares, so the LDS latency is paid once per 16.
__device__ __forceinline__ int rank_in_row(const float* row, int E, float v, int e) {
  int rank = 0, o = 0;
  for (; o + 16 <= E; o += 16) {
    float r[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) r[u] = row[o + u];
#pragma unroll
    for (int u = 0; u < 16; ++u) rank += better(r[u], o + u, v, e) ? 1 : 0;
  }
  for (; o < E; ++o) rank += better(row[o], o, v, e) ? 1 : 0;
  return rank;
}

}  // namespace moe
