// moe_align: expert-sorted permutation of the T*k (token, slot) pairs (ExactMoE,
// page "Every Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference",
// Abstract); the algorithm is align_block in align_block.hpp.
#include "align_block.hpp"

namespace moe {

__global__ __launch_bounds__(kAlignThreads) void k_align(const int32_t* __restrict__ ids, int P, int E, int block_m,
                                                         int id_bits, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ sorted_pairs,
                                                         int32_t* __restrict__ pair_pos,
                                                         int32_t* __restrict__ active,
                                                         int32_t* __restrict__ tile_offsets) {
  align_block(ids, P, E, block_m, id_bits, offsets, sorted_pairs, pair_pos, active, tile_offsets);
}

}  // namespace moe

using namespace moe;

extern "C" int moe_align(const int32_t* topk_ids, int T, int k, int E, int block_m, int32_t* expert_offsets,
                         int32_t* sorted_pairs, int32_t* pair_pos, int32_t* active_experts, int32_t* tile_offsets,
                         void* stream) {
  clear_error();
  MOE_CHECK_ARG(T >= 0 && k > 0 && E > 0 && block_m >= 0, MOE_ERR_INVALID_ARG,
                "moe_align: bad sizes T=%d k=%d E=%d block_m=%d", T, k, E, block_m);
  MOE_CHECK_ARG(E <= MOE_MAX_EXPERTS && k <= MOE_MAX_TOPK && (int64_t)T * k <= (1 << 24),
                MOE_ERR_UNSUPPORTED_SHAPE, "moe_align: unsupported E=%d k=%d T*k=%lld", E, k, (long long)T * k);
  MOE_CHECK_ARG(expert_offsets && active_experts, MOE_ERR_INVALID_ARG, "moe_align: null output pointer");
  MOE_CHECK_ARG(T == 0 || (topk_ids && sorted_pairs && pair_pos), MOE_ERR_INVALID_ARG,
                "moe_align: null pointer");
  MOE_CHECK_ARG(block_m == 0 || tile_offsets, MOE_ERR_INVALID_ARG, "moe_align: block_m > 0 needs tile_offsets");
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  hipStream_t s = (hipStream_t)stream;
  timing_begin(K_ALIGN, s);
  hipLaunchKernelGGL(k_align, dim3(1), dim3(kAlignThreads), 0, s, topk_ids, T * k, E, block_m, bits,
                     expert_offsets, sorted_pairs, pair_pos, active_experts, block_m > 0 ? tile_offsets : nullptr);
  timing_end(K_ALIGN, s);
  return check_launch("moe_align");
}
