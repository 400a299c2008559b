// moe_align: expert-sorted permutation of the T*k (token, slot) pairs (ExactMoE,
// page "Every Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference",
// Abstract): a stable counting sort, by one workgroup (align_block in
// align_block.hpp) or, from kAlignChunkedFrom pairs on, by one workgroup per chunk.
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

// Many pairs: workgroup b places the pairs of chunk b (chunks of `chunk` pairs, a
// multiple of kAlignChunk, in pair order), so the scattered stores are spread over
// many CUs; at most kAlignMaxChunks workgroups, so that the counting below, which
// every workgroup repeats, stays within a small multiple of the pairs.  Every
// workgroup first counts all pairs per expert, and those before its chunk (LDS
// atomics into its wavefront's own row), so it knows the offsets and its chunk's
// base per expert without a second launch; workgroup 0 publishes the offsets and
// the work list.  Inside the chunk the placement is align_block's: wavefront
// sub-chunks in pair order, ranks in lane order, so the order is the stable one.
constexpr int kAlignChunk = 2048;
static_assert(kAlignChunk % (kAlignWaves * 64) == 0, "whole batches per wavefront");
constexpr int kAlignChunkedFrom = 4096;  // pairs
constexpr int kAlignMaxChunks = 64;

__global__ __launch_bounds__(kAlignThreads) void k_align_chunks(const int32_t* __restrict__ ids, int P, int E,
                                                                int block_m, int id_bits,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted_pairs,
                                                                int32_t* __restrict__ pair_pos,
                                                                int32_t* __restrict__ active,
                                                                int32_t* __restrict__ tile_offsets, int chunk) {
  __shared__ int s_off[MOE_MAX_EXPERTS];
  __shared__ int s_bef[MOE_MAX_EXPERTS];
  __shared__ int s_wcnt[kAlignWaves][MOE_MAX_EXPERTS];
  __shared__ int s_wbef[kAlignWaves][MOE_MAX_EXPERTS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = (int)min<int64_t>(P, (int64_t)blockIdx.x * chunk), c1 = min(P, c0 + chunk);
  // the wavefront's sub-chunk of this chunk (whole batches of 64, in pair order), in
  // super-batches of kSubB batches; the first one is requested right away
  constexpr int kSubB = kAlignChunk / kAlignWaves / 64;
  constexpr int kSuper = 64 * kSubB;
  const int sub = ((c1 - c0 + kAlignWaves - 1) / kAlignWaves + 63) / 64 * 64;
  const int s0 = min(c1, c0 + wave * sub), s1 = min(c1, s0 + sub);
  const int n_super = (s1 - s0 + kSuper - 1) / kSuper;
  int es[kSubB];
  auto load_super = [&](int sb) {
#pragma unroll
    for (int i = 0; i < kSubB; ++i) {
      const int p = s0 + sb * kSuper + 64 * i + lane;
      es[i] = p < s1 ? ids[p] : -1;
    }
  };
  load_super(0);
  for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) {
    s_wcnt[i / E][i % E] = 0;
    s_wbef[i / E][i % E] = 0;
  }
  __syncthreads();
  // every pair: per-expert totals, and the pairs before this chunk (c0 is a multiple
  // of 64, so a batch of 64 lies wholly before it or not)
  constexpr int kU = 32;  // ids per lane in flight at once (32768 pairs per pass of the workgroup)
  for (int b0 = wave * 64; b0 < P; b0 += kAlignThreads * kU) {
    int ev[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int p = b0 + kAlignThreads * u + lane;
      ev[u] = p < P ? ids[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int b = b0 + kAlignThreads * u;
      if (b >= P) break;
      if (ev[u] >= 0 && ev[u] < E) {  // (lanes past P hold -1)
        atomicAdd(&s_wcnt[wave][ev[u]], 1);
        if (b + 64 <= c0) atomicAdd(&s_wbef[wave][ev[u]], 1);
      }
    }
  }
  __syncthreads();
  int tot = 0;
  if (tid < E) {  // (E <= kAlignThreads)
    int bef = 0;
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) {
      tot += s_wcnt[w][tid];
      bef += s_wbef[w][tid];
    }
    s_bef[tid] = bef;
  }
  __syncthreads();
  for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) s_wcnt[i / E][i % E] = 0;  // reused below
  align_scan(tot, E, block_m, tid, lane, wave, s_off, offsets, active, tile_offsets, blockIdx.x == 0);
  __syncthreads();
  // this chunk: the wavefront's sub-chunk
  for (int sb = 0; sb < n_super; ++sb) {
    if (sb > 0) load_super(sb);
#pragma unroll
    for (int i = 0; i < kSubB; ++i) {
      if (es[i] >= 0 && es[i] < E) atomicAdd(&s_wcnt[wave][es[i]], 1);  // (lanes past s1 hold -1)
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kAlignThreads) {
    int base = s_off[e] + s_bef[e];
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) {
      const int n = s_wcnt[w][e];
      s_wcnt[w][e] = base;
      base += n;
    }
  }
  __syncthreads();
  for (int sb = 0; sb < n_super; ++sb) {
    if (n_super > 1) load_super(sb);  // (one super-batch: still in registers)
#pragma unroll
    for (int i = 0; i < kSubB; ++i) {
      const int b = s0 + sb * kSuper + 64 * i;
      if (b >= s1) break;
      const int p = b + lane;
      const bool valid = p < s1 && es[i] >= 0 && es[i] < E;
      const int e = valid ? es[i] : 0;
      if (p < s1 && !valid) pair_pos[p] = -1;
      const LaneGroup lg = lane_group(e, valid, id_bits, lane);
      // every lane reads its base before the group leader advances it
      const int q = valid ? s_wcnt[wave][e] + lg.rank : 0;
      __builtin_amdgcn_wave_barrier();
      if (valid && lg.rank == 0) s_wcnt[wave][e] = q + lg.cnt;
      __builtin_amdgcn_wave_barrier();
      if (valid) {
        sorted_pairs[q] = p;
        pair_pos[p] = q;
      }
    }
  }
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
  const int P = T * k;
  if (P >= kAlignChunkedFrom) {
    const int chunk = (int)(ceil_div(ceil_div(P, kAlignMaxChunks), kAlignChunk) * kAlignChunk);
    hipLaunchKernelGGL(k_align_chunks, dim3((unsigned)ceil_div(P, chunk)), dim3(kAlignThreads), 0, s, topk_ids, P, E,
                       block_m, bits, expert_offsets, sorted_pairs, pair_pos, active_experts,
                       block_m > 0 ? tile_offsets : nullptr, chunk);
  }
  else
    hipLaunchKernelGGL(k_align, dim3(1), dim3(kAlignThreads), 0, s, topk_ids, P, E, block_m, bits, expert_offsets,
                       sorted_pairs, pair_pos, active_experts, block_m > 0 ? tile_offsets : nullptr);
  timing_end(K_ALIGN, s);
  return check_launch("moe_align");
}
