// The expert-sorted permutation of the T*k (token, slot) pairs, the grouping that
// lets all selected experts run in one fused grouped pass (ExactMoE, page "Every
// Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference", Abstract).  A
// stable counting sort in one 1024-thread workgroup:
//
//  1. histogram of expert ids (LDS atomics; the counts do not depend on order);
//  2. one block-wide scan gives the offsets, the compacted work list of active
//     experts ({id, first position, count} each) and the per-expert tile counts;
//  3. placement, 1024 pairs per pass in pair order: inside a wavefront the lanes
//     that carry the same expert are found with ballots over the id bits, their
//     rank is a popcount of the lower lanes; the per-wave counts are exchanged in
//     LDS so each wavefront adds the counts of the earlier wavefronts of the pass
//     and of the earlier passes.  Every pair lands at the unique stable position.
//
// Shared by moe_align (its own kernel) and moe_route_align (the last workgroup of
// the router kernel).
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

// The whole permutation, run by one workgroup of kAlignThreads threads.
__device__ __forceinline__ void align_block(const int32_t* __restrict__ ids, int P, int E, int block_m, int id_bits,
                                            int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
                                            int32_t* __restrict__ pair_pos, int32_t* __restrict__ active,
                                            int32_t* __restrict__ tile_offsets) {
  __shared__ int s_count[MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS];
  __shared__ uint16_t s_wcnt[kAlignWaves][MOE_MAX_EXPERTS];
  __shared__ int s_tot[3][kAlignWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kAlignThreads) {
    s_count[e] = 0;
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) s_wcnt[w][e] = 0;
  }
  __syncthreads();
  for (int p = tid; p < P; p += kAlignThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&s_count[e], 1);
  }
  __syncthreads();

  // block scan over experts (E <= 1024: one expert per thread)
  const int c = tid < E ? s_count[tid] : 0;
  const int a = c > 0 ? 1 : 0;
  const int tl = (block_m > 0) ? (c + block_m - 1) / block_m : 0;
  int ic = wave_incl_scan(c, lane), ia = wave_incl_scan(a, lane), it = wave_incl_scan(tl, lane);
  if (lane == 63) {
    s_tot[0][wave] = ic;
    s_tot[1][wave] = ia;
    s_tot[2][wave] = it;
  }
  __syncthreads();
  int bc = 0, ba = 0, bt = 0;
  for (int w = 0; w < wave; ++w) {
    bc += s_tot[0][w];
    ba += s_tot[1][w];
    bt += s_tot[2][w];
  }
  const int ex_c = bc + ic - c, ex_a = ba + ia - a, ex_t = bt + it - tl;
  if (tid < E) {
    s_off[tid] = ex_c;
    offsets[tid] = ex_c;
    if (a) {
      // work item of the active expert: {id, first sorted position, pair count, 0}
      const i32x4_t item = {tid, ex_c, c, 0};
      *reinterpret_cast<i32x4_t*>(active + 4 + 4 * ex_a) = item;
    }
    if (tile_offsets) tile_offsets[tid] = ex_t;
  }
  if (tid == E - 1) {
    offsets[E] = ex_c + c;
    const i32x4_t head = {ex_a + a, 0, 0, 0};
    *reinterpret_cast<i32x4_t*>(active) = head;
    if (tile_offsets) tile_offsets[E] = ex_t + tl;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kAlignThreads) s_count[e] = 0;  // now: pairs placed so far
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < P; base += kAlignThreads) {
    const int p = base + tid;
    const int e_in = p < P ? ids[p] : 0;
    const bool valid = p < P && e_in >= 0 && e_in < E;   // out-of-range ids are dropped
    const int e = valid ? e_in : 0;
    if (p < P && !valid) pair_pos[p] = -1;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(valid && bit);
      m &= bit ? bb : ~bb;
    }
    const int rank = __popcll(m & lt_mask);
    const int cnt = __popcll(m);
    if (valid && rank == 0) s_wcnt[wave][e] = (uint16_t)cnt;
    __syncthreads();
    if (valid) {
      int before = s_count[e];
      for (int w = 0; w < wave; ++w) before += s_wcnt[w][e];
      const int q = s_off[e] + before + rank;
      sorted_pairs[q] = p;
      pair_pos[p] = q;
    }
    __syncthreads();
    if (valid && rank == 0) {
      atomicAdd(&s_count[e], cnt);
      s_wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

}  // namespace moe
