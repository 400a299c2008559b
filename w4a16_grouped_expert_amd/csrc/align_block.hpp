// The expert-sorted permutation of the T*k (token, slot) pairs, the grouping that
// lets all selected experts run in one fused grouped pass (ExactMoE, page "Every
// Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference", Abstract).  A
// stable counting sort in one 1024-thread workgroup:
//
//  1. expert counts;
//  2. one block-wide scan gives the offsets, the compacted work list of active
//     experts ({id, first position, count} each) and the per-expert tile counts;
//  3. placement in pair order: inside a wavefront the lanes that carry the same
//     expert are found with ballots over the id bits, their rank is a popcount of
//     the lower lanes; the counts of the earlier wavefronts (and, for more than
//     1024 pairs, of the wavefront's earlier pairs) come from LDS.  Every pair
//     lands at the unique stable position.
// With at most 1024 pairs the per-wavefront counts of step 3 also give step 1;
// with more, each wavefront owns one contiguous chunk and counts it first.
//
// Shared by moe_align (its own kernel) and moe_route_align (the last workgroup of
// the router kernel).
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP moves: shifts by
// 1, 2, 4, 8 inside each 16-lane row (lanes with no source in the row add 0), then
// row 0's total is broadcast into row 1 and row 2's into row 3, and the total of
// rows 0-1 into rows 2-3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Pairs of one wavefront that carry the same expert: ballots over the id bits
// leave the mask of lanes with this lane's expert; the lane's rank is the number
// of such lanes below it.
struct LaneGroup {
  int rank, cnt;
};
__device__ __forceinline__ LaneGroup lane_group(int e, bool valid, int id_bits, int lane) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < id_bits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(valid && bit);
    m &= bit ? bb : ~bb;
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  return LaneGroup{(int)__popcll(m & lt_mask), (int)__popcll(m)};
}

// Block-wide scan over the experts (one per thread, E <= kAlignThreads) of the
// pair counts: offsets, the compacted work list of active experts and the
// per-expert tile counts (written only when publish is set; s_off always).  Every
// thread must call it (it synchronises when E > 64).
__device__ __forceinline__ void align_scan(int c, int E, int block_m, int tid, int lane, int wave,
                                           int32_t* __restrict__ s_off, int32_t* __restrict__ offsets,
                                           int32_t* __restrict__ active, int32_t* __restrict__ tile_offsets,
                                           bool publish = true) {
  __shared__ int s_tot[3][kAlignWaves];
  const int a = c > 0 ? 1 : 0;
  const int tl = (block_m > 0) ? (c + block_m - 1) / block_m : 0;
  const int ic = wave_incl_scan(c), ia = wave_incl_scan(a), it = wave_incl_scan(tl);
  int bc = 0, ba = 0, bt = 0;
  if (E > 64) {
    if (lane == 63) {
      s_tot[0][wave] = ic;
      s_tot[1][wave] = ia;
      s_tot[2][wave] = it;
    }
    __syncthreads();
    for (int w = 0; w < wave; ++w) {
      bc += s_tot[0][w];
      ba += s_tot[1][w];
      bt += s_tot[2][w];
    }
  }
  const int ex_c = bc + ic - c, ex_a = ba + ia - a, ex_t = bt + it - tl;
  if (tid < E) {
    s_off[tid] = ex_c;
  }
  if (publish && tid < E) {
    offsets[tid] = ex_c;
    if (a) {
      // work item of the active expert: {id, first sorted position, pair count, 0}
      const i32x4_t item = {tid, ex_c, c, 0};
      *reinterpret_cast<i32x4_t*>(active + 4 + 4 * ex_a) = item;
    }
    if (tile_offsets) tile_offsets[tid] = ex_t;
  }
  if (publish && tid == E - 1) {
    offsets[E] = ex_c + c;
    const i32x4_t head = {ex_a + a, 0, 0, 0};
    *reinterpret_cast<i32x4_t*>(active) = head;
    if (tile_offsets) tile_offsets[E] = ex_t + tl;
  }
}

// The whole permutation, run by one workgroup of kAlignThreads threads.
// Up to kAlignThreads pairs: one pass.  Every wavefront groups its pairs by
// expert (lane_group) and its group leaders record the per-wavefront counts; the
// expert totals are sums of those, and a pair's position is its expert's offset
// plus the counts of its expert in the earlier wavefronts plus its rank.
// More pairs: each wavefront owns a contiguous chunk of the pairs (chunks in
// pair order); it counts its chunk's experts, one block-wide pass turns the
// counts into every (wavefront, expert) base position, and each wavefront places
// its chunk 64 pairs at a time in order, advancing its own bases.
__device__ __forceinline__ void align_block(const int32_t* __restrict__ ids, int P, int E, int block_m, int id_bits,
                                            int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
                                            int32_t* __restrict__ pair_pos, int32_t* __restrict__ active,
                                            int32_t* __restrict__ tile_offsets) {
  __shared__ int s_off[MOE_MAX_EXPERTS];
  __shared__ int s_wcnt[kAlignWaves][MOE_MAX_EXPERTS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) s_wcnt[i / E][i % E] = 0;
  __syncthreads();
  if (P <= kAlignThreads) {
    const int p = tid;
    const int e_in = p < P ? ids[p] : 0;
    const bool valid = p < P && e_in >= 0 && e_in < E;  // out-of-range ids are dropped
    const int e = valid ? e_in : 0;
    if (p < P && !valid) pair_pos[p] = -1;
    const LaneGroup lg = lane_group(e, valid, id_bits, lane);
    if (valid && lg.rank == 0) s_wcnt[wave][e] = lg.cnt;
    __syncthreads();
    int c = 0;
    if (tid < E) {
#pragma unroll
      for (int w = 0; w < kAlignWaves; ++w) c += s_wcnt[w][tid];
    }
    align_scan(c, E, block_m, tid, lane, wave, s_off, offsets, active, tile_offsets);
    __syncthreads();
    if (valid) {
      int before = 0;
      for (int w = 0; w < wave; ++w) before += s_wcnt[w][e];
      const int q = s_off[e] + before + lg.rank;
      sorted_pairs[q] = p;
      pair_pos[p] = q;
    }
    return;
  }

  // chunk of each wavefront: a multiple of 64 pairs, in pair order
  const int chunk = (int)((((int64_t)P + kAlignWaves - 1) / kAlignWaves + 63) / 64 * 64);
  const int c0 = min(P, wave * chunk), c1 = min(P, c0 + chunk);
  constexpr int kU = 32;  // ids per lane loaded at once (2048 pairs per wavefront per batch)
  for (int b = c0; b < c1; b += 64 * kU) {
    int ev[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int p = b + 64 * u + lane;
      ev[u] = p < c1 ? ids[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (ev[u] >= 0 && ev[u] < E) atomicAdd(&s_wcnt[wave][ev[u]], 1);
  }
  __syncthreads();
  // expert totals, offsets and work list; then each column of counts becomes the
  // base positions of the wavefronts' chunks
  int c = 0;
  if (tid < E) {
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) c += s_wcnt[w][tid];
  }
  align_scan(c, E, block_m, tid, lane, wave, s_off, offsets, active, tile_offsets);
  __syncthreads();
  if (tid < E) {
    int base = s_off[tid];
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) {
      const int n = s_wcnt[w][tid];
      s_wcnt[w][tid] = base;
      base += n;
    }
  }
  __syncthreads();
  for (int b = c0; b < c1; b += 64 * kU) {
    int ev[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int p = b + 64 * u + lane;
      ev[u] = p < c1 ? ids[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int p = b + 64 * u + lane;
      if (b + 64 * u >= c1) break;
      const bool valid = p < c1 && ev[u] >= 0 && ev[u] < E;
      const int e = valid ? ev[u] : 0;
      if (p < c1 && !valid) pair_pos[p] = -1;
      const LaneGroup lg = lane_group(e, valid, id_bits, lane);
      // every lane reads its base before the group leader advances it (one wavefront:
      // the LDS read and write are issued in this order)
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

// Active experts of the step in ascending id order, from the routing table in
// LDS (s_ids[t][j], -1 = none): a bit mask (s_mask), then one wavefront
// compacts it into s_act (skipped when s_act is null).  Returns U; every
// workgroup builds the same list.
__device__ inline int build_active(const int (*s_ids)[MOE_MAX_TOPK], int T, int k, int E, uint32_t* s_mask, int* s_act,
                            int* s_u) {
  const int tid = threadIdx.x, n = blockDim.x;
  for (int i = tid; i < MOE_MAX_EXPERTS / 32; i += n) s_mask[i] = 0u;
  __syncthreads();
  for (int i = tid; i < T * k; i += n) {
    const int id = s_ids[i / k][i % k];
    if (id >= 0 && id < E) atomicOr(&s_mask[id >> 5], 1u << (id & 31));
  }
  __syncthreads();
  if (tid < 64) {
    uint32_t m = tid < MOE_MAX_EXPERTS / 32 ? s_mask[tid] : 0u;
    const int c = __popc(m);
    const int incl = wave_incl_scan(c);
    int pos = incl - c;
    while (s_act && m) {
      const int b = __ffs(m) - 1;
      s_act[pos++] = tid * 32 + b;
      m &= m - 1u;
    }
    if (tid == 63) *s_u = incl;
  }
  __syncthreads();
  return *s_u;
}

}  // namespace moe
