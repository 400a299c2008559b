// The fused down projection + routing-weighted combine pass of the decode paths
// (steps of at most 16 tokens), shared by the grouped entry point, the fused
// decode layer on four-bit blobs and the fused decode layer on nested blobs.
#pragma once

#include "align_block.hpp"
#include "ffn_common.hpp"
#include "mat_format.hpp"

namespace moe {

// fused down + combine: tiles per stripe, prefetch distance in groups, wavefronts
// per workgroup and resident wavefronts per SIMD
constexpr int kDcRT = 2, kDcD = 2, kDcWaves = 8, kDcOcc = 4;

// Down projection and routing-weighted combine in one pass, for steps of at most
// 16 tokens whose experts all take part in the call.  The combine is linear, so
// every group's contribution is scaled by the routing weight of its (token,
// expert) pair as it is accumulated: each partial sum is then already a sum over
// the token's routed outputs, and no per-pair fp32 result leaves the kernel.
//
// Work split: a wavefront owns one output stripe of RT tiles (16 RT rows of d),
// one active expert and one slice of UPW of its K groups (the 16 MFMA columns
// being the step's tokens, as in the gate/up pass); a workgroup holds WAVES
// consecutive (expert, slice) items of one stripe, a chunk of the stripe's list.
// The slice is unrolled completely: the loads of group i + D (weights and the
// pairs' h fragments; the slice's scales come in once, at its start, and are
// read from LDS) go out before group i is multiplied, in straight-line
// code with no branch, so the compiler counts the loads to wait for exactly and
// never moves registers that a load in flight will write.  The wavefronts meet
// in LDS in wavefront order, and the workgroup stores its 16 tokens x 16 RT rows
// of partial sums with device-coherent stores; the workgroup that counts itself
// last on the stripe's counter adds the chunks' partials in chunk order and
// writes the bf16 rows.  The counters are zeroed by the gate/up pass, which runs
// before this one on the stream.
constexpr int kDcMaxChunks = 32;

// PAIR: h rows in pair order (t * k + j) and the active experts built from the
// routing table in each workgroup (the fused decode layer); else h rows in
// expert-sorted order with the active list of moe_align.  route_ctr (PAIR): the
// n_route_ctr counters of the routing pass, zeroed here for the next step.
// PREC (LayerPrec): layout v1, whose weights come in K units of one group, or
// layout m1, in plane tiles of two groups (a lane's 16 bytes of a tile in the
// high plane and, at four bits, the low plane); the weights come D groups ahead
// of their unit's first group, the activations per group, D groups ahead (layout
// v1) or one (layout m1, whose two-group weight buffers leave no registers for
// more).  The low plane is read through a buffer resource without records for an
// item at two bits (zeros, no memory traffic; the four-bit decode of a zero low
// plane is the two-bit operand).  With kPrecMixed an item is at four bits when
// one of its pairs' routing weights reaches f.tau, and a prefetched item's low
// plane goes out once the routing table is read.
template <int RT, int D, int UPW, int WAVES, int OCC, bool PAIR, bool SPEC, int PREC = kPrecW4>
__global__ __launch_bounds__(WAVES * 64, OCC) void k_down_combine(FfnDev f, const uint16_t* __restrict__ h,
                                                                  uint16_t* __restrict__ out,
                                                                  float* __restrict__ part,
                                                                  int32_t* __restrict__ counters,
                                                                  int32_t* __restrict__ route_ctr, int n_route_ctr) {
  constexpr bool MAT = PREC != kPrecW4;
  constexpr bool kLo = PREC == kPrecAll4 || PREC == kPrecMixed;  // m1: the low plane is read
  constexpr int kGpu = MAT ? 2 : 1;                               // groups per K unit
  static_assert(UPW % kGpu == 0 && D % kGpu == 0, "whole units per slice and prefetch distance");
  constexpr int UPU = UPW / kGpu;           // units per slice
  constexpr int WR = D / kGpu + 1;          // weight buffers: the unit in use and those in flight
  constexpr int NPRO = (D - 1) / kGpu + 1;  // units of the first D groups
  constexpr int DX = MAT ? 1 : D;           // activation prefetch distance in groups
  constexpr int kRows = RT * kTileRows, kValues = 16 * kRows;  // 16 tokens x the stripe's rows
  constexpr int kThreads = WAVES * 64, kPer = kValues / kThreads;
  static_assert(kValues % kThreads == 0, "whole partial values per thread");
  const int G = f.I / kGroup;
  const int NU = G / kGpu;
  const int n_slices = (NU + UPU - 1) / UPU;
  const int n_stripes = f.d / (kTileRows * RT);
  const int stripe = blockIdx.x % n_stripes, chunk = blockIdx.x / n_stripes;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = lane_id();
  const int col = lane & 15, kq = lane >> 4;
  const int item = chunk * WAVES + wave;
  // the active count, the wavefront's work record (read within the work list's
  // capacity, used only if the item exists) and the routing table: one round trip
  int U = (PAIR || SPEC) ? 0 : f.active[0];
  i32x4_t rec = (PAIR || SPEC) ? i32x4_t{0, 0, 0, 0}
                               : reinterpret_cast<const i32x4_t*>(f.active + 4)[min(item / n_slices, f.umax - 1)];

  const uint32_t voff_c = 16u * lane;
  const uint32_t soff_c = (uint32_t)(f.off_w2_codes + (int64_t)(RT * stripe) * NU * kTileBytes);
  const uint32_t soff_l = MAT ? (uint32_t)(f.off_w2_lo + (int64_t)(RT * stripe) * NU * kTileBytes) : 0u;
  const uint32_t soff_s = (uint32_t)(f.off_w2_scales + (int64_t)(RT * stripe) * G * kTileRows * 2);
  struct Buf {
    u32x4_t c[RT];            // codes (v1) or high plane (m1)
    u32x4_t l[MAT ? RT : 1];  // low plane (m1)
  };
  // The slice's scales (per tile its UPW groups x 16 rows of bf16,
  // contiguous in the blob) come in with the item's first loads, 16 bytes per lane,
  // and wait in the wavefront's own LDS area for their groups (one LDS read per
  // tile and group instead of a memory load)
  constexpr int kSclTile = UPW * kTileRows * 2;                      // bytes per tile (UPW groups)
  constexpr int kSclLd = (RT * kSclTile + 1023) / 1024;              // 16-byte loads per lane
  __shared__ u32x4_t s_scl[WAVES][kSclLd * 64];
  __amdgpu_buffer_rsrc_t scl_res = __builtin_amdgcn_make_buffer_rsrc((void*)f.bank, (short)0, 0, kBufferRsrcWord3);
  u32x4_t scl_v[kSclLd];
  struct XBuf {
    u32x4_t x[4];
  };
  Buf buf[WR];
  __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc((void*)f.bank, (short)0, 0, kBufferRsrcWord3);
  __amdgpu_buffer_rsrc_t lres = wres;  // low plane: the blob, without records for an item at two bits
  int u0 = 0, nu = 1;
  auto lo_load = [&](Buf& b, int i) {
    if constexpr (MAT) {
      const int u = u0 + min(i, nu - 1);
#pragma unroll
      for (int r = 0; r < RT; ++r)
        b.l[r] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         lres, voff_c, soff_l + (uint32_t)(r * NU + u) * kTileBytes, kCacheNonTemporal));
    }
  };
  // unit i of the slice; past the slice's end the loads repeat its last unit
  // (weight 0), so the loads and their waits do not depend on the slice length.
  // LO (m1): with the low plane
  auto wload = [&](auto lo_c, Buf& b, int i) {
    constexpr bool LO = decltype(lo_c)::value;
    const int u = u0 + min(i, nu - 1);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      b.c[r] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                       wres, voff_c, soff_c + (uint32_t)(r * NU + u) * kTileBytes, kCacheNonTemporal));
      if constexpr (MAT && LO)
        b.l[r] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         lres, voff_c, soff_l + (uint32_t)(r * NU + u) * kTileBytes, kCacheNonTemporal));
    }
  };
  // chunk c = lane + 64 j of the slice's scales: tile c * 16 / kSclTile, bytes c * 16 % kSclTile
  // from its first group; past the stripe's scales the loads read zeros
  auto scl_load = [&]() {
#pragma unroll
    for (int j = 0; j < kSclLd; ++j) {
      const int c = lane + 64 * j, r = c * 16 / kSclTile, within = c * 16 % kSclTile;
      scl_v[j] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                       scl_res, (uint32_t)((r * G + kGpu * u0) * kTileRows * 2 + within), 0, 0));
    }
  };
  auto scl_store = [&]() {
#pragma unroll
    for (int j = 0; j < kSclLd; ++j) s_scl[wave][lane + 64 * j] = scl_v[j];
  };
  auto set_expert = [&](int e) {
    const int slot = f.slot_of_expert ? f.slot_of_expert[e] : e;
    wres = __builtin_amdgcn_make_buffer_rsrc((void*)(f.bank + (int64_t)slot * f.bank_stride), (short)0, 0x7FFFFFFF,
                                             kBufferRsrcWord3);
    scl_res = __builtin_amdgcn_make_buffer_rsrc((void*)(f.bank + (int64_t)slot * f.bank_stride + soff_s), (short)0,
                                                RT * G * kTileRows * 2, kBufferRsrcWord3);
    if constexpr (PREC == kPrecAll4) lres = wres;
    u0 = (item % n_slices) * UPU;
    nu = min(UPU, NU - u0);
  };
  // the loads issued before the routing table is read carry the low plane when
  // the precision does not depend on it
  using PreLo = std::integral_constant<bool, PREC == kPrecAll4>;
  using ItemLo = std::integral_constant<bool, kLo>;
  // SPEC: items over every expert in id order (steps that route at least one
  // pair per expert on average): the wavefront knows its expert before the
  // routing table is read and requests the weights of its first D groups at once
  // (kPrecMixed: without the low plane); an expert without pairs computes nothing
  const bool early = SPEC && item < f.E * n_slices;
  if (early) {
    rec[0] = item / n_slices;
    if (!PAIR) rec[1] = f.offsets[rec[0]];
    set_expert(rec[0]);
    scl_load();
#pragma unroll
    for (int j = 0; j < NPRO; ++j) wload(PreLo{}, buf[j], j);
  }

  __shared__ int s_ids[16][MOE_MAX_TOPK];
  __shared__ float s_w[16][MOE_MAX_TOPK];
  __shared__ f32x4_t s_red[WAVES][RT][64];
  __shared__ int s_last;
  __shared__ uint32_t s_mask[PAIR ? MOE_MAX_EXPERTS / 32 : 1];
  __shared__ int s_act[PAIR ? 16 * MOE_MAX_TOPK : 1];
  __shared__ int s_u;
  for (int i = tid; i < 16 * MOE_MAX_TOPK; i += kThreads) {
    const int t = i / MOE_MAX_TOPK, j = i % MOE_MAX_TOPK;
    const bool in = j < f.k && t < f.T;
    s_ids[t][j] = in ? f.topk_ids[t * f.k + j] : -1;
    s_w[t][j] = in ? f.topk_weights[t * f.k + j] : 0.f;
  }
  if (PAIR) {
    if (blockIdx.x == 0)
      for (int i = tid; i < n_route_ctr; i += kThreads) route_ctr[i] = 0;
    if (!SPEC) {
      __syncthreads();
      U = build_active(s_ids, f.T, f.k, f.E, s_mask, s_act, &s_u);
      rec[0] = s_act[min(item / n_slices, max(U - 1, 0))];
    }
  }
  const int n_items = SPEC ? f.E * n_slices : U * n_slices;
  const int nch = (n_items + WAVES - 1) / WAVES;          // chunks with work on every stripe
  if (chunk >= nch && !(chunk == 0 && nch == 0)) return;  // (no active expert: chunk 0 writes zeros)
  __syncthreads();

  f32x4_t tot[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) tot[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the lane's token: its slot for the item's expert (if routed there), its h row
  const int e = rec[0];
  int hit = -1;
  if (item < n_items)
    for (int j = 0; j < f.k; ++j) hit = s_ids[col][j] == e ? j : hit;
  const uint32_t colmask = (uint32_t)__ballot(hit >= 0) & 0xFFFFu;
  if (item < n_items && colmask != 0u) {
    if (!early) set_expert(e);
    const uint32_t kMask = MAT ? 0u : vgpr_const(0x00780078u), kOne = vgpr_const(0x3F803F80u);
    const uint32_t kMhi = MAT ? vgpr_const(0x00600060u) : 0u, kMlo = MAT ? vgpr_const(0x00180018u) : 0u;
    const u32x4_t ones_w = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const bf16x8_t ones = as_bf16x8(ones_w);
    const __amdgpu_buffer_rsrc_t hres =
        __builtin_amdgcn_make_buffer_rsrc((void*)h, (short)0, (int)(f.P * f.I * 2), kBufferRsrcWord3);
    const int hrow = PAIR ? col * f.k + hit : rec[1] + __popc(colmask & ((1u << col) - 1u));
    const uint32_t hoff = hit >= 0 ? (uint32_t)(hrow * f.I + 8 * kq) * 2u : 0x7F000000u;  // else reads zeros
    const float wt = hit >= 0 ? s_w[col][hit] : 0.f;
    // the item's precision: four bits when one of its pairs' weights reaches tau
    float xcoef = PREC == kPrecAll2 ? -22.5f : -24.f;  // X term of a group
    if constexpr (PREC == kPrecMixed) {
      const bool full = __ballot(hit >= 0 && wt >= f.tau) != 0;
      lres = full ? wres : __builtin_amdgcn_make_buffer_rsrc((void*)f.bank, (short)0, 0, kBufferRsrcWord3);
      xcoef = full ? -24.f : -22.5f;
    }
    // activations of group i of the slice (past its end: its last group again)
    auto xload = [&](XBuf& b, int i) {
      const int g = kGpu * u0 + min(i, kGpu * nu - 1);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        b.x[i4] = __builtin_bit_cast(
            u32x4_t,
            __builtin_amdgcn_raw_buffer_load_b128(hres, hoff + (uint32_t)(g * kGroup + 32 * i4) * 2u, 0, 0));
    };
    // group i of the slice: half i % kGpu of its unit's weights
    auto compute = [&](const Buf& b, const XBuf& xb, int i) {
      const int hg = i % kGpu;
      const float w = i / kGpu < nu ? wt : 0.f;
      f32x4_t acc[RT], as = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[r] = as;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const bf16x8_t xv = as_bf16x8(xb.x[i4]);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          u32x4_t wv;
          if constexpr (MAT) {
            const int step = 4 * hg + i4;
            wv = decode_step<kLo>(b.c[r][step >> 1], kLo ? b.l[r][step >> 1] : 0u, step & 1, kMhi, kMlo, kOne);
          } else {
            wv = decode_word_biased(b.c[r][i4], kMask, kOne);
          }
          acc[r] = mfma16x16x32(as_bf16x8(wv), xv, acc[r]);
        }
        as = mfma16x16x32(ones, xv, as);
      }
      const float xs = xcoef * as[0];  // every row of the ones product holds the column's group sum
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const int gi = kGpu * min(i / kGpu, nu - 1) + hg;  // the group within the slice
        const u32x2_t sw = reinterpret_cast<const u32x2_t*>(s_scl[wave])[r * (kSclTile / 8) + gi * 4 + kq];
        const float s4[4] = {__uint_as_float(sw[0] << 16), __uint_as_float(sw[0] & 0xFFFF0000u),
                             __uint_as_float(sw[1] << 16), __uint_as_float(sw[1] & 0xFFFF0000u)};
#pragma unroll
        for (int q = 0; q < 4; ++q) tot[r][q] = fmaf(w * s4[q], fmaf(16.f, acc[r][q], xs), tot[r][q]);
      }
    };
    XBuf xbuf[DX + 1];
    if (!early) {
      scl_load();
#pragma unroll
      for (int j = 0; j < NPRO; ++j) wload(ItemLo{}, buf[j], j);
    } else if constexpr (PREC == kPrecMixed) {
#pragma unroll
      for (int j = 0; j < NPRO; ++j) lo_load(buf[j], j);
    }
#pragma unroll
    for (int j = 0; j < DX; ++j) xload(xbuf[j], j);
    scl_store();
    // the scheduling barriers keep each group's loads ahead of the multiply that
    // precedes their use (the scheduler would otherwise sink them to their users)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      if (i + D < UPW && (i + D) % kGpu == 0) wload(ItemLo{}, buf[((i + D) / kGpu) % WR], (i + D) / kGpu);
      if (i + DX < UPW) xload(xbuf[(i + DX) % (DX + 1)], i + DX);
      __builtin_amdgcn_sched_barrier(0);
      compute(buf[(i / kGpu) % WR], xbuf[i % (DX + 1)], i);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // wavefronts' sums in wavefront order; value v = rows * t + n of the
  // workgroup's partial (token t, stripe row n) is owned by thread v % threads
#pragma unroll
  for (int r = 0; r < RT; ++r) s_red[wave][r][lane] = tot[r];
  __syncthreads();
  float* pp = part + (int64_t)stripe * kDcMaxChunks * kValues;
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int vi = tid + kThreads * m, t = vi / kRows, n = vi % kRows;
    const int rt = n >> 4, src = ((n & 15) >> 2) * 16 + t, q = n & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += s_red[w][rt][src][q];
    __hip_atomic_store(pp + chunk * kValues + vi, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's partials have reached device scope
  __syncthreads();
  const int n_arrive = max(nch, 1);
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(counters + stripe, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_arrive - 1;
  __syncthreads();
  if (!s_last) return;
  if (tid == 0) counters[stripe] = 0;  // left at zero for the next call
  // every chunk's partial is complete at device scope: add them in chunk order
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int vi = tid + kThreads * m, t = vi / kRows, n = vi % kRows;
    float pv[kDcMaxChunks];
#pragma unroll
    for (int c = 0; c < kDcMaxChunks; ++c)
      pv[c] = c < n_arrive ? __hip_atomic_load(pp + c * kValues + vi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : 0.f;
    float sum = pv[0];
#pragma unroll
    for (int c = 1; c < kDcMaxChunks; ++c)
      if (c < n_arrive) sum += pv[c];
    if (t < f.T) out[(int64_t)t * f.d + kRows * stripe + n] = (uint16_t)f32_to_bf16_bits(sum);
  }
}

template <int UPW, bool SPEC, int PREC>
static void launch_dc(const FfnDev& f, const uint16_t* h, uint16_t* out, float* part, int32_t* counters,
                      int32_t* route_ctr, int n_route_ctr, hipStream_t s, bool pair, dim3 grid) {
  const dim3 block(kDcWaves * 64);
  if constexpr (PREC != kPrecW4) {
    // nested blobs: the fused decode layer only (h rows in pair order)
    hipLaunchKernelGGL((k_down_combine<kDcRT, kDcD, UPW, kDcWaves, kDcOcc, true, SPEC, PREC>), grid, block, 0, s, f,
                       h, out, part, counters, route_ctr, n_route_ctr);
  } else if (pair) {
    hipLaunchKernelGGL((k_down_combine<kDcRT, kDcD, UPW, kDcWaves, kDcOcc, true, SPEC>), grid, block, 0, s, f, h, out,
                       part, counters, route_ctr, n_route_ctr);
  } else {
    hipLaunchKernelGGL((k_down_combine<kDcRT, kDcD, UPW, kDcWaves, kDcOcc, false, SPEC>), grid, block, 0, s, f, h,
                       out, part, counters, route_ctr, n_route_ctr);
  }
}

// The fused down + combine pass for format / precision PREC (nested blobs: pair
// order only).  Groups per wavefront from dc_units_per_wave (checked when the
// call chose this path; even for nested blobs, whose I is a multiple of 256).
template <int PREC>
void launch_down_combine_t(const FfnDev& f, const uint16_t* h, uint16_t* out, float* part, int32_t* counters,
                           int32_t* route_ctr, int n_route_ctr, hipStream_t s, bool pair) {
  const int stripes = f.d / (kTileRows * kDcRT);
  const int upw = dc_units_per_wave(f.umax, f.I / kGroup, stripes);
  const int64_t slices = ceil_div(f.I / kGroup, upw);
  const dim3 grid((unsigned)(stripes * ceil_div((int64_t)f.umax * slices, kDcWaves)));
  // every expert in id order when the step routes at least one pair per expert
  // on average (umax == E then), else the active experts
  const bool spec = (int64_t)f.T * f.k >= f.E;
  if (upw <= 2) {
    if (spec) launch_dc<2, true, PREC>(f, h, out, part, counters, route_ctr, n_route_ctr, s, pair, grid);
    else launch_dc<2, false, PREC>(f, h, out, part, counters, route_ctr, n_route_ctr, s, pair, grid);
  } else if (upw <= 4) {
    if (spec) launch_dc<4, true, PREC>(f, h, out, part, counters, route_ctr, n_route_ctr, s, pair, grid);
    else launch_dc<4, false, PREC>(f, h, out, part, counters, route_ctr, n_route_ctr, s, pair, grid);
  } else if (upw <= 8) {
    if (spec) launch_dc<8, true, PREC>(f, h, out, part, counters, route_ctr, n_route_ctr, s, pair, grid);
    else launch_dc<8, false, PREC>(f, h, out, part, counters, route_ctr, n_route_ctr, s, pair, grid);
  } else {
    if (spec) launch_dc<16, true, PREC>(f, h, out, part, counters, route_ctr, n_route_ctr, s, pair, grid);
    else launch_dc<16, false, PREC>(f, h, out, part, counters, route_ctr, n_route_ctr, s, pair, grid);
  }
}

}  // namespace moe
