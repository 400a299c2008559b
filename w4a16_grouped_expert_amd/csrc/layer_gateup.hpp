// The fused decode layer (moe_decode_layer, and moe_mat_decode_layer on nested
// two/four-bit blobs): a whole decode step of the W4A16 MoE layer (at most 16
// tokens) in two launches: routing + grouped gate/up + SwiGLU, then the grouped
// down projection with the routing-weighted combine (ExactMoE, page "Every
// Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference", Abstract: the
// BF16 router and its unchanged top-k, every selected expert through fused
// grouped kernels on four-bit weights).  This header holds the first launch's
// kernel and the host code both entry points share.
//
// The first launch is persistent (every workgroup resident).  Each wavefront
// first issues the weight loads of its first gate/up item when that item is
// known without the routing (every expert in order, used when the step routes
// at least as many pairs as there are experts, so that few are idle); the
// workgroups with the lowest indices then compute the router logits, one
// (token, expert) dot product per wavefront, with the arithmetic of moe_route
// (float64 sums of the exact bf16 products, rounded once); the wavefront that
// completes a token's logits selects its top-k and weights and publishes the
// ids in a ready table, and the workgroups stage their activations in LDS.  The
// gate/up items run as in the grouped decode pass, h going to rows in pair order
// (t * k + j): no expert-sorted permutation is needed when every MFMA column is a
// token.  Items over every expert do not depend on the routing, so a workgroup
// waits for it (a bounded poll of the ready table) only before its first h
// store, and skips the items of experts without pairs after that; items over
// the active experts wait for it before the first item.  The
// second launch is the fused down + combine pass (down_combine.hpp), which builds
// the active expert list from the routing table itself.  Routing results are
// bit-identical to moe_route_align; the arithmetic of every gate/up item and of
// the down pass is that of moe_w4a16_grouped_ffn's decode kernels with one
// wavefront per item.
#pragma once

#include "align_block.hpp"
#include "down_combine.hpp"
#include "ffn_common.hpp"
#include "mat_format.hpp"
#include "route_rank.hpp"

namespace moe {

// counters (MOE_DECODE_LAYER_COUNTERS int32, zero between calls); the counters
// that many workgroups update or poll sit on 128-byte lines of their own
constexpr int kLine = 32;                         // int32 per 128-byte line
constexpr int kCtrLogits = kLine;                 // [kLine * (1 + t)]: logits of token t written
// [t * k + j]: expert id + 1 once token t is routed, plus kReadyHeavy when the
// pair's routing weight reaches the four-bit threshold of nested blobs
constexpr int kCtrReady = kLine * 17;
constexpr int kReadyHeavy = 1 << 16;              // above every expert id + 1 (E <= 1024)
constexpr int kCtrRouteEnd = kCtrReady + 16 * MOE_MAX_TOPK;  // routing counters: [0, kCtrRouteEnd)
constexpr int kCtrDown = kCtrRouteEnd;            // fused down + combine stripe counters (d / 32 <= 128)
constexpr int kCtrError = MOE_DECODE_LAYER_COUNTERS - 1;
static_assert(kCtrDown + 128 <= kCtrError, "counter block too small");
constexpr int kSpinLimit = 1 << 22;

struct RouteDev {
  const uint16_t* wr;
  int renormalize;
  float tau;  // kReadyHeavy threshold (+inf when no pair is ever heavy)
  float* logits;
  int32_t* ids;
  float* weights;
  int32_t* ctr;
};

// Top-k and weights of token t by one wavefront, from its E logits (read with
// device-coherent loads), in the order and with the sums of moe_route: for E up
// to kRankMaxE every logit's rank (the logits it loses to, by value desc, index
// asc) is counted against the row in the wavefront's LDS area, and the k best
// land at their rank; beyond that, k rounds of a wave-wide argmax.  The ids also
// go, plus one, to the ready table with device-coherent stores: a non-zero
// entry is a routed pair.
constexpr int kRankMaxE = 128;

__device__ void route_token(const RouteDev& r, int t, int E, int k, float* s_lg, float* s_sel_v, int* s_sel_i) {
  const int lane = lane_id();
  const int nper = (E + 63) / 64;  // <= 16
  const float* lg = r.logits + (int64_t)t * E;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    v[i] = (i < nper && e < E) ? __hip_atomic_load(lg + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : -INFINITY;
  }
  float sel_v = 0.f, lmax = 0.f;  // lane j < k: selection j
  int sel_i = 0;
  if (E <= kRankMaxE) {
#pragma unroll
    for (int i = 0; i < kRankMaxE / 64; ++i)
      if (lane + 64 * i < E) s_lg[lane + 64 * i] = v[i];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < kRankMaxE / 64; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        const int rank = rank_in_row(s_lg, E, v[i], e);
        if (rank < k) {
          s_sel_v[rank] = v[i];
          s_sel_i[rank] = e;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    lmax = s_sel_v[0];
    if (lane < k) {
      sel_v = s_sel_v[lane];
      sel_i = s_sel_i[lane];
    }
  } else {
    uint32_t taken = 0;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j >= k) break;
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;  // sentinel below every candidate
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = lane + 64 * i;
        if (i < nper && e < E && !((taken >> i) & 1u) && better(v[i], e, bv, bi)) {
          bv = v[i];
          bi = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (j == 0) lmax = bv;
      if (lane == j) {
        sel_v = bv;
        sel_i = bi;
      }
    }
  }
  const float ex = lane < k ? expf(sel_v - lmax) : 0.f;
  float den = 0.f;
  if (r.renormalize) {
    for (int j = 0; j < k; ++j) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
  } else {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i < nper && lane + 64 * i < E) part += expf(v[i] - lmax);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    den = part;
  }
  if (lane < k) {
    const float wv = ex / den;
    r.ids[(int64_t)t * k + lane] = sel_i;
    r.weights[(int64_t)t * k + lane] = wv;
    __hip_atomic_store(r.ctr + kCtrReady + t * k + lane, sel_i + 1 + (wv >= r.tau ? kReadyHeavy : 0),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Routing + grouped gate/up + SwiGLU.  SPEC: items are (expert, stripe) over
// every expert in id order, the first one prefetched before the routing is
// known (an item of an expert without pairs is skipped); else over the active
// experts, known after the routing.
// KS > 1 (with !SPEC, for steps with few items): each item's K units are split
// over KS wavefronts of one workgroup, whose partial sums meet in LDS in part
// order before the SwiGLU.
// PREC (LayerPrec): the weight format.  Layout v1 is walked one group (K unit)
// at a time, layout m1 one plane tile (two groups) at a time: a lane's 16 bytes
// of a tile in the high plane and, at four bits, the low plane.  The low plane
// of an m1 item is read through a buffer resource that has no records when the
// item runs at two bits (the loads then return zeros without touching memory,
// and the four-bit decode of a zero low plane is the two-bit operand), so one
// code path serves both precisions.  With kPrecMixed an item's precision comes
// from the routing (the heavy flags of the ready table): a prefetched first item
// requests its high plane and scales before the routing and its low plane after
// it.  The arithmetic per group is that of the nested grouped pass, at four bits
// that of layout v1 term for term.
template <int RT, int NB, int MAXG, bool SPEC, int KS, int PREC>
__global__ __launch_bounds__(512, 4) void k_layer_gateup(FfnDev f, RouteDev r, uint16_t* __restrict__ hout) {
  constexpr bool MAT = PREC != kPrecW4;
  constexpr bool kLo = PREC == kPrecAll4 || PREC == kPrecMixed;  // m1: the low plane is read
  constexpr int kWaves = 8;
  zero_down_counters(f);
  const int G = f.d / kGroup;
  constexpr int kGpu = MAT ? 2 : 1;  // groups per K unit
  const int NU = G / kGpu;           // K units per item
  const int T = f.T, E = f.E, k = f.k;
  const int n_stripes = 2 * f.I / (kTileRows * RT);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int col = lane & 15, kq = lane >> 4;
  const int worker = blockIdx.x * kWaves + wave, n_workers = gridDim.x * kWaves;
  const int64_t tile_stride_c = (int64_t)NU * kTileBytes;  // a row tile of codes (v1) or of one plane (m1)
  const int64_t tile_stride_s = (int64_t)G * kTileRows;

  struct Buf {
    u32x4_t c[RT];            // codes (v1) or high plane (m1)
    u32x4_t l[MAT ? RT : 1];  // low plane (m1)
  };
  Buf buf[NB];
  const uint8_t* codes = nullptr;
  // The item's scales (RT tiles x G groups x 16 rows of bf16, contiguous in the
  // blob) come in at the item's start, one 16-byte load per lane, and wait in the
  // wavefront's own LDS area for their groups (one LDS read per tile and group
  // instead of a memory load)
  constexpr int kSclLd = RT * MAXG * 32 / 1024;  // 16-byte loads per lane
  __shared__ u32x4_t s_scl[kWaves][kSclLd * 64];
  __amdgpu_buffer_rsrc_t scl_res = __builtin_amdgcn_make_buffer_rsrc((void*)f.bank, (short)0, 0, kBufferRsrcWord3);
  u32x4_t scl_v[kSclLd];
  auto scl_load = [&]() {
#pragma unroll
    for (int j = 0; j < kSclLd; ++j)
      scl_v[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(scl_res, 16u * (lane + 64 * j), 0, 0));
  };
  auto scl_store = [&]() {
#pragma unroll
    for (int j = 0; j < kSclLd; ++j) s_scl[wave][lane + 64 * j] = scl_v[j];
  };
  // m1: the item's low plane through a buffer resource
  __amdgpu_buffer_rsrc_t lres = __builtin_amdgcn_make_buffer_rsrc((void*)f.bank, (short)0, 0, kBufferRsrcWord3);
  uint32_t lo_off = 0;  // the item's stripe of the low plane in its blob
  float xcoef = PREC == kPrecAll2 ? -22.5f : -24.f;  // X term of a group (kPrecMixed: per item)
  // past the item's last unit (g_lim, NU or the end of the wavefront's K part)
  // the loads repeat the last one and the unit's weight is 0, so no load sits
  // under a branch and the wait counts stay exact
  int g_lim = NU;
  auto lo_load = [&](Buf& b, int rr, int ul) {
    if constexpr (MAT)
      b.l[rr] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                       lres, 16u * lane, lo_off + (uint32_t)(rr * tile_stride_c + ul * kTileBytes), kCacheNonTemporal));
  };
  // LO (m1): with the low plane
  // unit u's loads; LO (m1): with the low plane
  auto load = [&](auto lo_c, Buf& b, int u) {
    constexpr bool LO = decltype(lo_c)::value;
    const int ul = min(u, g_lim - 1);
#pragma unroll
    for (int rr = 0; rr < RT; ++rr) {
      b.c[rr] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(codes + rr * tile_stride_c + (int64_t)ul * kTileBytes));
      if constexpr (MAT && LO) lo_load(b, rr, ul);
    }
  };
  // the low plane alone, for units whose other loads went out before the item's precision was known
  auto load_lo = [&](Buf& b, int u) {
    if constexpr (MAT) {
      const int ul = min(u, g_lim - 1);
#pragma unroll
      for (int rr = 0; rr < RT; ++rr) lo_load(b, rr, ul);
    }
  };
  auto set_item = [&](int e, int stripe) {
    const uint8_t* blob = f.bank + (int64_t)e * f.bank_stride;
    const int64_t roff = (int64_t)(RT * stripe) * tile_stride_c;
    codes = blob + f.off_w13_codes + roff + 16 * lane;
    if constexpr (MAT) lo_off = (uint32_t)(f.off_w13_lo + roff);
    scl_res = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(blob + f.off_w13_scales + (int64_t)(RT * stripe) * tile_stride_s * 2), (short)0, RT * G * 32,
        kBufferRsrcWord3);
  };
  // the item's precision (m1): the low plane's records and the X coefficient
  auto set_precision = [&](int e, bool full) {
    if constexpr (kLo)
      lres = __builtin_amdgcn_make_buffer_rsrc((void*)(f.bank + (int64_t)e * f.bank_stride), (short)0,
                                               full ? 0x7FFFFFFF : 0, kBufferRsrcWord3);
    (void)e;
    if constexpr (PREC == kPrecMixed) xcoef = full ? -24.f : -22.5f;
  };
  // the loads issued before the routing is known leave out the low plane (m1): it
  // goes out with the first item (few registers stay live over the routing)
  using ItemLo = std::integral_constant<bool, kLo>;

  // 1. the first item's weights, when it does not depend on the routing (the
  //    wavefronts that compute logits issue them after their router loads)
  // items are dealt to the workgroups in turn (item i to workgroup i mod the grid),
  // so every workgroup, and every CU, gets the same share of them, idle experts
  // included
  int item = wave * gridDim.x + blockIdx.x;
  const bool prefetched = SPEC && item < E * n_stripes;
  const int n_tasks = T * E;
  const int n_logit = min(n_workers, n_tasks);
  auto prefetch = [&]() {
    if (prefetched) {
      set_item(item / n_stripes, item % n_stripes);
      scl_load();
#pragma unroll
      for (int j = 0; j < NB - 1; ++j) load(std::false_type{}, buf[j], j);
    }
  };

  // 2. router logits, one (token, expert) per wavefront of the lowest workgroups
  __shared__ float s_lg[kWaves][kRankMaxE];
  __shared__ float s_sel_v[kWaves][MOE_MAX_TOPK];
  __shared__ int s_sel_i[kWaves][MOE_MAX_TOPK];
  __shared__ int s_route[kWaves];
  const int nch = f.d / 8;
  // logit of task (t, e), rounded once; lane 0 stores it with a device-coherent store
  auto logit = [&](int task) {
    const int t = task / E, e = task % E;
    const uint16_t* xr = f.x + (int64_t)t * f.d;
    const uint16_t* wrow = r.wr + (int64_t)e * f.d;
    double acc = 0.0;
    constexpr int kB = 4;  // chunks per lane in flight (the sum order does not depend on it)
    for (int c0 = 0; c0 < nch; c0 += 64 * kB) {
      u32x4_t xq[kB], wq[kB];
#pragma unroll
      for (int c = 0; c < kB; ++c) {
        const int ch = c0 + lane + 64 * c;
        xq[c] = ch < nch ? *reinterpret_cast<const u32x4_t*>(xr + 8 * ch) : u32x4_t{0u, 0u, 0u, 0u};
        wq[c] = ch < nch ? *reinterpret_cast<const u32x4_t*>(wrow + 8 * ch) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int c = 0; c < kB; ++c)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc = fma((double)bf16_bits_to_f32(xq[c][m] & 0xFFFFu), (double)bf16_bits_to_f32(wq[c][m] & 0xFFFFu),
                    acc);
          acc = fma((double)bf16_bits_to_f32(xq[c][m] >> 16), (double)bf16_bits_to_f32(wq[c][m] >> 16), acc);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0)
      __hip_atomic_store(r.logits + (int64_t)t * E + e, (float)acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the logit has reached device scope
  };
  if (n_tasks <= n_workers) {
    // one task per wavefront, counted once per workgroup and token: the
    // workgroup that completes a token's E logits routes it (a wavefront per token)
    if ((int)blockIdx.x * kWaves < n_tasks) {
      if (worker < n_tasks) logit(worker);
      __syncthreads();
      if (threadIdx.x == 0) {
        const int first = blockIdx.x * kWaves, last_task = min(first + kWaves, n_tasks) - 1;
        int n_done = 0;
        for (int t = first / E; t <= last_task / E; ++t) {
          const int cnt = min(last_task, t * E + E - 1) - max(first, t * E) + 1;
          if (__hip_atomic_fetch_add(r.ctr + kCtrLogits + kLine * t, cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) +
                  cnt == E)
            s_route[n_done++] = t;
        }
        for (int j = n_done; j < kWaves; ++j) s_route[j] = -1;
      }
      __syncthreads();
      const int t = s_route[wave];
      if (t >= 0) route_token(r, t, E, k, s_lg[wave], s_sel_v[wave], s_sel_i[wave]);
    }
    prefetch();
  } else if (worker >= n_logit) {
    prefetch();
  } else {
    for (int task = worker; task < n_tasks; task += n_logit) {
      logit(task);
      const int t = task / E;
      int last = 0;
      if (lane == 0)
        last = __hip_atomic_fetch_add(r.ctr + kCtrLogits + kLine * t, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == E - 1;
      if (__builtin_amdgcn_readfirstlane(last)) route_token(r, t, E, k, s_lg[wave], s_sel_v[wave], s_sel_i[wave]);
    }
    prefetch();
  }

  // 3. activations in LDS (as the grouped gate/up pass), while the routing completes
  __shared__ u32x4_t s_x[MAXG * 4 * 64];
  __shared__ float s_xs[MAXG * 16];
  __shared__ int s_ids[16][MOE_MAX_TOPK];
  __shared__ uint32_t s_mask[MOE_MAX_EXPERTS / 32];
  __shared__ int s_act[SPEC ? 1 : MOE_MAX_EXPERTS];
  __shared__ int s_u;
  {
    const u32x4_t ones_w = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const bf16x8_t ones = as_bf16x8(ones_w);
    const __amdgpu_buffer_rsrc_t xres =
        __builtin_amdgcn_make_buffer_rsrc((void*)f.x, (short)0, (int)(f.T * f.d * 2), kBufferRsrcWord3);
    const uint32_t xoff = (uint32_t)(col * f.d + 8 * kq) * 2u;
    for (int g = wave; g < G; g += kWaves) {
      u32x4_t xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xv[i] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xres, xoff + (uint32_t)(g * kGroup + 32 * i) * 2u, 0, 0));
      f32x4_t as = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s_x[(4 * g + i) * 64 + lane] = xv[i];
        as = mfma16x16x32(ones, as_bf16x8(xv[i]), as);
      }
      if (lane < 16) s_xs[g * 16 + lane] = as[0];  // C column = lane, every row the same sum
    }
  }

  // 4. the routing table in LDS: wavefront 0 polls the ready table until every
  //    pair's entry is set (bounded: a timeout is flagged in the counters and the
  //    pass goes on with whatever the table holds).  SPEC: items do not depend on
  //    the routing, so the wait moves to the first h store (below; with
  //    kPrecMixed, to the first item); s_routed tells the other wavefronts that
  //    s_ids, s_mask and s_fmask are filled.
  __shared__ int s_routed;
  __shared__ uint32_t s_fmask[PREC == kPrecMixed ? MOE_MAX_EXPERTS / 32 : 1];  // experts at four bits
  auto read_routing = [&]() {
    const int n = T * k;  // <= 256: at most 4 entries per lane
    int id[4];
    int spins = 0;
    for (;;) {
      bool ready = true;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i = lane + 64 * m;
        id[m] = i < n ? __hip_atomic_load(r.ctr + kCtrReady + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1;
        ready &= id[m] != 0;
      }
      if (__builtin_amdgcn_read_exec() == __ballot(ready)) break;
      if (++spins > kSpinLimit) {
        if (lane == 0) __hip_atomic_store(r.ctr + kCtrError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int i = lane + 64 * m;
      if (i < 16 * MOE_MAX_TOPK) {
        const int t = i / MOE_MAX_TOPK, j = i % MOE_MAX_TOPK;
        s_ids[t][j] = -1;
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int i = lane + 64 * m;
      if (i < n) s_ids[i / k][i % k] = (id[m] & (kReadyHeavy - 1)) - 1;
    }
    if (SPEC) {
      for (int i = lane; i < MOE_MAX_EXPERTS / 32; i += 64) s_mask[i] = 0u;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i = lane + 64 * m, ex = (id[m] & (kReadyHeavy - 1)) - 1;
        if (i < n && ex >= 0 && ex < E) atomicOr(&s_mask[ex >> 5], 1u << (ex & 31));
      }
    }
    if constexpr (PREC == kPrecMixed) {
      for (int i = lane; i < MOE_MAX_EXPERTS / 32; i += 64) s_fmask[i] = 0u;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i = lane + 64 * m, ex = (id[m] & (kReadyHeavy - 1)) - 1;
        if (i < n && ex >= 0 && ex < E && (id[m] & kReadyHeavy)) atomicOr(&s_fmask[ex >> 5], 1u << (ex & 31));
      }
    }
  };
  // SPEC: wavefront 0 publishes the routing table; the others wait for it (bounded)
  auto await_routing = [&]() {
    if (wave == 0) {
      read_routing();
      __hip_atomic_store(&s_routed, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
      for (int spins = 0; __hip_atomic_load(&s_routed, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0 &&
                          spins < kSpinLimit;
           ++spins)
        __builtin_amdgcn_s_sleep(2);
    }
  };
  if (!SPEC && wave == 0) read_routing();
  if (SPEC && threadIdx.x == 0) s_routed = 0;
  __syncthreads();
  const int U = SPEC ? E : build_active(s_ids, T, k, E, s_mask, s_act, &s_u);
  const int n_items = U * n_stripes;

  // an item's precision (uniform over the wavefront)
  auto item_full = [&](int e) -> bool {
    if constexpr (PREC == kPrecMixed)
      return __builtin_amdgcn_readfirstlane((int)((s_fmask[e >> 5] >> (e & 31)) & 1u)) != 0;
    else
      return PREC != kPrecAll2;
  };

  // 5. gate/up items
  const uint32_t kMask = MAT ? 0u : vgpr_const(0x00780078u), kOne = vgpr_const(0x3F803F80u);
  const uint32_t kMhi = MAT ? vgpr_const(0x00600060u) : 0u, kMlo = MAT ? vgpr_const(0x00180018u) : 0u;
  auto compute = [&](const Buf& b, int u, f32x4_t* tot) {
    const int ul = min(u, g_lim - 1);
    const float gv = u < g_lim ? 1.f : 0.f;
#pragma unroll
    for (int hg = 0; hg < kGpu; ++hg) {
      const int g = kGpu * ul + hg;
      const float xs = xcoef * s_xs[g * 16 + col];
      f32x4_t acc[RT];
#pragma unroll
      for (int rr = 0; rr < RT; ++rr) acc[rr] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8_t xv = as_bf16x8(s_x[(4 * g + i) * 64 + lane]);
#pragma unroll
        for (int rr = 0; rr < RT; ++rr) {
          u32x4_t wv;
          if constexpr (MAT) {
            const int step = 4 * hg + i;
            wv = decode_step<kLo>(b.c[rr][step >> 1], kLo ? b.l[rr][step >> 1] : 0u, step & 1, kMhi, kMlo, kOne);
          } else {
            wv = decode_word_biased(b.c[rr][i], kMask, kOne);
          }
          acc[rr] = mfma16x16x32(as_bf16x8(wv), xv, acc[rr]);
        }
      }
#pragma unroll
      for (int rr = 0; rr < RT; ++rr) {
        const u32x2_t sw = reinterpret_cast<const u32x2_t*>(s_scl[wave])[rr * G * 4 + g * 4 + kq];
        const float s4[4] = {__uint_as_float(sw[0] << 16), __uint_as_float(sw[0] & 0xFFFF0000u),
                             __uint_as_float(sw[1] << 16), __uint_as_float(sw[1] & 0xFFFF0000u)};
#pragma unroll
        for (int q = 0; q < 4; ++q) tot[rr][q] = fmaf(gv * s4[q], fmaf(16.f, acc[rr][q], xs), tot[rr][q]);
      }
    }
  };
  // SwiGLU of a finished item and its h stores (pair order)
  auto store_h = [&](const f32x4_t* tot, int e, int stripe) {
    int hit = -1;
    for (int j = 0; j < k; ++j) hit = s_ids[col][j] == e ? j : hit;
#pragma unroll
    for (int p = 0; p < RT / 2; ++p) {
      float hf[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hf[q] = silu_f32(tot[2 * p][q]) * tot[2 * p + 1][q];
      if (hit >= 0) {
        const int hcol = kTileRows * ((RT / 2) * stripe + p) + 4 * kq;
        const u32x2_t o = pack_bf16x4(hf[0], hf[1], hf[2], hf[3]);
        *reinterpret_cast<u32x2_t*>(hout + (int64_t)(col * k + hit) * f.I + hcol) = o;
      }
    }
  };
  if constexpr (KS > 1) {
    static_assert(!SPEC, "K parts only for items over the active experts");
    __shared__ f32x4_t s_part[kWaves][RT][64];
    constexpr int kGroups = kWaves / KS;  // items per workgroup and round
    const int grp = wave / KS, kp = wave % KS;
    const int gq = (NU + KS - 1) / KS;
    const int g0 = min(NU, kp * gq);
    g_lim = min(NU, g0 + gq);
    for (int rnd = 0; (rnd * kGroups) * (int)gridDim.x + (int)blockIdx.x < n_items; ++rnd) {
      const int it = (rnd * kGroups + grp) * gridDim.x + blockIdx.x;
      const bool valid = it < n_items && g0 < g_lim;
      f32x4_t tot[RT];
#pragma unroll
      for (int rr = 0; rr < RT; ++rr) tot[rr] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (valid) {
        const int e = s_act[it / n_stripes];
        set_item(e, it % n_stripes);
        set_precision(e, item_full(e));
        scl_load();
#pragma unroll
        for (int j = 0; j < NB - 1; ++j) load(ItemLo{}, buf[j], g0 + j);
        scl_store();
        for (int gc = g0; gc < g_lim; gc += NB) {
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            load(ItemLo{}, buf[(j + NB - 1) % NB], gc + j + NB - 1);
            compute(buf[j], gc + j, tot);
          }
        }
      }
      if (kp > 0) {
#pragma unroll
        for (int rr = 0; rr < RT; ++rr) s_part[wave][rr][lane] = tot[rr];
      }
      __syncthreads();
      if (kp == 0 && it < n_items) {
#pragma unroll
        for (int q = 1; q < KS; ++q)
#pragma unroll
          for (int rr = 0; rr < RT; ++rr) {
            const f32x4_t o = s_part[wave + q][rr][lane];
#pragma unroll
            for (int c = 0; c < 4; ++c) tot[rr][c] = tot[rr][c] + o[c];
          }
        store_h(tot, s_act[it / n_stripes], it % n_stripes);
      }
      __syncthreads();  // s_part is free for the next round
    }
  } else {
    // SPEC: an item is skipped for an expert without pairs once the routing is
    // known; the items before the first store run whatever their expert
    bool routed = !SPEC;
    if constexpr (SPEC && PREC == kPrecMixed) {
      await_routing();  // the items' precision comes from the routing
      routed = true;
    }
    // (m1) the current item's loads went out without its low plane
    bool lo_pending = kLo && prefetched;
    auto start_item = [&](bool have_loads) -> int {
      for (; item < n_items; item += n_workers) {
        const int u = item / n_stripes;
        const int e = SPEC ? u : s_act[u];
        if (SPEC && routed && !((s_mask[e >> 5] >> (e & 31)) & 1u)) {
          have_loads = false;  // an expert without pairs: nothing to compute
          continue;
        }
        if (!have_loads) {
          set_item(e, item % n_stripes);
          set_precision(e, item_full(e));
          scl_load();
#pragma unroll
          for (int j = 0; j < NB - 1; ++j) load(ItemLo{}, buf[j], j);
          lo_pending = false;
        }
        return e;
      }
      return -1;
    };
    int e = start_item(prefetched);
    while (e >= 0) {
      const int stripe = item % n_stripes, cur_e = e;
      scl_store();  // the item's scales, loaded with its first groups
      f32x4_t tot[RT];
#pragma unroll
      for (int rr = 0; rr < RT; ++rr) tot[rr] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (kLo) {
        if (lo_pending) {  // the prefetched item: its precision, then its low plane
          set_precision(e, item_full(e));
#pragma unroll
          for (int j = 0; j < NB - 1; ++j) load_lo(buf[j], j);
        }
      }
      for (int gc = 0; gc < NU; gc += NB) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          load(ItemLo{}, buf[(j + NB - 1) % NB], gc + j + NB - 1);
          compute(buf[j], gc + j, tot);
        }
      }
      lo_pending = false;
      // the next item's first loads go out before this item's stores
      item += n_workers;
      if (!routed) {
        await_routing();
        routed = true;
      }
      e = start_item(false);
      store_h(tot, cur_e, stripe);
    }
    if (!routed && wave == 0) await_routing();  // the other wavefronts may wait for the table
  }
}

constexpr int kLayerRT = 2, kLayerNB = 4;  // row tiles per item, ring depth in K units (layout v1: groups)
constexpr int kMatLayerNB = 2;             // layout m1: plane tiles of two groups

// Resident workgroups of a kernel (the CU count times its occupancy), cached per
// slot; each translation unit has its own cache, and the slots of one unit name
// distinct kernels.
template <typename Kern>
static int layer_grid(Kern kern, int slot) {
  static int cached[32] = {0};
  if (!cached[slot]) {
    int dev = 0, cus = 0, per_cu = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 512, 0);
    cached[slot] = std::max(1, cus) * std::max(1, per_cu);
  }
  return cached[slot];
}

// every workgroup resident (the launch waits on its own routing): the grid is
// capped at the resident count
template <typename Kern>
static void launch_layer_gateup(Kern kern, int slot, const FfnDev& f, const RouteDev& r, uint16_t* h, int64_t want,
                                hipStream_t s) {
  const int cap = layer_grid(kern, slot);
  hipLaunchKernelGGL(kern, dim3((unsigned)std::min<int64_t>(cap, want)), dim3(512), 0, s, f, r, h);
}

// The routing + gate/up launch of the fused decode layer for format / precision
// PREC: every expert in order (prefetch before routing) when the step routes at
// least one pair per expert on average, else the active experts, each item's K
// units split over 4 or 2 wavefronts when the parts still fit in one round of
// the grid.
template <int PREC>
static void launch_layer_gateup_prec(const FfnDev& f, const RouteDev& r, uint16_t* h, hipStream_t s) {
  constexpr int NB = PREC == kPrecW4 ? kLayerNB : kMatLayerNB;
  constexpr int S0 = 8 * PREC;  // cache slots of this precision
  const bool spec = (int64_t)f.T * f.k >= f.E;
  const int G = f.d / kGroup;
  const int NU = PREC == kPrecW4 ? G : G / 2;  // K units per item
  const int n_stripes = 2 * f.I / (kTileRows * kLayerRT);
  const int64_t items = (int64_t)(spec ? f.E : f.umax) * n_stripes;
  const int64_t logit_wg = ceil_div((int64_t)f.T * f.E, 8);
  const int64_t want = std::max<int64_t>(ceil_div(items, 8), logit_wg);
  if (G <= 16) {
    if (spec) {
      launch_layer_gateup(k_layer_gateup<kLayerRT, NB, 16, true, 1, PREC>, S0 + 0, f, r, h, want, s);
    } else {
      const int cap4 = layer_grid(k_layer_gateup<kLayerRT, NB, 16, false, 4, PREC>, S0 + 4);
      const int cap2 = layer_grid(k_layer_gateup<kLayerRT, NB, 16, false, 2, PREC>, S0 + 5);
      if (NU >= 8 && items * 4 <= (int64_t)cap4 * 8)
        launch_layer_gateup(k_layer_gateup<kLayerRT, NB, 16, false, 4, PREC>, S0 + 4, f, r, h,
                            std::max<int64_t>(ceil_div(items * 4, 8), logit_wg), s);
      else if (NU >= 4 && items * 2 <= (int64_t)cap2 * 8)
        launch_layer_gateup(k_layer_gateup<kLayerRT, NB, 16, false, 2, PREC>, S0 + 5, f, r, h,
                            std::max<int64_t>(ceil_div(items * 2, 8), logit_wg), s);
      else
        launch_layer_gateup(k_layer_gateup<kLayerRT, NB, 16, false, 1, PREC>, S0 + 1, f, r, h, want, s);
    }
  } else {
    if (spec)
      launch_layer_gateup(k_layer_gateup<kLayerRT, NB, 32, true, 1, PREC>, S0 + 2, f, r, h, want, s);
    else
      launch_layer_gateup(k_layer_gateup<kLayerRT, NB, 32, false, 1, PREC>, S0 + 3, f, r, h, want, s);
  }
}

static int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

static int64_t layer_ws_h(int T, int I, int k) { return align256((int64_t)T * k * I * 2); }

// Checks and launches of the fused decode layer, common to both weight formats:
// lay holds the blob size and section offsets of the caller's layout (the codes
// being the high planes in layout m1), tau the four-bit threshold (kPrecMixed),
// name the entry point for error messages.
struct LayerLayout {
  int64_t blob_bytes, w13_codes, w13_scales, w2_codes, w2_scales, w13_lo, w2_lo;
};

template <int PREC>
static int decode_layer_launch(const moe_decode_layer_args* a, const LayerLayout& lay, float tau, const char* name,
                               void* stream) {
  MOE_CHECK_ARG(a->T >= 0 && a->d > 0 && a->I > 0 && a->E > 0 && a->k > 0, MOE_ERR_INVALID_ARG,
                "%s: bad sizes T=%d d=%d I=%d E=%d k=%d", name, a->T, a->d, a->I, a->E, a->k);
  MOE_CHECK_ARG(a->T <= 16 && a->d % kGroup == 0 && a->d <= 32 * kGroup && a->I % kGroup == 0 &&
                    a->E <= MOE_MAX_EXPERTS && a->k <= MOE_MAX_TOPK && a->k <= a->E &&
                    (int64_t)a->T * a->k * a->I * 2 < ((int64_t)1 << 31),
                MOE_ERR_UNSUPPORTED_SHAPE,
                "%s: unsupported shape T=%d d=%d I=%d E=%d k=%d (T <= 16, d <= 4096, d and I "
                "multiples of 128, E <= 1024, k <= min(E,16))",
                name, a->T, a->d, a->I, a->E, a->k);
  if (a->T == 0) return MOE_OK;
  MOE_CHECK_ARG(a->x && a->w_router && a->bank && a->logits && a->topk_ids && a->topk_weights && a->out &&
                    a->workspace && a->counters,
                MOE_ERR_INVALID_ARG, "%s: null pointer", name);
  MOE_CHECK_ARG(a->bank_stride >= lay.blob_bytes && a->bank_stride % 256 == 0 && ((uintptr_t)a->bank % 256) == 0 &&
                    a->bank_stride < ((int64_t)1 << 31),
                MOE_ERR_INVALID_ARG,
                "%s: bank must be 256-byte aligned with stride >= %lld (multiple of 256, below 2^31), got %lld", name,
                (long long)lay.blob_bytes, (long long)a->bank_stride);
  MOE_CHECK_ARG(((uintptr_t)a->x % 16) == 0 && ((uintptr_t)a->w_router % 16) == 0 &&
                    ((uintptr_t)a->workspace % 256) == 0,
                MOE_ERR_INVALID_ARG, "%s: x and w_router must be 16-byte, workspace 256-byte aligned", name);
  const int64_t need = moe_decode_layer_workspace_bytes(a->T, a->d, a->I, a->E, a->k);
  MOE_CHECK_ARG(a->workspace_bytes >= need, MOE_ERR_WORKSPACE, "%s: workspace %lld bytes < %lld needed", name,
                (long long)a->workspace_bytes, (long long)need);
  const int umax = (int)std::min<int64_t>(a->E, (int64_t)a->T * a->k);
  const int dc_stripes = a->d / 32;
  MOE_CHECK_ARG(dc_units_per_wave(umax, a->I / kGroup, dc_stripes) > 0, MOE_ERR_UNSUPPORTED_SHAPE,
                "%s: too many (expert, K slice) items for the down pass (E=%d k=%d I=%d)", name, a->E, a->k, a->I);

  FfnDev f = {};
  f.x = a->x;
  f.T = a->T;
  f.d = a->d;
  f.I = a->I;
  f.E = a->E;
  f.k = a->k;
  f.P = (int64_t)a->T * a->k;
  f.umax = umax;
  f.topk_ids = a->topk_ids;
  f.topk_weights = a->topk_weights;
  f.bank = a->bank;
  f.bank_stride = a->bank_stride;
  f.off_w13_codes = lay.w13_codes;
  f.off_w13_scales = lay.w13_scales;
  f.off_w2_codes = lay.w2_codes;
  f.off_w2_scales = lay.w2_scales;
  f.off_w13_lo = lay.w13_lo;
  f.off_w2_lo = lay.w2_lo;
  f.tau = tau;
  f.zero_ctr = a->counters + kCtrDown;
  f.n_zero_ctr = dc_stripes;

  RouteDev r;
  r.wr = a->w_router;
  r.renormalize = a->renormalize;
  r.tau = PREC == kPrecMixed ? tau : INFINITY;
  r.logits = a->logits;
  r.ids = a->topk_ids;
  r.weights = a->topk_weights;
  r.ctr = a->counters;

  uint8_t* ws = static_cast<uint8_t*>(a->workspace);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws);
  float* dc_part = reinterpret_cast<float*>(ws + layer_ws_h(a->T, a->I, a->k));
  hipStream_t s = (hipStream_t)stream;

  timing_begin(K_GATEUP_DECODE, s);
  launch_layer_gateup_prec<PREC>(f, r, h, s);
  timing_end(K_GATEUP_DECODE, s);
  int rc = check_launch(PREC == kPrecW4 ? "moe_decode_layer (routing + gate/up)" : "moe_mat_decode_layer (routing + gate/up)");
  if (rc) return rc;
  timing_begin(K_DOWN_DECODE, s);
  launch_down_combine_t<PREC>(f, h, a->out, dc_part, a->counters + kCtrDown, a->counters, kCtrRouteEnd, s, true);
  timing_end(K_DOWN_DECODE, s);
  return check_launch(PREC == kPrecW4 ? "moe_decode_layer (down + combine)" : "moe_mat_decode_layer (down + combine)");
}

}  // namespace moe
