// Grouped W4A16 expert kernels for few tokens per expert (decode): the weight
// stream from HBM is the whole cost, so each packed byte is read once, with one
// 16-byte load per lane per 1 KiB tile (ExactMoE, page "Every Expert Counts:
// ExactMoE for Memory-Efficient W4A16 Inference", Abstract: all selected
// experts through fused grouped kernels on four-bit group-128 weights).
//
// Contraction on the matrix cores, weights on the 16-row side of a
// 16x16x32 bf16 MFMA and up to 16 tokens on the other.  A packed word decodes to
// bf16 values 1 + c/16 (c = q + 8) with one rotate and one and-or per pair of
// weights; since sum_k (c_k - 8) x_k = 16 * sum_k (1 + c_k/16) x_k - 24 * sum_k x_k,
// a second MFMA with an all-ones weight operand yields the per-token group sums
// sum_k x_k, and each 128-wide group is finished in fp32 as
//   total += scale * (16 * acc - 24 * xsum).
// The integer weights are exact in bf16, the products exact in fp32, and the
// scale is applied once per group in fp32, so the arithmetic is that of the
// dequantised weights q * scale with fp32 accumulation.
//
// Work split: a block (4 wavefronts) owns one active expert and four adjacent
// stripes of RT packed 16-row tiles, one per wavefront (gate/up: RT/2 gate+up
// tile pairs, so SwiGLU is applied in the wavefront; down: RT*16 output rows).
// Each wavefront runs its stripe over the whole K range of the block's split,
// issuing the loads of up to GPW groups x RT tiles at once before decoding; the
// four share the token block's activations, which each thread stages into LDS
// with one load per group instead of every wavefront loading all of them.  Down
// may further split K over blocks (partials summed in a fixed order by the
// combine kernel).
#include "align_block.hpp"
#include "down_combine.hpp"
#include "ffn_common.hpp"

namespace moe {

// Decode with at most 16 tokens in the step (so at most 16 pairs per expert):
// one 16-column MFMA block covers every pair of an expert.
//
// Persistent workers.  Every wavefront is an independent worker that walks the
// work items (active expert u, stripe of RT 16-row tiles, K split) with a stride
// of the total worker count, so the items in flight at any moment are
// neighbours and the weight stream sweeps memory in order.  A worker owns the
// whole K range of its item (no cross-wavefront reduction, no barrier) and runs
// a two-stage software pipeline over the groups: group j+1's weights (RT tiles),
// scales and activation fragments are in flight while group j is decoded and
// multiplied.  The work item {expert, first position, count} of the next item is
// fetched while the current one streams.
// DENSE (gate/up): the 16 MFMA columns are the step's tokens themselves, so the
// activation addresses need no permutation lookup; columns whose token is not
// routed to the expert read zeros (buffer loads past the end) and store nothing,
// and the SwiGLU row of a routed token goes to its expert-sorted position
// row0 + (rank of the token among the expert's tokens), which is where the
// stable permutation puts it.
template <int RT>
struct GroupBuf {
  u32x4_t c[RT];  // packed codes, one 16-byte slice per tile
  u32x2_t s[RT];  // four bf16 scales per tile (the lane's C rows)
  u32x4_t x[4];   // activation fragments, one per 32-wide K step
};

template <int RT, int NG, bool GATEUP, bool DENSE, bool RING>
__global__ __launch_bounds__(256) void k_decode_persist(FfnDev f, const uint16_t* __restrict__ hin,
                                                        uint16_t* __restrict__ hout, float* __restrict__ y,
                                                        int ksplit) {
  if (GATEUP) zero_down_counters(f);
  const int K = GATEUP ? f.d : f.I;
  const int N = GATEUP ? 2 * f.I : f.d;
  const int G = K / kGroup;
  const int n_stripes = N / (kTileRows * RT);
  const int per_u = n_stripes * ksplit;
  const int n_items = f.umax * per_u;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int col = lane & 15, kq = lane >> 4;
  const int worker = blockIdx.x * 4 + wave, n_workers = gridDim.x * 4;
  const int U = f.active[0];
  const int gs_per = (G + ksplit - 1) / ksplit;

  // the first item's record is in flight while the routing table is staged
  const i32x4_t* work = reinterpret_cast<const i32x4_t*>(f.active + 4);
  int item = worker;
  i32x4_t next_w = work[min(item / per_u, f.umax - 1)];

  // DENSE: the step's routing table (token -> its k experts) staged once in LDS
  __shared__ int s_ids[16][MOE_MAX_TOPK];
  if (DENSE) {
    for (int i = threadIdx.x; i < 16 * MOE_MAX_TOPK; i += 256) {
      const int t = i / MOE_MAX_TOPK, j = i % MOE_MAX_TOPK;
      s_ids[t][j] = (j < f.k && t < f.T) ? f.topk_ids[t * f.k + j] : -1;
    }
    __syncthreads();
  }
  const uint32_t kMask = vgpr_const(0x00780078u), kOne = vgpr_const(0x3F803F80u);
  const u32x4_t ones_w = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const bf16x8_t ones = as_bf16x8(ones_w);
  const uint32_t kNoRow = 0x7F000000u;
  const __amdgpu_buffer_rsrc_t xres =
      GATEUP ? __builtin_amdgcn_make_buffer_rsrc((void*)f.x, (short)0, (int)(f.T * f.d * 2), kBufferRsrcWord3)
             : __builtin_amdgcn_make_buffer_rsrc((void*)hin, (short)0, (int)(f.P * f.I * 2), kBufferRsrcWord3);
  for (; item < n_items; item += n_workers) {
    const int u = item / per_u;
    const int rem = item % per_u;
    const int stripe = rem / ksplit, split = rem % ksplit;
    const i32x4_t w4 = next_w;
    next_w = work[min((item + n_workers) / per_u, f.umax - 1)];  // next item's record, in flight now
    if (u >= U) break;  // items are visited in increasing u: nothing active remains
    const int e = w4[0], row0 = w4[1], n_e = w4[2];
    const uint8_t* blob = f.blob(e);
    if (!blob) continue;
    const int g0 = min(G, split * gs_per), g1 = min(G, g0 + gs_per);

    const uint8_t* codes = blob + (GATEUP ? f.off_w13_codes : f.off_w2_codes) +
                           (int64_t)(RT * stripe) * G * kTileBytes + 16 * lane;
    const uint16_t* scales =
        reinterpret_cast<const uint16_t*>(blob + (GATEUP ? f.off_w13_scales : f.off_w2_scales)) +
        (int64_t)(RT * stripe) * G * kTileRows + 4 * kq;
    const int64_t tile_stride_c = (int64_t)G * kTileBytes;
    const int64_t tile_stride_s = (int64_t)G * kTileRows;

    int out_row;
    bool valid;
    uint32_t xoff;
    if (DENSE) {
      bool routed = false;
      for (int j = 0; j < f.k; ++j) routed |= (s_ids[col][j] == e);
      const uint32_t colmask = (uint32_t)__ballot(routed) & 0xFFFFu;
      valid = routed;
      out_row = row0 + __popc(colmask & ((1u << col) - 1u));
      xoff = routed ? (uint32_t)(col * f.d + 8 * kq) * 2u : kNoRow;
    } else {
      valid = col < n_e;
      out_row = row0 + col;
      xoff = !valid ? kNoRow
                    : (GATEUP ? (uint32_t)((f.sorted_pairs[row0 + col] / f.k) * f.d + 8 * kq) * 2u
                              : (uint32_t)((row0 + col) * f.I + 8 * kq) * 2u);
    }

    f32x4_t tot[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) tot[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Group g's loads; past the item's last group the reads repeat an in-range
    // group and the group's weight (gv) is 0, so no load or compute sits under a
    // branch and the compiler can count exactly which loads to wait for.
    auto load = [&](GroupBuf<RT>& b, int g) {
      const int gl = min(g, G - 1);
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        b.c[r] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(codes + r * tile_stride_c + (int64_t)gl * kTileBytes));
        b.s[r] = *reinterpret_cast<const u32x2_t*>(scales + r * tile_stride_s + gl * kTileRows);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        b.x[i] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xres, xoff + (uint32_t)(gl * kGroup + 32 * i) * 2u, 0, 0));
    };
    auto compute = [&](const GroupBuf<RT>& b, float gv) {
      f32x4_t acc[RT], as = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[r] = as;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8_t xv = as_bf16x8(b.x[i]);
#pragma unroll
        for (int r = 0; r < RT; ++r)
          acc[r] = mfma16x16x32(as_bf16x8(decode_word_biased(b.c[r][i], kMask, kOne)), xv, acc[r]);
        as = mfma16x16x32(ones, xv, as);
      }
      float xs[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) xs[q] = -24.f * as[q];
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const float s4[4] = {__uint_as_float(b.s[r][0] << 16), __uint_as_float(b.s[r][0] & 0xFFFF0000u),
                             __uint_as_float(b.s[r][1] << 16), __uint_as_float(b.s[r][1] & 0xFFFF0000u)};
#pragma unroll
        for (int q = 0; q < 4; ++q) tot[r][q] = fmaf(gv * s4[q], fmaf(16.f, acc[r][q], xs[q]), tot[r][q]);
      }
    };

    if (RING) {
      // ring of NG buffers: the loads of group g + NG - 1 are issued before group g
      // is computed, so NG - 1 groups are in flight behind the one being multiplied
      // (few tokens: little compute per group to hide the memory latency behind)
      GroupBuf<RT> buf[NG];
#pragma unroll
      for (int j = 0; j < NG - 1; ++j) load(buf[j], g0 + j);
      for (int gc = g0; gc < g1; gc += NG) {
#pragma unroll
        for (int j = 0; j < NG; ++j) {
          load(buf[(j + NG - 1) % NG], gc + j + NG - 1);
          compute(buf[j], (gc + j < g1) ? 1.f : 0.f);
        }
      }
    } else {
      // two buffers, restarted every NG groups
      GroupBuf<RT> buf[2];
      for (int gc = g0; gc < g1; gc += NG) {
        load(buf[0], gc);
#pragma unroll
        for (int j = 0; j < NG; ++j) {
          if (j + 1 < NG) load(buf[(j + 1) & 1], gc + j + 1);
          compute(buf[j & 1], (gc + j < g1) ? 1.f : 0.f);
        }
      }
    }

    if (GATEUP) {
#pragma unroll
      for (int p = 0; p < RT / 2; ++p) {
        float hf[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) hf[q] = silu_f32(tot[2 * p][q]) * tot[2 * p + 1][q];
        if (valid) {
          const int hcol = kTileRows * ((RT / 2) * stripe + p) + 4 * kq;
          const u32x2_t o = pack_bf16x4(hf[0], hf[1], hf[2], hf[3]);
          *reinterpret_cast<u32x2_t*>(hout + (int64_t)out_row * f.I + hcol) = o;
        }
      }
    } else {
      float* yout = y + (int64_t)split * f.P * f.d;
      if (valid) {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const int n = kTileRows * (RT * stripe + r) + 4 * kq;
          *reinterpret_cast<f32x4_t*>(yout + (int64_t)out_row * f.d + n) = tot[r];
        }
      }
    }
  }
}

// Grouped gate/up + SwiGLU for steps of at most 16 tokens, the activations shared
// through LDS.  The 16 MFMA columns are the step's tokens (rows past T read as
// zeros), the same for every expert, so a workgroup of 8 wavefronts stages the
// whole activation block once, already in B-fragment order (fragment (g, i) of
// lane l at (4g + i) * 64 + l: one conflict-free 16-byte LDS read per lane), with
// the per-token group sums sum_k x_k that the biased decode needs, formed by the
// same all-ones MFMA as elsewhere.  After that the only global reads are the
// packed weights and their scales: each wavefront is a worker over (expert,
// stripe of RT = 2 tiles = 16 gate rows + the matching 16 up rows) items with a
// ring of NB group loads, so twice as many independent weight streams as 4-tile
// stripes, which the HBM serves at a higher rate.  The first item's weight loads
// are issued before the staging, whose latency they hide.
template <int RT, int NB, int MAXG>
__global__ __launch_bounds__(512, 4) void k_gateup_dense(FfnDev f, uint16_t* __restrict__ hout) {
  zero_down_counters(f);
  constexpr int kWaves = 8;
  const int G = f.d / kGroup;
  const int n_stripes = 2 * f.I / (kTileRows * RT);
  const int n_items = f.umax * n_stripes;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int col = lane & 15, kq = lane >> 4;
  const int worker = blockIdx.x * kWaves + wave, n_workers = gridDim.x * kWaves;
  const i32x4_t* work = reinterpret_cast<const i32x4_t*>(f.active + 4);
  const int U = f.active[0];
  const int64_t tile_stride_c = (int64_t)G * kTileBytes;
  const int64_t tile_stride_s = (int64_t)G * kTileRows;

  struct Buf {
    u32x4_t c[RT];
    u32x2_t s[RT];
  };
  Buf buf[NB];
  const uint8_t* codes = nullptr;
  const uint16_t* scales = nullptr;
  // past the item's last group the loads repeat group G - 1 and the group's
  // weight is 0, so no load sits under a branch and the wait counts stay exact
  auto load = [&](Buf& b, int g) {
    const int gl = min(g, G - 1);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      b.c[r] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(codes + r * tile_stride_c + (int64_t)gl * kTileBytes));
      b.s[r] = *reinterpret_cast<const u32x2_t*>(scales + r * tile_stride_s + gl * kTileRows);
    }
  };
  // Item setup: its record, its weight pointers and the loads of its first NB - 1
  // groups.  Returns the expert (-1: no item left for this worker).
  int item = worker, row0 = 0;
  i32x4_t w4 = work[min(item / n_stripes, f.umax - 1)];
  auto start_item = [&]() -> int {
    for (; item < n_items; item += n_workers) {
      const i32x4_t cur = w4;
      w4 = work[min((item + n_workers) / n_stripes, f.umax - 1)];  // next record, in flight now
      if (item / n_stripes >= U) break;  // items are visited in increasing u: nothing active remains
      const uint8_t* blob = f.blob(cur[0]);
      if (!blob) continue;
      const int stripe = item % n_stripes;
      codes = blob + f.off_w13_codes + (int64_t)(RT * stripe) * G * kTileBytes + 16 * lane;
      scales = reinterpret_cast<const uint16_t*>(blob + f.off_w13_scales) + (int64_t)(RT * stripe) * G * kTileRows +
               4 * kq;
#pragma unroll
      for (int j = 0; j < NB - 1; ++j) load(buf[j], j);
      row0 = cur[1];
      return cur[0];
    }
    item = n_items;
    return -1;
  };
  int e = start_item();

  __shared__ u32x4_t s_x[MAXG * 4 * 64];
  __shared__ float s_xs[MAXG * 16];
  __shared__ int s_ids[16][MOE_MAX_TOPK];
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
    for (int i = threadIdx.x; i < 16 * MOE_MAX_TOPK; i += kWaves * 64) {
      const int t = i / MOE_MAX_TOPK, j = i % MOE_MAX_TOPK;
      s_ids[t][j] = (j < f.k && t < f.T) ? f.topk_ids[t * f.k + j] : -1;
    }
  }
  __syncthreads();
  const uint32_t kMask = vgpr_const(0x00780078u), kOne = vgpr_const(0x3F803F80u);

  while (e >= 0) {
    const int stripe = item % n_stripes;
    bool routed = false;
    for (int j = 0; j < f.k; ++j) routed |= (s_ids[col][j] == e);
    const uint32_t colmask = (uint32_t)__ballot(routed) & 0xFFFFu;
    const int out_row = row0 + __popc(colmask & ((1u << col) - 1u));
    const int cur_stripe = stripe;

    f32x4_t tot[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) tot[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const Buf& b, int g) {
      const int gl = min(g, G - 1);
      const float gv = g < G ? 1.f : 0.f;
      const float xs = -24.f * s_xs[gl * 16 + col];
      f32x4_t acc[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8_t xv = as_bf16x8(s_x[(4 * gl + i) * 64 + lane]);
#pragma unroll
        for (int r = 0; r < RT; ++r)
          acc[r] = mfma16x16x32(as_bf16x8(decode_word_biased(b.c[r][i], kMask, kOne)), xv, acc[r]);
      }
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const float s4[4] = {__uint_as_float(b.s[r][0] << 16), __uint_as_float(b.s[r][0] & 0xFFFF0000u),
                             __uint_as_float(b.s[r][1] << 16), __uint_as_float(b.s[r][1] & 0xFFFF0000u)};
#pragma unroll
        for (int q = 0; q < 4; ++q) tot[r][q] = fmaf(gv * s4[q], fmaf(16.f, acc[r][q], xs), tot[r][q]);
      }
    };
    for (int gc = 0; gc < G; gc += NB) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        load(buf[(j + NB - 1) % NB], gc + j + NB - 1);
        compute(buf[j], gc + j);
      }
    }
    // the next item's first loads go out before this item's stores
    item += n_workers;
    e = start_item();
#pragma unroll
    for (int p = 0; p < RT / 2; ++p) {
      float hf[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hf[q] = silu_f32(tot[2 * p][q]) * tot[2 * p + 1][q];
      if (routed) {
        const int hcol = kTileRows * ((RT / 2) * cur_stripe + p) + 4 * kq;
        const u32x2_t o = pack_bf16x4(hf[0], hf[1], hf[2], hf[3]);
        *reinterpret_cast<u32x2_t*>(hout + (int64_t)out_row * f.I + hcol) = o;
      }
    }
  }
}

// The same gate/up pass with each stripe's K range split over a pair of
// wavefronts of the workgroup, for steps with few active experts (few stripes):
// twice the wavefronts stream weights.  Wavefront w works on stripe slot w % 4 of
// the workgroup's round and K half w / 4; the upper half hands its sums to the
// lower half through LDS (lower + upper, in that order), which applies SwiGLU.
// Rounds are workgroup-uniform (every wavefront meets every barrier).
template <int RT, int NB, int MAXG>
__global__ __launch_bounds__(512, 4) void k_gateup_dense_ks2(FfnDev f, uint16_t* __restrict__ hout) {
  zero_down_counters(f);
  constexpr int kWaves = 8, kSlots = 4;
  const int G = f.d / kGroup;
  const int n_stripes = 2 * f.I / (kTileRows * RT);
  const int n_items = f.umax * n_stripes;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int slot = wave & (kSlots - 1), half = wave >> 2;
  const int col = lane & 15, kq = lane >> 4;
  const int stride_items = gridDim.x * kSlots;
  const i32x4_t* work = reinterpret_cast<const i32x4_t*>(f.active + 4);
  const int U = f.active[0];
  const int64_t tile_stride_c = (int64_t)G * kTileBytes;
  const int64_t tile_stride_s = (int64_t)G * kTileRows;
  const int gh = (G + 1) / 2;
  const int g0 = half ? gh : 0, g1 = half ? G : gh;

  struct Buf {
    u32x4_t c[RT];
    u32x2_t s[RT];
  };
  Buf buf[NB];
  const uint8_t* codes = nullptr;
  const uint16_t* scales = nullptr;
  auto load = [&](Buf& b, int g) {
    const int gl = min(g, g1 - 1);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      b.c[r] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(codes + r * tile_stride_c + (int64_t)gl * kTileBytes));
      b.s[r] = *reinterpret_cast<const u32x2_t*>(scales + r * tile_stride_s + gl * kTileRows);
    }
  };
  // round setup: this wavefront's item, its pointers and its first NB - 1 loads
  int e = -1, row0 = 0, stripe = 0;
  auto setup = [&](int base) {
    const int item = base + slot;
    e = -1;
    if (item < n_items && item / n_stripes < U) {
      const i32x4_t cur = work[item / n_stripes];
      const uint8_t* blob = f.blob(cur[0]);
      if (blob) {
        stripe = item % n_stripes;
        codes = blob + f.off_w13_codes + (int64_t)(RT * stripe) * G * kTileBytes + 16 * lane;
        scales = reinterpret_cast<const uint16_t*>(blob + f.off_w13_scales) + (int64_t)(RT * stripe) * G * kTileRows +
                 4 * kq;
#pragma unroll
        for (int j = 0; j < NB - 1; ++j) load(buf[j], g0 + j);
        e = cur[0];
        row0 = cur[1];
      }
    }
  };
  int base = blockIdx.x * kSlots;
  setup(base);

  __shared__ u32x4_t s_x[MAXG * 4 * 64];
  __shared__ float s_xs[MAXG * 16];
  __shared__ int s_ids[16][MOE_MAX_TOPK];
  __shared__ f32x4_t s_part[kSlots][RT][64];
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
      if (lane < 16) s_xs[g * 16 + lane] = as[0];
    }
    for (int i = threadIdx.x; i < 16 * MOE_MAX_TOPK; i += kWaves * 64) {
      const int t = i / MOE_MAX_TOPK, j = i % MOE_MAX_TOPK;
      s_ids[t][j] = (j < f.k && t < f.T) ? f.topk_ids[t * f.k + j] : -1;
    }
  }
  __syncthreads();
  const uint32_t kMask = vgpr_const(0x00780078u), kOne = vgpr_const(0x3F803F80u);

  // rounds continue while the workgroup's first slot has an active item (items are
  // visited in increasing expert order, so later slots have none either otherwise)
  while (base < n_items && base / n_stripes < U) {
    f32x4_t tot[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) tot[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int cur_e = e, cur_row0 = row0, cur_stripe = stripe;
    if (cur_e >= 0) {
      auto compute = [&](const Buf& b, int g) {
        const int gl = min(g, g1 - 1);
        const float gv = g < g1 ? 1.f : 0.f;
        const float xs = -24.f * s_xs[gl * 16 + col];
        f32x4_t acc[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8_t xv = as_bf16x8(s_x[(4 * gl + i) * 64 + lane]);
#pragma unroll
          for (int r = 0; r < RT; ++r)
            acc[r] = mfma16x16x32(as_bf16x8(decode_word_biased(b.c[r][i], kMask, kOne)), xv, acc[r]);
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const float s4[4] = {__uint_as_float(b.s[r][0] << 16), __uint_as_float(b.s[r][0] & 0xFFFF0000u),
                               __uint_as_float(b.s[r][1] << 16), __uint_as_float(b.s[r][1] & 0xFFFF0000u)};
#pragma unroll
          for (int q = 0; q < 4; ++q) tot[r][q] = fmaf(gv * s4[q], fmaf(16.f, acc[r][q], xs), tot[r][q]);
        }
      };
      for (int gc = g0; gc < g1; gc += NB) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          load(buf[(j + NB - 1) % NB], gc + j + NB - 1);
          compute(buf[j], gc + j);
        }
      }
    }
    base += stride_items;
    setup(base);  // the next round's first loads go out before the hand-over
    if (half == 1 && cur_e >= 0) {
#pragma unroll
      for (int r = 0; r < RT; ++r) s_part[slot][r][lane] = tot[r];
    }
    __syncthreads();
    if (half == 0 && cur_e >= 0) {
      bool routed = false;
      for (int j = 0; j < f.k; ++j) routed |= (s_ids[col][j] == cur_e);
      const uint32_t colmask = (uint32_t)__ballot(routed) & 0xFFFFu;
      const int out_row = cur_row0 + __popc(colmask & ((1u << col) - 1u));
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const f32x4_t o = s_part[slot][r][lane];
#pragma unroll
        for (int q = 0; q < 4; ++q) tot[r][q] = tot[r][q] + o[q];
      }
#pragma unroll
      for (int p = 0; p < RT / 2; ++p) {
        float hf[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) hf[q] = silu_f32(tot[2 * p][q]) * tot[2 * p + 1][q];
        if (routed) {
          const int hcol = kTileRows * ((RT / 2) * cur_stripe + p) + 4 * kq;
          const u32x2_t o = pack_bf16x4(hf[0], hf[1], hf[2], hf[3]);
          *reinterpret_cast<u32x2_t*>(hout + (int64_t)out_row * f.I + hcol) = o;
        }
      }
    }
    __syncthreads();  // s_part is free for the next round
  }
}

// One token block (at most 16 pairs per expert): the wavefronts of a block split
// one stripe's K groups (short chains of loads per wavefront) and add their
// partial sums in LDS in a fixed order; each loads its own activations.  With so
// little arithmetic per group, sharing the activations through LDS costs more in
// barriers than the loads it saves (measured), unlike two token blocks below.
template <int NB, int RT, int GPW, bool GATEUP>
__global__ __launch_bounds__(256) void k_ffn_decode_ksw(FfnDev f, const uint16_t* __restrict__ hin,
                                                    uint16_t* __restrict__ hout, float* __restrict__ y, int ksplit) {
  const int K = GATEUP ? f.d : f.I;
  const int N = GATEUP ? 2 * f.I : f.d;
  const int G = K / kGroup;
  const int n_stripes = N / (kTileRows * RT);
  const int per_u = n_stripes * ksplit;
  const int u = blockIdx.x / per_u;
  const int rem = blockIdx.x % per_u;
  const int stripe = rem / ksplit, split = rem % ksplit;
  // both loads issued together: one round trip before the weight stream starts
  const int U = f.active[0];
  const i32x4_t item = reinterpret_cast<const i32x4_t*>(f.active + 4)[u];  // u < min(E, T*k): in bounds
  if (u >= U) return;
  const int e = item[0], row0 = item[1], n_e = item[2];
  const uint8_t* blob = f.blob(e);
  if (!blob) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int col = lane & 15, kq = lane >> 4;
  const int gs_per = (G + ksplit - 1) / ksplit;
  const int gs0 = min(G, split * gs_per), gs1 = min(G, gs0 + gs_per);
  const int gw_per = (gs1 - gs0 + 3) / 4;
  const int g0 = min(gs1, gs0 + wave * gw_per), g1 = min(gs1, g0 + gw_per);

  const uint8_t* codes = blob + (GATEUP ? f.off_w13_codes : f.off_w2_codes) +
                         (int64_t)(RT * stripe) * G * kTileBytes + 16 * lane;
  // a chunk's scales (RT tiles x GPW groups x 16 rows of bf16) in one 16-byte load
  // per lane: lane c holds half c % 2 of group (c / 2) % GPW of tile c / (2 GPW);
  // they go through the wavefront's LDS area to the lanes that apply them
  static_assert(RT * GPW * 2 <= 64, "a chunk's scales in one load per lane");
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(blob + (GATEUP ? f.off_w13_scales : f.off_w2_scales) + (int64_t)(RT * stripe) * G * kTileRows * 2),
      (short)0, RT * G * kTileRows * 2, kBufferRsrcWord3);
  const int sc_r = lane / (2 * GPW), sc_gi = (lane / 2) % GPW, sc_half = lane & 1;
  __shared__ u32x4_t s_sw[4][64];
  u32x4_t swv;
  const int64_t tile_stride_c = (int64_t)G * kTileBytes;  // bytes between row tiles
  const u32x4_t ones_w = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const bf16x8_t ones = as_bf16x8(ones_w);

  u32x4_t cw[GPW][RT];
  auto load_chunk = [&](int gc) {
    {  // the scales first: waiting for them does not wait for the codes
      const int g = gc + sc_gi;
      const uint32_t off = (sc_r < RT && g < g1) ? (uint32_t)((sc_r * G + g) * kTileRows + 8 * sc_half) * 2u
                                                 : 0x7F000000u;  // else zeros
      swv = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sres, off, 0, 0));
    }
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const int g = gc + gi;
      if (g < g1) {
#pragma unroll
        for (int r = 0; r < RT; ++r)
          cw[gi][r] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4_t*>(codes + r * tile_stride_c + (int64_t)g * kTileBytes));
      }
    }
  };
  load_chunk(g0);

  __shared__ float red[4][RT][NB][4][64];

  for (int tb0 = 0; tb0 < n_e; tb0 += 16 * NB) {
    const uint16_t* arow[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int c = tb0 + 16 * b + col;
      if (c < n_e) {
        arow[b] = GATEUP ? f.x + (int64_t)(f.sorted_pairs[row0 + c] / f.k) * f.d + 8 * kq
                         : hin + (int64_t)(row0 + c) * f.I + 8 * kq;
      } else {
        arow[b] = nullptr;
      }
    }
    f32x4_t tot[RT][NB];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) tot[r][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int gc = g0; gc < g1; gc += GPW) {
      if (gc != g0 || tb0 != 0) load_chunk(gc);
      s_sw[wave][lane] = swv;  // the chunk's scales (the wavefront's LDS ops run in order)
      // activation fragments: with one token block the whole chunk's are issued
      // together (they come from L2); with more blocks, group by group (registers)
      constexpr int XG = (NB == 1) ? GPW : 1;
      u32x4_t xb[XG][NB][4];
      auto load_x = [&](int slot, int g) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            xb[slot][b][i] = (arow[b] && g < g1)
                                 ? *reinterpret_cast<const u32x4_t*>(arow[b] + g * kGroup + 32 * i)
                                 : u32x4_t{0u, 0u, 0u, 0u};
      };
      if constexpr (XG == GPW) {
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) load_x(gi, gc + gi);
      }
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        if (gc + gi >= g1) break;
        const int xs = (XG == GPW) ? gi : 0;
        if constexpr (XG != GPW) load_x(0, gc + gi);
        f32x4_t acc[RT][NB], as[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          as[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = 0; r < RT; ++r) acc[r][b] = as[b];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            const bf16x8_t w = as_bf16x8(decode_word_biased(cw[gi][r][i], 0x00780078u, 0x3F803F80u));
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[r][b] = mfma16x16x32(w, as_bf16x8(xb[xs][b][i]), acc[r][b]);
          }
#pragma unroll
          for (int b = 0; b < NB; ++b) as[b] = mfma16x16x32(ones, as_bf16x8(xb[xs][b][i]), as[b]);
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const u32x2_t sw = reinterpret_cast<const u32x2_t*>(s_sw[wave])[(r * GPW + gi) * 4 + kq];
          const float s4[4] = {bf16_bits_to_f32(sw[0] & 0xFFFFu), bf16_bits_to_f32(sw[0] >> 16),
                               bf16_bits_to_f32(sw[1] & 0xFFFFu), bf16_bits_to_f32(sw[1] >> 16)};
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              tot[r][b][q] = fmaf(s4[q], fmaf(16.f, acc[r][b][q], -24.f * as[b][q]), tot[r][b][q]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[wave][r][b][q][lane] = tot[r][b][q];
    __syncthreads();
    if (GATEUP) {
      for (int combo = wave; combo < (RT / 2) * NB; combo += 4) {
        const int p = combo / NB, b = combo % NB;
        const int c = tb0 + 16 * b + col;
        float hf[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float gsum = 0.f, usum = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            gsum += red[w][2 * p][b][q][lane];
            usum += red[w][2 * p + 1][b][q][lane];
          }
          hf[q] = silu_f32(gsum) * usum;
        }
        if (c < n_e) {
          const int hcol = kTileRows * ((RT / 2) * stripe + p) + 4 * kq;
          const u32x2_t o = pack_bf16x4(hf[0], hf[1], hf[2], hf[3]);
          *reinterpret_cast<u32x2_t*>(hout + (int64_t)(row0 + c) * f.I + hcol) = o;
        }
      }
    } else {
      float* yout = y + (int64_t)split * f.P * f.d;
      for (int combo = wave; combo < RT * NB; combo += 4) {
        const int r = combo / NB, b = combo % NB;
        const int c = tb0 + 16 * b + col;
        f32x4_t o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) v += red[w][r][b][q][lane];
          o[q] = v;
        }
        if (c < n_e) {
          const int n = kTileRows * (RT * stripe + r) + 4 * kq;
          *reinterpret_cast<f32x4_t*>(yout + (int64_t)(row0 + c) * f.d + n) = o;
        }
      }
    }
    __syncthreads();
  }
}

// Two token blocks: a block's wavefronts take four adjacent stripes and share
// the activations through LDS (the work split described at the top of the file).
template <int NB, int RT, int GPW, bool GATEUP>
__global__ __launch_bounds__(256) void k_ffn_decode(FfnDev f, const uint16_t* __restrict__ hin,
                                                    uint16_t* __restrict__ hout, float* __restrict__ y, int ksplit) {
  const int K = GATEUP ? f.d : f.I;
  const int N = GATEUP ? 2 * f.I : f.d;
  const int G = K / kGroup;
  const int n_stripes = N / (kTileRows * RT);
  const int n_quads = (n_stripes + 3) / 4;
  const int per_u = n_quads * ksplit;
  const int u = blockIdx.x / per_u;
  const int rem = blockIdx.x % per_u;
  const int quad = rem / ksplit, split = rem % ksplit;
  // both loads issued together: one round trip before the weight stream starts
  const int U = f.active[0];
  const i32x4_t item = reinterpret_cast<const i32x4_t*>(f.active + 4)[u];  // u < min(E, T*k): in bounds
  if (u >= U) return;  // uniform over the block, as is the next return
  const int e = item[0], row0 = item[1], n_e = item[2];
  const uint8_t* blob = f.blob(e);
  if (!blob) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int col = lane & 15, kq = lane >> 4;
  const int gs_per = (G + ksplit - 1) / ksplit;
  const int g0 = min(G, split * gs_per), g1 = min(G, g0 + gs_per);
  // wavefront w owns stripe 4 quad + w; past the last stripe it still stages the
  // activations and meets the barriers, reading the last stripe's weights (unused)
  const int stripe = quad * 4 + wave;
  const bool has_stripe = stripe < n_stripes;
  const int wstripe = min(stripe, n_stripes - 1);

  const uint8_t* codes = blob + (GATEUP ? f.off_w13_codes : f.off_w2_codes) +
                         (int64_t)(RT * wstripe) * G * kTileBytes + 16 * lane;
  // a chunk's scales (RT tiles x GPW groups x 16 rows of bf16) in one 16-byte load
  // per lane: lane c holds half c % 2 of group (c / 2) % GPW of tile c / (2 GPW);
  // they go through the wavefront's LDS area to the lanes that apply them
  static_assert(RT * GPW * 2 <= 64, "a chunk's scales in one load per lane");
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(blob + (GATEUP ? f.off_w13_scales : f.off_w2_scales) + (int64_t)(RT * wstripe) * G * kTileRows * 2),
      (short)0, RT * G * kTileRows * 2, kBufferRsrcWord3);
  const int sc_r = lane / (2 * GPW), sc_gi = (lane / 2) % GPW, sc_half = lane & 1;
  __shared__ u32x4_t s_sw[4][64];
  u32x4_t swv;
  const int64_t tile_stride_c = (int64_t)G * kTileBytes;  // bytes between row tiles
  const u32x4_t ones_w = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const bf16x8_t ones = as_bf16x8(ones_w);

  u32x4_t cw[GPW][RT];
  auto load_chunk = [&](int gc) {
    {  // the scales first: waiting for them does not wait for the codes
      const int g = gc + sc_gi;
      const uint32_t off = (sc_r < RT && g < g1) ? (uint32_t)((sc_r * G + g) * kTileRows + 8 * sc_half) * 2u
                                                 : 0x7F000000u;  // else zeros
      swv = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sres, off, 0, 0));
    }
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const int g = gc + gi;
      if (g < g1) {
#pragma unroll
        for (int r = 0; r < RT; ++r)
          cw[gi][r] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4_t*>(codes + r * tile_stride_c + (int64_t)g * kTileBytes));
      }
    }
  };

  // The pass's activations, shared by the four wavefronts through a ring of three
  // LDS stages in MFMA fragment order: slot (b * 4 + i) * 64 + l holds the 16 bytes
  // of K step i that lane l of token block b multiplies.  Thread t fills slots
  // t + 256 m (m < NB), one 16-byte load each per group; group g + 1 is staged
  // while group g is multiplied and group g + 2 is in flight, with one barrier per
  // group (a stage is rewritten two groups after its last reader).
  constexpr int kStages = 3;
  __shared__ u32x4_t s_x[kStages][NB * 4 * 64];
  // Per-token activation sums of a group, split by K step: wavefront w sums step w
  // of the group staged one ahead (one MFMA per token block against all-ones
  // weights) and stores it at [stage][16 b + token][w]; each wavefront then adds
  // the four parts instead of every wavefront summing the whole group itself.
  __shared__ f32x4_t s_xs[kStages][NB * 16];
  const int tid = threadIdx.x;
  auto xsum_part = [&](int stage) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      const f32x4_t p = mfma16x16x32(ones, as_bf16x8(s_x[stage][(b * 4 + wave) * 64 + lane]), z);
      if (kq == 0) reinterpret_cast<float*>(&s_xs[stage][16 * b + col])[wave] = p[0];
    }
  };

  for (int tb0 = 0; tb0 < n_e; tb0 += 16 * NB) {
    const uint16_t* xrow[NB];  // this thread's staging source of each slot (null: a padding token)
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      const int sl = tid + 256 * m, b = sl / 256, i = (sl / 64) % 4, l = sl % 64;
      const int c = tb0 + 16 * b + (l & 15);
      const uint16_t* base = nullptr;
      if (c < n_e)
        base = GATEUP ? f.x + (int64_t)(f.sorted_pairs[row0 + c] / f.k) * f.d
                      : hin + (int64_t)(row0 + c) * f.I;
      xrow[m] = base ? base + 32 * i + 8 * (l >> 4) : nullptr;
    }
    u32x4_t xr[2][NB];
    auto xload = [&](u32x4_t* v, int g) {
#pragma unroll
      for (int m = 0; m < NB; ++m)
        v[m] = (xrow[m] && g < g1) ? *reinterpret_cast<const u32x4_t*>(xrow[m] + g * kGroup)
                                   : u32x4_t{0u, 0u, 0u, 0u};
    };
    auto xstage = [&](int stage, const u32x4_t* v) {
#pragma unroll
      for (int m = 0; m < NB; ++m) s_x[stage][tid + 256 * m] = v[m];
    };
    f32x4_t tot[RT][NB];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) tot[r][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // the previous pass is done with every stage
    xload(xr[0], g0);
    xstage(0, xr[0]);
    xload(xr[1], g0 + 1);
    __syncthreads();
    xsum_part(0);
    int j = 0;  // groups done in this pass
    for (int gc = g0; gc < g1; gc += GPW) {
      load_chunk(gc);
      s_sw[wave][lane] = swv;  // the chunk's scales (the wavefront's LDS ops run in order)
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi, ++j) {
        const int g = gc + gi;
        if (g >= g1) break;  // uniform
        xstage((j + 1) % kStages, xr[(j + 1) & 1]);  // group g + 1 (zeros past the range)
        xload(xr[j & 1], g + 2);
        __syncthreads();
        const u32x4_t* st = s_x[j % kStages];
        float xs[NB];  // the group's activation sums (parts stored at the previous group or the prologue)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const f32x4_t v = s_xs[j % kStages][16 * b + col];
          xs[b] = (v[0] + v[1]) + (v[2] + v[3]);
        }
        xsum_part((j + 1) % kStages);  // group g + 1, staged before the barrier above
        f32x4_t acc[RT][NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < RT; ++r) acc[r][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x8_t xv[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) xv[b] = as_bf16x8(st[(b * 4 + i) * 64 + lane]);
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            const bf16x8_t w = as_bf16x8(decode_word_biased(cw[gi][r][i], 0x00780078u, 0x3F803F80u));
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[r][b] = mfma16x16x32(w, xv[b], acc[r][b]);
          }
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const u32x2_t sw = reinterpret_cast<const u32x2_t*>(s_sw[wave])[(r * GPW + gi) * 4 + kq];
          const float s4[4] = {bf16_bits_to_f32(sw[0] & 0xFFFFu), bf16_bits_to_f32(sw[0] >> 16),
                               bf16_bits_to_f32(sw[1] & 0xFFFFu), bf16_bits_to_f32(sw[1] >> 16)};
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              tot[r][b][q] = fmaf(s4[q], fmaf(16.f, acc[r][b][q], -24.f * xs[b]), tot[r][b][q]);
        }
      }
    }
    // the wavefront's stripe over the split's whole K range: SwiGLU and h (gate/up)
    // or the split's fp32 part of the output rows (down)
    if (has_stripe) {
      if (GATEUP) {
#pragma unroll
        for (int p = 0; p < RT / 2; ++p)
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const int c = tb0 + 16 * b + col;
            float hf[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) hf[q] = silu_f32(tot[2 * p][b][q]) * tot[2 * p + 1][b][q];
            if (c < n_e) {
              const int hcol = kTileRows * ((RT / 2) * stripe + p) + 4 * kq;
              const u32x2_t o = pack_bf16x4(hf[0], hf[1], hf[2], hf[3]);
              *reinterpret_cast<u32x2_t*>(hout + (int64_t)(row0 + c) * f.I + hcol) = o;
            }
          }
      } else {
        float* yout = y + (int64_t)split * f.P * f.d;
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const int c = tb0 + 16 * b + col;
            if (c < n_e) {
              const int n = kTileRows * (RT * stripe + r) + 4 * kq;
              *reinterpret_cast<f32x4_t*>(yout + (int64_t)(row0 + c) * f.d + n) = tot[r][b];
            }
          }
      }
    }
  }
}

constexpr int kGateUpRT = 2, kDownRT = 4;
constexpr int kPersistRT = 4, kPersistNG = 8, kRingRT = 2, kRingNG = 4;
constexpr int kDenseRT = 2, kDenseNB = 4;  // LDS-activation gate/up: tiles per stripe, ring depth

int decode_down_gpw(int I, int ksplit, int nb) {
  const int G = I / kGroup;
  const int gs_per = (G + ksplit - 1) / ksplit;
  if (nb <= 1) return (gs_per + 3) / 4 <= 2 ? 2 : 4;  // a quarter of the split per wavefront
  return gs_per <= 8 ? 2 : 4;  // 2: one occupancy step more (fewer registers)
}

// Resident blocks per CU for a kernel, times the CU count (cached per slot).
template <typename Kern>
static int persistent_grid(Kern kern, int slot, int threads = 256) {
  static int cached[16] = {0};
  if (!cached[slot]) {
    int dev = 0, cus = 0, per_cu = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0);
    cached[slot] = std::max(1, cus) * std::max(1, per_cu);
  }
  return cached[slot];
}

template <int NB, int GPW, bool GATEUP>
static void launch_one(const FfnDev& f, const uint16_t* hin, uint16_t* hout, float* y, int ksplit, int64_t grid,
                       hipStream_t s) {
  if constexpr (NB == 1)
    hipLaunchKernelGGL((k_ffn_decode_ksw<1, GATEUP ? 2 : 4, GPW, GATEUP>), dim3((unsigned)grid), dim3(256), 0, s, f,
                       hin, hout, y, ksplit);
  else
    hipLaunchKernelGGL((k_ffn_decode<NB, GATEUP ? 2 : 4, GPW, GATEUP>), dim3((unsigned)grid), dim3(256), 0, s, f,
                       hin, hout, y, ksplit);
}

template <int NB>
static void launch_nb(const FfnDev& f, uint16_t* h, float* y, int ksplit, hipStream_t s, int64_t grid_gu,
                      int64_t grid_dn, int gpw_dn) {
  timing_begin(K_GATEUP_DECODE, s);
  launch_one<NB, 4, true>(f, nullptr, h, nullptr, 1, grid_gu, s);
  timing_end(K_GATEUP_DECODE, s);
  timing_begin(K_DOWN_DECODE, s);
  if (gpw_dn == 2)
    launch_one<NB, 2, false>(f, h, nullptr, y, ksplit, grid_dn, s);
  else
    launch_one<NB, 4, false>(f, h, nullptr, y, ksplit, grid_dn, s);
  timing_end(K_DOWN_DECODE, s);
}

// K groups per wavefront of the fused down + combine pass: the largest of 16, 8,
// 4 (not above G rounded up to a power of two) that still gives at least 2048
// wavefronts, else 4, or 2 when 4 leaves fewer than 2048; 0 if the step has too
// many (expert, slice) items for kDcMaxChunks workgroups per stripe.
int dc_units_per_wave(int umax, int G, int stripes) {
  auto fits = [&](int u) { return (int64_t)umax * ((G + u - 1) / u) <= (int64_t)kDcMaxChunks * kDcWaves; };
  auto waves = [&](int u) { return (int64_t)umax * ((G + u - 1) / u) * stripes; };
  int upw = 4;
  for (int u = 16; u > 4; u /= 2)
    if (u / 2 < G && waves(u) >= 2048) {
      upw = u;
      break;
    }
  if (upw == 4 && waves(4) < 2048 && G > 2 && fits(2)) upw = 2;  // few items: shorter runs, more of them
  return fits(upw) ? upw : 0;
}

void launch_down_combine(const FfnDev& f, const uint16_t* h, uint16_t* out, float* part, int32_t* counters,
                         int32_t* route_ctr, int n_route_ctr, hipStream_t s, bool pair) {
  launch_down_combine_t<kPrecW4>(f, h, out, part, counters, route_ctr, n_route_ctr, s, pair);
}

int launch_decode(const FfnDev& f_in, uint16_t* h, float* y, int ksplit, int nb, hipStream_t s, uint16_t* out,
                  float* dc_part, int32_t* dc_counters) {
  FfnDev f = f_in;
  const int64_t umax = f.umax;
  if (f.T <= 16) {
    const bool fused = out && dc_part && dc_counters;
    const int dc_stripes = f.d / (kTileRows * kDcRT);
    if (fused) {
      f.zero_ctr = dc_counters;
      f.n_zero_ctr = dc_stripes;
    }
    // gate/up: activations in LDS when they fit (d <= 4096), else read per group;
    // down: up to 4 tokens a 4-deep ring of group loads over 2-tile stripes (twice
    // the weight streams), more tokens double buffering over 4-tile stripes (more
    // compute per group covers the latency, and it keeps 3 waves per SIMD)
    const bool ring = f.T <= 4;
    auto kdn = ring ? k_decode_persist<kRingRT, kRingNG, false, false, true>
                    : k_decode_persist<kPersistRT, kPersistNG, false, false, false>;
    const int64_t items_dn = umax * (f.d / (kTileRows * (ring ? kRingRT : kPersistRT))) * ksplit;
    const int64_t grid_dn = std::min<int64_t>(persistent_grid(kdn, ring ? 3 : 1), ceil_div(items_dn, 4));
    timing_begin(K_GATEUP_DECODE, s);
    if (f.d <= 32 * kGroup) {
      const int G = f.d / kGroup;
      // d <= 2048: 2 workgroups per CU and 4 wavefronts per SIMD; d <= 4096: 1 (LDS).
      // Few stripes (at most half the resident wavefronts): K split over wavefront pairs.
      const int64_t items_gu = umax * (2 * f.I / (kTileRows * kDenseRT));
      auto kgu = G <= 16 ? k_gateup_dense<kDenseRT, kDenseNB, 16> : k_gateup_dense<kDenseRT, kDenseNB, 32>;
      const int64_t cap = persistent_grid(kgu, G <= 16 ? 4 : 5, 512);
      if (G >= 2 * kDenseNB && items_gu * 2 <= cap * 8) {
        auto kks = G <= 16 ? k_gateup_dense_ks2<kDenseRT, kDenseNB, 16> : k_gateup_dense_ks2<kDenseRT, kDenseNB, 32>;
        const int64_t grid_ks = std::min<int64_t>(persistent_grid(kks, G <= 16 ? 6 : 7, 512), ceil_div(items_gu, 4));
        hipLaunchKernelGGL(kks, dim3((unsigned)grid_ks), dim3(512), 0, s, f, h);
      } else {
        hipLaunchKernelGGL(kgu, dim3((unsigned)std::min<int64_t>(cap, ceil_div(items_gu, 8))), dim3(512), 0, s, f, h);
      }
    } else {
      auto kgu = ring ? k_decode_persist<kPersistRT, kRingNG, true, true, true>
                      : k_decode_persist<kPersistRT, kPersistNG, true, true, false>;
      const int64_t items_gu = umax * (2 * f.I / (kTileRows * kPersistRT));
      const int64_t grid_gu = std::min<int64_t>(persistent_grid(kgu, ring ? 2 : 0), ceil_div(items_gu, 4));
      hipLaunchKernelGGL(kgu, dim3((unsigned)grid_gu), dim3(256), 0, s, f, (const uint16_t*)nullptr, h,
                         (float*)nullptr, 1);
    }
    timing_end(K_GATEUP_DECODE, s);
    timing_begin(K_DOWN_DECODE, s);
    if (fused) {
      launch_down_combine(f, h, out, dc_part, dc_counters, nullptr, 0, s, false);
    } else {
      hipLaunchKernelGGL(kdn, dim3((unsigned)grid_dn), dim3(256), 0, s, f, (const uint16_t*)h, (uint16_t*)nullptr, y,
                         ksplit);
    }
    timing_end(K_DOWN_DECODE, s);
    return check_launch("grouped expert FFN (decode, T <= 16)");
  }
  // a block per (active expert, stripe[, K split]) with one token block, else
  // per (active expert, four stripes[, K split])
  const int per_block = nb <= 1 ? 1 : 4;
  const int64_t grid_gu = umax * ceil_div(2 * f.I / (kTileRows * kGateUpRT), per_block);
  const int64_t grid_dn = umax * ceil_div(f.d / (kTileRows * kDownRT), per_block) * ksplit;
  const int gpw_dn = decode_down_gpw(f.I, ksplit, nb);
  if (nb <= 1)
    launch_nb<1>(f, h, y, ksplit, s, grid_gu, grid_dn, gpw_dn);
  else
    launch_nb<2>(f, h, y, ksplit, s, grid_gu, grid_dn, gpw_dn);
  return check_launch("grouped expert FFN (decode)");
}

}  // namespace moe
