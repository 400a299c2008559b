// Grouped W4A16 expert GEMMs for many tokens per expert (prefill), MFMA-tiled
// (ExactMoE, page "Every Expert Counts: ExactMoE for Memory-Efficient W4A16
// Inference", Abstract: all selected experts through fused grouped kernels on
// four-bit group-128 weights).
//
// A block computes a 128 (weight rows) x 128 (tokens of one expert) tile with
// four wavefronts of 64 x 64 (4 x 4 blocks of 16x16x32 bf16 MFMA).  Per K group
// of 128: the block stages the tile's 128 activation rows (gathered through the
// permutation) in LDS by LDS-DMA loads (no registers), double-buffered, with an
// XOR swizzle of the 16-byte chunks so the MFMA B-fragment reads are bank-conflict
// free; each wavefront loads its four packed
// weight tiles straight from HBM (one 16-byte load per lane per tile) and decodes
// them in registers to bf16 1 + c/16.  The group is finished in fp32 as
//   total += scale * (16 * acc - 24 * sum_k x)
// with the per-token group sums sum_k x precomputed (activations: a small pass;
// SwiGLU output: written by the gate/up epilogue as two half-group partials).
// Tiles are walked by persistent blocks; the tile list (active expert, row tile,
// token tile) is built per block from the work list of moe_align.
#include "ffn_common.hpp"

namespace moe {

constexpr int kPBM = 128;               // tokens per block tile
constexpr int kPBN = 128;               // weight rows per block tile

// xsum[t][g] = sum of x[t][128 g .. 128 g + 127] in fp32 (one wavefront per token).
__global__ __launch_bounds__(256) void k_group_sums(const uint16_t* __restrict__ x, int T, int d,
                                                    float* __restrict__ xsum) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int G = d / kGroup;
  for (int c0 = 0; c0 < d / 8; c0 += 64) {
    const int ch = c0 + lane;  // 16-byte chunk; a group is 16 chunks
    float s = 0.f;
    if (ch < d / 8) {
      const u32x4_t q = *reinterpret_cast<const u32x4_t*>(x + (int64_t)t * d + 8 * ch);
#pragma unroll
      for (int m = 0; m < 4; ++m) s += __uint_as_float(q[m] << 16) + __uint_as_float(q[m] & 0xFFFF0000u);
    }
    s += __shfl_xor(s, 8);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 1);
    if ((lane & 15) == 0 && ch < d / 8) xsum[(int64_t)t * G + ch / 16] = s;
  }
}

template <bool GATEUP>
__global__ __launch_bounds__(256) void k_prefill(
    FfnDev f, const uint16_t* __restrict__ act, const float* __restrict__ asum, uint16_t* __restrict__ hout,
    float* __restrict__ hsum_out, float* __restrict__ yout) {
  const int K = GATEUP ? f.d : f.I;
  const int N = GATEUP ? 2 * f.I : f.d;
  const int G = K / kGroup;
  const int NT = N / kPBN;
  const int GH = (2 * f.I) / kPBN;  // h-sum partials per pair (two per group of h)

  // activation tile of one K group: 128 tokens x 16 chunks of 16 bytes; chunk kc of
  // token t sits at slot 16 t + (kc ^ (t & 15)), so the 16 tokens of an MFMA
  // B fragment read 16 different 16-byte bank groups
  __shared__ u32x4_t sx[2][kPBM * 16];
  __shared__ int s_row[kPBM];        // activation row (token for gate/up, sorted position for down), -1 = none
  __shared__ int s_pref[MOE_MAX_EXPERTS + 1];
  __shared__ float s_hs[2][kPBM];    // gate/up: per-token h sums of the two row halves
  __shared__ int s_wsum[4];

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave & 1, wt = wave >> 1;  // row half, token half of the block tile
  const int col = lane & 15, kq = lane >> 4;
  const int U = f.active[0];
  const i32x4_t* work = reinterpret_cast<const i32x4_t*>(f.active + 4);

  // tiles of active expert u: ceil(count / 128) token tiles x NT row tiles; exclusive prefix in LDS
  if (tid == 0) s_pref[0] = 0;
  for (int base = 0; base < U; base += 256) {
    __syncthreads();
    const int u = base + tid;
    const int n_e = u < U ? work[u][2] : 0;
    int v = ((n_e + kPBM - 1) / kPBM) * NT;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(v, off);
      if (lane >= off) v += o;
    }
    if (lane == 63) s_wsum[wave] = v;
    __syncthreads();
    int add = s_pref[base];
    for (int w = 0; w < wave; ++w) add += s_wsum[w];
    if (u < U) s_pref[u + 1] = add + v;
  }
  __syncthreads();
  const int total = s_pref[U];

  const uint32_t kMask = vgpr_const(0x00780078u), kOne = vgpr_const(0x3F803F80u);

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    int lo = 0, hi = U;  // s_pref[lo] <= tile < s_pref[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= tile) lo = mid; else hi = mid;
    }
    const int u = lo;
    const i32x4_t w4 = work[u];
    const int e = w4[0], row0 = w4[1], n_e = w4[2];
    const int n_mt = (n_e + kPBM - 1) / kPBM;
    const int local = tile - s_pref[u];
    const int nt = local / n_mt, mt = local % n_mt;
    const uint8_t* blob = f.blob(e);
    if (!blob) continue;  // uniform over the block

    __syncthreads();  // the previous tile is done with s_row / sx / s_hs
    if (tid < kPBM) {
      const int r = mt * kPBM + tid;
      s_row[tid] = r < n_e ? (GATEUP ? f.sorted_pairs[row0 + r] / f.k : row0 + r) : -1;
    }
    __syncthreads();

    const uint8_t* codes = blob + (GATEUP ? f.off_w13_codes : f.off_w2_codes) +
                           (int64_t)(nt * (kPBN / kTileRows) + wr * 4) * G * kTileBytes + 16 * lane;
    const uint16_t* scales =
        reinterpret_cast<const uint16_t*>(blob + (GATEUP ? f.off_w13_scales : f.off_w2_scales)) +
        (int64_t)(nt * (kPBN / kTileRows) + wr * 4) * G * kTileRows + 4 * kq;
    const int64_t tsc = (int64_t)G * kTileBytes, tss = (int64_t)G * kTileRows;

    // staging by LDS DMA: wave w fills slots [w*512, w*512 + 512) of the tile, 64 per
    // instruction; lane l of instruction j fills slot s = w*512 + 64 j + l
    // rows are gathered tokens for gate/up (offsets from x, below 4 GiB by the host
    // check) and consecutive sorted positions for down (offsets from the tile's first row)
    const uint16_t* act_tile = GATEUP ? act : act + (int64_t)(row0 + mt * kPBM) * K;
    uint32_t soff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int slot = wave * 512 + 64 * j + lane;
      const int t = slot >> 4, kc = (slot & 15) ^ (t & 15);
      int row = 0;  // padding tokens read row 0 of the tile (a real row); their outputs are dropped
      if (GATEUP) row = s_row[t] >= 0 ? s_row[t] : s_row[0];
      else row = s_row[t] >= 0 ? t : 0;
      soff[j] = ((uint32_t)row * (uint32_t)K + 8u * (uint32_t)kc) * 2u;  // byte offset of the chunk in group 0
    }
    // per-token group sums of this lane's four token columns
    int xrow[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) xrow[b] = s_row[wt * 64 + b * 16 + col];

    auto stage = [&](int buf, int g) {
      const uint8_t* base = reinterpret_cast<const uint8_t*>(act_tile) + (int64_t)g * kGroup * 2;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t*>(base + soff[j]),
                                         &sx[buf][wave * 512 + 64 * j], 16, 0, 0);
    };
    auto load_sums = [&](float (&xs)[4], int g) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int r = xrow[b];
        float v = 0.f;
        if (r >= 0) v = GATEUP ? asum[(int64_t)r * G + g] : asum[(int64_t)r * GH + 2 * g] + asum[(int64_t)r * GH + 2 * g + 1];
        xs[b] = -24.f * v;
      }
    };
    auto load_w = [&](u32x4_t (&cw)[4], u32x2_t (&sw)[4], int g) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        cw[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(codes + t * tsc + (int64_t)g * kTileBytes));
        sw[t] = *reinterpret_cast<const u32x2_t*>(scales + t * tss + g * kTileRows);
      }
    };

    f32x4_t tot[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) tot[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t cw[4], cwn[4];
    u32x2_t sw[4], swn[4];
    float xs[4], xsn[4];
    load_w(cw, sw, 0);
    load_sums(xs, 0);
    stage(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int g = 0; g < G; ++g) {
      const int buf = g & 1;
      if (g + 1 < G) {
        load_w(cwn, swn, g + 1);
        load_sums(xsn, g + 1);
        stage(buf ^ 1, g + 1);
      }
      f32x4_t acc[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8_t wa[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) wa[t] = as_bf16x8(decode_word_biased(cw[t][i], kMask, kOne));
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int tok = wt * 64 + b * 16 + col;
          const u32x4_t xb = sx[buf][tok * 16 + ((4 * i + kq) ^ (tok & 15))];
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[t][b] = mfma16x16x32(wa[t], as_bf16x8(xb), acc[t][b]);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float s4[4] = {__uint_as_float(sw[t][0] << 16), __uint_as_float(sw[t][0] & 0xFFFF0000u),
                             __uint_as_float(sw[t][1] << 16), __uint_as_float(sw[t][1] & 0xFFFF0000u)};
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) tot[t][b][q] = fmaf(s4[q], fmaf(16.f, acc[t][b][q], xs[b]), tot[t][b][q]);
      }
      if (g + 1 < G) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          cw[t] = cwn[t];
          sw[t] = swn[t];
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) xs[b] = xsn[b];
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the next group's tile has landed in LDS
      __syncthreads();                                   // and every wavefront is done with `buf`
    }

    if (GATEUP) {
      // tiles (0,1) and (2,3) are gate/up pairs: h columns nt*64 + wr*32 + 16p + 4kq + q
      float hs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int r = wt * 64 + b * 16 + col;
        const int pos = row0 + mt * kPBM + r;
        const bool ok = mt * kPBM + r < n_e;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          uint32_t hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            hv[q] = f32_to_bf16_bits(silu_f32(tot[2 * p][b][q]) * tot[2 * p + 1][b][q]);
            hs[b] += __uint_as_float(hv[q] << 16);
          }
          if (ok) {
            const int hcol = nt * 64 + wr * 32 + 16 * p + 4 * kq;
            u32x2_t o = {hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16)};
            *reinterpret_cast<u32x2_t*>(hout + (int64_t)pos * f.I + hcol) = o;
          }
        }
      }
      // per-token sum of this block's 64 h columns: lanes kq = 0..3, then the two row halves
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        hs[b] += __shfl_xor(hs[b], 16);
        hs[b] += __shfl_xor(hs[b], 32);
        if (kq == 0) s_hs[wr][wt * 64 + b * 16 + col] = hs[b];
      }
      __syncthreads();
      if (tid < kPBM) {
        const int r = mt * kPBM + tid;
        if (r < n_e) hsum_out[(int64_t)(row0 + r) * GH + nt] = s_hs[0][tid] + s_hs[1][tid];
      }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int r = wt * 64 + b * 16 + col;
        if (mt * kPBM + r < n_e) {
          const int pos = row0 + mt * kPBM + r;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int n = nt * kPBN + wr * 64 + t * 16 + 4 * kq;
            *reinterpret_cast<f32x4_t*>(yout + (int64_t)pos * f.d + n) = tot[t][b];
          }
        }
      }
    }
  }
}

template <typename Kern>
static int prefill_grid(Kern kern, int slot) {
  static int cached[2] = {0, 0};
  if (!cached[slot]) {
    int dev = 0, cus = 0, per_cu = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0);
    cached[slot] = std::max(1, cus) * std::max(1, per_cu);
  }
  return cached[slot];
}

int64_t prefill_extra_bytes(int T, int d, int I, int k) {
  const int64_t P = (int64_t)T * k;
  return (int64_t)T * (d / kGroup) * 4 + P * ((2 * I) / kPBN) * 4 + 512;
}

int launch_prefill(const FfnDev& f, uint16_t* h, float* y, float* xsum, float* hsum, hipStream_t s) {
  // gate/up gathers token rows by 32-bit byte offsets from x
  if ((int64_t)f.T * f.d * 2 >= (int64_t(1) << 32)) {
    set_error("moe_w4a16_grouped_ffn: prefill needs T * d * 2 < 4 GiB (T=%d d=%d)", f.T, f.d);
    return MOE_ERR_UNSUPPORTED_SHAPE;
  }
  hipLaunchKernelGGL(k_group_sums, dim3((unsigned)ceil_div(f.T, 4)), dim3(256), 0, s, f.x, f.T, f.d, xsum);
  int rc = check_launch("activation group sums");
  if (rc) return rc;
  // upper bound of tiles: sum over experts of ceil(n_e / 128) <= P / 128 + U
  const int64_t mt_bound = f.P / kPBM + f.umax;
  const int64_t tiles_gu = mt_bound * ((2 * f.I) / kPBN);
  const int64_t tiles_dn = mt_bound * (f.d / kPBN);
  auto kgu = k_prefill<true>;
  auto kdn = k_prefill<false>;
  const int64_t grid_gu = std::min<int64_t>(prefill_grid(kgu, 0), tiles_gu);
  const int64_t grid_dn = std::min<int64_t>(prefill_grid(kdn, 1), tiles_dn);
  timing_begin(K_GATEUP_PREFILL, s);
  hipLaunchKernelGGL(kgu, dim3((unsigned)grid_gu), dim3(256), 0, s, f, f.x, (const float*)xsum, h, hsum,
                     (float*)nullptr);
  timing_end(K_GATEUP_PREFILL, s);
  rc = check_launch("grouped gate/up (prefill)");
  if (rc) return rc;
  timing_begin(K_DOWN_PREFILL, s);
  hipLaunchKernelGGL(kdn, dim3((unsigned)grid_dn), dim3(256), 0, s, f, (const uint16_t*)h, (const float*)hsum,
                     (uint16_t*)nullptr, (float*)nullptr, y);
  timing_end(K_DOWN_PREFILL, s);
  return check_launch("grouped down (prefill)");
}

}  // namespace moe
