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
// Work split: a block (4 wavefronts) owns one active expert and one stripe of
// two packed 16-row tiles (gate/up: the gate and up tiles of 16 output columns,
// so SwiGLU is applied in the block; down: 32 output rows).  The wavefronts
// split the expert's K groups; their partial sums meet in LDS in a fixed order.
// Down may further split K over blocks (partials summed by the combine kernel).
#include "ffn_common.hpp"

namespace moe {

template <int NB>
__global__ __launch_bounds__(256) void k_gateup_decode(FfnDev f, uint16_t* __restrict__ h) {
  const int n_stripes = f.I / 16;
  const int u = blockIdx.x / n_stripes;
  const int stripe = blockIdx.x % n_stripes;
  if (u >= f.active[0]) return;
  const int e = f.active[1 + u];
  const uint8_t* blob = f.blob(e);
  if (!blob) return;
  const int row0 = f.offsets[e];
  const int n_e = f.offsets[e + 1] - row0;
  const int G = f.d / kGroup;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int col = lane & 15, kq = lane >> 4;
  const int g_per = (G + 3) / 4;
  const int g0 = min(G, wave * g_per), g1 = min(G, g0 + g_per);

  const uint8_t* codes_g = blob + f.off_w13_codes + (int64_t)(2 * stripe) * G * kTileBytes + 16 * lane;
  const uint8_t* codes_u = codes_g + (int64_t)G * kTileBytes;
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(blob + f.off_w13_scales);
  const uint16_t* sc_g = sc + (int64_t)(2 * stripe) * G * kTileRows + 4 * kq;
  const uint16_t* sc_u = sc_g + (int64_t)G * kTileRows;
  const u32x4_t ones_w = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const bf16x8_t ones = as_bf16x8(ones_w);

  __shared__ float red[4][2][NB][4][64];

  for (int tb0 = 0; tb0 < n_e; tb0 += 16 * NB) {
    const uint16_t* arow[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int c = tb0 + 16 * b + col;
      arow[b] = (c < n_e) ? f.x + (int64_t)(f.sorted_pairs[row0 + c] / f.k) * f.d + 8 * kq : nullptr;
    }
    f32x4_t tg[NB], tu[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      tg[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      tu[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (int g = g0; g < g1; ++g) {
      const u32x4_t cg = *reinterpret_cast<const u32x4_t*>(codes_g + (int64_t)g * kTileBytes);
      const u32x4_t cu = *reinterpret_cast<const u32x4_t*>(codes_u + (int64_t)g * kTileBytes);
      const u32x2_t sg = *reinterpret_cast<const u32x2_t*>(sc_g + g * kTileRows);
      const u32x2_t su = *reinterpret_cast<const u32x2_t*>(sc_u + g * kTileRows);
      u32x4_t xb[NB][4];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xb[b][i] = arow[b] ? *reinterpret_cast<const u32x4_t*>(arow[b] + g * kGroup + 32 * i)
                             : u32x4_t{0u, 0u, 0u, 0u};
      f32x4_t ag[NB], au[NB], as[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        ag[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        au[b] = ag[b];
        as[b] = ag[b];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8_t wg = as_bf16x8(decode_word_biased(cg[i]));
        const bf16x8_t wu = as_bf16x8(decode_word_biased(cu[i]));
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const bf16x8_t xv = as_bf16x8(xb[b][i]);
          ag[b] = mfma16x16x32(wg, xv, ag[b]);
          au[b] = mfma16x16x32(wu, xv, au[b]);
          as[b] = mfma16x16x32(ones, xv, as[b]);
        }
      }
      const float sgr[4] = {bf16_bits_to_f32(sg[0] & 0xFFFFu), bf16_bits_to_f32(sg[0] >> 16),
                            bf16_bits_to_f32(sg[1] & 0xFFFFu), bf16_bits_to_f32(sg[1] >> 16)};
      const float sur[4] = {bf16_bits_to_f32(su[0] & 0xFFFFu), bf16_bits_to_f32(su[0] >> 16),
                            bf16_bits_to_f32(su[1] & 0xFFFFu), bf16_bits_to_f32(su[1] >> 16)};
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float xs = 24.f * as[b][r];
          tg[b][r] = fmaf(sgr[r], fmaf(16.f, ag[b][r], -xs), tg[b][r]);
          tu[b][r] = fmaf(sur[r], fmaf(16.f, au[b][r], -xs), tu[b][r]);
        }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        red[wave][0][b][r][lane] = tg[b][r];
        red[wave][1][b][r][lane] = tu[b][r];
      }
    __syncthreads();
    if (wave < NB) {
      const int b = wave;
      const int c = tb0 + 16 * b + col;
      uint32_t hv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float gsum = 0.f, usum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          gsum += red[w][0][b][r][lane];
          usum += red[w][1][b][r][lane];
        }
        hv[r] = f32_to_bf16_bits(silu_f32(gsum) * usum);
      }
      if (c < n_e) {
        u32x2_t o = {hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16)};
        *reinterpret_cast<u32x2_t*>(h + (int64_t)(row0 + c) * f.I + 16 * stripe + 4 * kq) = o;
      }
    }
    __syncthreads();
  }
}

template <int NB>
__global__ __launch_bounds__(256) void k_down_decode(FfnDev f, const uint16_t* __restrict__ h, float* __restrict__ y,
                                                     int ksplit) {
  const int n_stripes = f.d / 32;
  const int per_u = n_stripes * ksplit;
  const int u = blockIdx.x / per_u;
  const int rem = blockIdx.x % per_u;
  const int stripe = rem / ksplit, split = rem % ksplit;
  if (u >= f.active[0]) return;
  const int e = f.active[1 + u];
  const uint8_t* blob = f.blob(e);
  if (!blob) return;
  const int row0 = f.offsets[e];
  const int n_e = f.offsets[e + 1] - row0;
  const int G = f.I / kGroup;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int col = lane & 15, kq = lane >> 4;
  // groups of this block, then of this wavefront
  const int gs_per = (G + ksplit - 1) / ksplit;
  const int gs0 = min(G, split * gs_per), gs1 = min(G, gs0 + gs_per);
  const int g_per = (gs1 - gs0 + 3) / 4;
  const int g0 = min(gs1, gs0 + wave * g_per), g1 = min(gs1, g0 + g_per);

  const uint8_t* codes0 = blob + f.off_w2_codes + (int64_t)(2 * stripe) * G * kTileBytes + 16 * lane;
  const uint8_t* codes1 = codes0 + (int64_t)G * kTileBytes;
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(blob + f.off_w2_scales);
  const uint16_t* sc0 = sc + (int64_t)(2 * stripe) * G * kTileRows + 4 * kq;
  const uint16_t* sc1 = sc0 + (int64_t)G * kTileRows;
  const u32x4_t ones_w = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const bf16x8_t ones = as_bf16x8(ones_w);
  float* yout = y + (int64_t)split * f.P * f.d;

  __shared__ float red[4][2][NB][4][64];

  for (int tb0 = 0; tb0 < n_e; tb0 += 16 * NB) {
    const uint16_t* arow[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int c = tb0 + 16 * b + col;
      arow[b] = (c < n_e) ? h + (int64_t)(row0 + c) * f.I + 8 * kq : nullptr;
    }
    f32x4_t t0[NB], t1[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      t0[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      t1[b] = t0[b];
    }
    for (int g = g0; g < g1; ++g) {
      const u32x4_t c0 = *reinterpret_cast<const u32x4_t*>(codes0 + (int64_t)g * kTileBytes);
      const u32x4_t c1 = *reinterpret_cast<const u32x4_t*>(codes1 + (int64_t)g * kTileBytes);
      const u32x2_t s0 = *reinterpret_cast<const u32x2_t*>(sc0 + g * kTileRows);
      const u32x2_t s1 = *reinterpret_cast<const u32x2_t*>(sc1 + g * kTileRows);
      u32x4_t xb[NB][4];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xb[b][i] = arow[b] ? *reinterpret_cast<const u32x4_t*>(arow[b] + g * kGroup + 32 * i)
                             : u32x4_t{0u, 0u, 0u, 0u};
      f32x4_t a0[NB], a1[NB], as[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        a0[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        a1[b] = a0[b];
        as[b] = a0[b];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8_t w0 = as_bf16x8(decode_word_biased(c0[i]));
        const bf16x8_t w1 = as_bf16x8(decode_word_biased(c1[i]));
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const bf16x8_t xv = as_bf16x8(xb[b][i]);
          a0[b] = mfma16x16x32(w0, xv, a0[b]);
          a1[b] = mfma16x16x32(w1, xv, a1[b]);
          as[b] = mfma16x16x32(ones, xv, as[b]);
        }
      }
      const float s0r[4] = {bf16_bits_to_f32(s0[0] & 0xFFFFu), bf16_bits_to_f32(s0[0] >> 16),
                            bf16_bits_to_f32(s0[1] & 0xFFFFu), bf16_bits_to_f32(s0[1] >> 16)};
      const float s1r[4] = {bf16_bits_to_f32(s1[0] & 0xFFFFu), bf16_bits_to_f32(s1[0] >> 16),
                            bf16_bits_to_f32(s1[1] & 0xFFFFu), bf16_bits_to_f32(s1[1] >> 16)};
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float xs = 24.f * as[b][r];
          t0[b][r] = fmaf(s0r[r], fmaf(16.f, a0[b][r], -xs), t0[b][r]);
          t1[b][r] = fmaf(s1r[r], fmaf(16.f, a1[b][r], -xs), t1[b][r]);
        }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        red[wave][0][b][r][lane] = t0[b][r];
        red[wave][1][b][r][lane] = t1[b][r];
      }
    __syncthreads();
    if (wave < NB) {
      const int b = wave;
      const int c = tb0 + 16 * b + col;
      f32x4_t o0, o1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v0 = 0.f, v1 = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          v0 += red[w][0][b][r][lane];
          v1 += red[w][1][b][r][lane];
        }
        o0[r] = v0;
        o1[r] = v1;
      }
      if (c < n_e) {
        float* dst = yout + (int64_t)(row0 + c) * f.d + 32 * stripe + 4 * kq;
        *reinterpret_cast<f32x4_t*>(dst) = o0;
        *reinterpret_cast<f32x4_t*>(dst + 16) = o1;
      }
    }
    __syncthreads();
  }
}

int launch_decode(const FfnDev& f, uint16_t* h, float* y, int ksplit, int nb, hipStream_t s) {
  const int64_t umax = f.umax;
  const int64_t grid_gu = umax * (f.I / 16);
  const int64_t grid_dn = umax * (f.d / 32) * ksplit;
  timing_begin(K_GATEUP_DECODE, s);
  if (nb <= 1)
    hipLaunchKernelGGL(k_gateup_decode<1>, dim3((unsigned)grid_gu), dim3(256), 0, s, f, h);
  else
    hipLaunchKernelGGL(k_gateup_decode<2>, dim3((unsigned)grid_gu), dim3(256), 0, s, f, h);
  timing_end(K_GATEUP_DECODE, s);
  int rc = check_launch("grouped gate/up (decode)");
  if (rc) return rc;
  timing_begin(K_DOWN_DECODE, s);
  if (nb <= 1)
    hipLaunchKernelGGL(k_down_decode<1>, dim3((unsigned)grid_dn), dim3(256), 0, s, f, h, y, ksplit);
  else
    hipLaunchKernelGGL(k_down_decode<2>, dim3((unsigned)grid_dn), dim3(256), 0, s, f, h, y, ksplit);
  timing_end(K_DOWN_DECODE, s);
  return check_launch("grouped down (decode)");
}

}  // namespace moe
