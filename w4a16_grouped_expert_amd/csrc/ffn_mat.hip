#include "ffn_common.hpp"
#include "mat_format.hpp"

namespace moe {

constexpr int kMatRT = 2;     // row tiles per stripe (gate/up: 16 gate + 16 up rows; down: 32 rows)
constexpr int kMatNB = 3;     // ring depth (plane tiles of two groups in flight)

// Two v1 tiles (one row tile, groups 2kb and 2kb + 1) -> one plane tile per plane.
// Code of element m of v1 word i: field at (3 + 4 (m/2) + 16 (m%2)) mod 32.
__global__ __launch_bounds__(256) void k_mat_convert(const uint8_t* __restrict__ src, int64_t src_stride,
                                                     uint8_t* __restrict__ dst, int64_t dst_stride, int E,
                                                     int64_t ptiles13, int64_t ptiles2, int64_t off_c13,
                                                     int64_t off_c2, MatOffsets mo) {
  const int lane = lane_id();
  const int64_t per_e = ptiles13 + ptiles2;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= per_e * E) return;
  const int e = (int)(gw / per_e);
  const int64_t t = gw % per_e;
  const bool w13 = t < ptiles13;
  const int64_t pt = w13 ? t : t - ptiles13;  // plane tile = v1 tiles 2 pt, 2 pt + 1 (same row tile)
  const uint8_t* s = src + e * src_stride + (w13 ? off_c13 : off_c2) + 2 * pt * kTileBytes + 16 * lane;
  uint32_t hi[4] = {0u, 0u, 0u, 0u}, lo[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const u32x4_t words = *reinterpret_cast<const u32x4_t*>(s + half * kTileBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = __builtin_amdgcn_alignbit(words[i], words[i], 3);  // undo the rotation by 3
      const int step = 4 * half + i, j = step >> 1, tt = step & 1;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t c = (u >> (4 * (m >> 1) + 16 * (m & 1))) & 0xFu;
        const int sh = 2 * (4 * tt + (m >> 1)) + 16 * (m & 1);
        hi[j] |= (c >> 2) << sh;
        lo[j] |= (c & 3u) << sh;
      }
    }
  }
  uint8_t* d = dst + e * dst_stride;
  const int64_t po = pt * kPlaneTileBytes + 16 * lane;
  u32x4_t h4, l4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h4[j] = (hi[j] << 5) | (hi[j] >> 27);
    l4[j] = (lo[j] << 5) | (lo[j] >> 27);
  }
  *reinterpret_cast<u32x4_t*>(d + (w13 ? mo.hi13 : mo.hi2) + po) = h4;
  *reinterpret_cast<u32x4_t*>(d + (w13 ? mo.lo13 : mo.lo2) + po) = l4;
}

// Loads and products of one stripe of RT plane row tiles over plane tiles
// [p0, p1) (two groups each), accumulated into tot; the activation fragment of
// group g, K step i comes from xfrag(g, i), the group's sum of x from xsum(g).
template <bool FULL, int RT, int NB, typename XF, typename XS>
__device__ __forceinline__ void mat_stripe(const uint8_t* hip, const uint8_t* lop, const uint16_t* scales,
                                           int64_t tile_stride_p, int64_t tile_stride_s, int P2, int p0, int p1,
                                           XF xfrag, XS xsum, f32x4_t (&tot)[RT]) {
  struct Buf {
    u32x4_t h[RT], l[RT];
    u32x2_t s[RT][2];
  };
  // past the last plane tile the loads repeat tile p1 - 1 and are not used
  auto load = [&](Buf& b, int pt) {
    const int pl = min(pt, p1 - 1);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      b.h[r] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(hip + r * tile_stride_p + (int64_t)pl * kPlaneTileBytes));
      if (FULL)
        b.l[r] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(lop + r * tile_stride_p + (int64_t)pl * kPlaneTileBytes));
#pragma unroll
      for (int hg = 0; hg < 2; ++hg)
        b.s[r][hg] = *reinterpret_cast<const u32x2_t*>(scales + r * tile_stride_s + (2 * pl + hg) * kTileRows);
    }
  };
  auto compute = [&](const Buf& b, int pt) {
    const float gv = pt < p1 ? 1.f : 0.f;
    const int pl = min(pt, p1 - 1);
#pragma unroll
    for (int hg = 0; hg < 2; ++hg) {
      const int g = 2 * pl + hg;
      f32x4_t acc[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8_t xv = as_bf16x8(xfrag(g, i));
        const int step = 4 * hg + i;
#pragma unroll
        for (int r = 0; r < RT; ++r)
          acc[r] = mfma16x16x32(
              as_bf16x8(decode_step<FULL>(b.h[r][step >> 1], FULL ? b.l[r][step >> 1] : 0u, step & 1)), xv, acc[r]);
      }
      const f32x4_t xs4 = xsum(g);
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const u32x2_t sw = b.s[r][hg];
        const float s4[4] = {__uint_as_float(sw[0] << 16), __uint_as_float(sw[0] & 0xFFFF0000u),
                             __uint_as_float(sw[1] << 16), __uint_as_float(sw[1] & 0xFFFF0000u)};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          tot[r][q] = fmaf(gv * s4[q], fmaf(16.f, acc[r][q], (FULL ? -24.f : -22.5f) * xs4[q]), tot[r][q]);
      }
    }
  };
  (void)P2;
  Buf buf[NB];
#pragma unroll
  for (int j = 0; j < NB - 1; ++j) load(buf[j], p0 + j);
  for (int pc = p0; pc < p1; pc += NB) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      load(buf[(j + NB - 1) % NB], pc + j + NB - 1);
      compute(buf[j], pc + j);
    }
  }
}

// Gate/up + SwiGLU for steps of at most 16 tokens, activations shared through LDS
// as in the four-bit kernel; per item the expert's precision decides whether the
// low plane is read.
template <int MAXG>
__global__ __launch_bounds__(512, 4) void k_mat_gateup(FfnDev f, MatOffsets mo, float tau,
                                                       uint16_t* __restrict__ hout) {
  constexpr int kWaves = 8, RT = kMatRT, NB = kMatNB;
  const int G = f.d / kGroup, P2 = f.d / kPlaneK;
  const int n_stripes = 2 * f.I / (kTileRows * RT);
  const int n_items = f.umax * n_stripes;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int col = lane & 15, kq = lane >> 4;
  const int worker = blockIdx.x * kWaves + wave, n_workers = gridDim.x * kWaves;
  const i32x4_t* work = reinterpret_cast<const i32x4_t*>(f.active + 4);
  const int U = f.active[0];

  __shared__ u32x4_t s_x[MAXG * 4 * 64];
  __shared__ float s_xs[MAXG * 16];
  __shared__ int s_ids[16][MOE_MAX_TOPK];
  __shared__ float s_w[16][MOE_MAX_TOPK];
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
      const bool in = j < f.k && t < f.T;
      s_ids[t][j] = in ? f.topk_ids[t * f.k + j] : -1;
      s_w[t][j] = in ? f.topk_weights[t * f.k + j] : 0.f;
    }
  }
  __syncthreads();
  const int64_t tile_stride_p = (int64_t)P2 * kPlaneTileBytes;
  const int64_t tile_stride_s = (int64_t)G * kTileRows;
  auto xfrag = [&](int g, int i) { return s_x[(4 * g + i) * 64 + lane]; };
  auto xsum = [&](int g) {
    const float v = s_xs[g * 16 + col];
    return f32x4_t{v, v, v, v};
  };

  for (int item = worker; item < n_items; item += n_workers) {
    const int u = item / n_stripes, stripe = item % n_stripes;
    if (u >= U) break;
    const i32x4_t w4 = work[u];
    const int e = w4[0], row0 = w4[1];
    const uint8_t* blob = f.blob(e);
    if (!blob) continue;
    bool routed = false, heavy = false;
    for (int j = 0; j < f.k; ++j) {
      const bool hit = s_ids[col][j] == e;
      routed |= hit;
      heavy |= hit && s_w[col][j] >= tau;
    }
    const uint32_t colmask = (uint32_t)__ballot(routed) & 0xFFFFu;
    const bool full = __ballot(heavy) != 0;  // four bits when any of the expert's pairs reaches tau
    const int out_row = row0 + __popc(colmask & ((1u << col) - 1u));
    const int64_t poff = (int64_t)(RT * stripe) * P2 * kPlaneTileBytes + 16 * lane;
    const uint8_t* hip = blob + mo.hi13 + poff;
    const uint8_t* lop = blob + mo.lo13 + poff;
    const uint16_t* scales =
        reinterpret_cast<const uint16_t*>(blob + mo.sc13) + (int64_t)(RT * stripe) * G * kTileRows + 4 * kq;
    f32x4_t tot[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) tot[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (full)
      mat_stripe<true, RT, NB>(hip, lop, scales, tile_stride_p, tile_stride_s, P2, 0, P2, xfrag, xsum, tot);
    else
      mat_stripe<false, RT, NB>(hip, lop, scales, tile_stride_p, tile_stride_s, P2, 0, P2, xfrag, xsum, tot);
    float hf[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) hf[q] = silu_f32(tot[0][q]) * tot[1][q];
    if (routed) {
      const int hcol = kTileRows * stripe + 4 * kq;
      const u32x2_t o = pack_bf16x4(hf[0], hf[1], hf[2], hf[3]);
      *reinterpret_cast<u32x2_t*>(hout + (int64_t)out_row * f.I + hcol) = o;
    }
  }
}

// Down for steps of at most 16 tokens: each wavefront owns (expert, 32 output rows,
// K split) items; the expert's h rows are read per group (buffer loads, rows past
// the expert's pairs read zeros) and X by the all-ones MFMA.
__global__ __launch_bounds__(256) void k_mat_down(FfnDev f, MatOffsets mo, float tau,
                                                  const uint16_t* __restrict__ hin, float* __restrict__ y,
                                                  int ksplit) {
  constexpr int RT = kMatRT, NB = kMatNB;
  const int G = f.I / kGroup, P2 = f.I / kPlaneK;
  const int n_stripes = f.d / (kTileRows * RT);
  const int per_u = n_stripes * ksplit;
  const int n_items = f.umax * per_u;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int col = lane & 15, kq = lane >> 4;
  const int worker = blockIdx.x * 4 + wave, n_workers = gridDim.x * 4;
  const int U = f.active[0];
  const int ps_per = (P2 + ksplit - 1) / ksplit;
  const u32x4_t ones_w = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const bf16x8_t ones = as_bf16x8(ones_w);
  const uint32_t kNoRow = 0x7F000000u;
  const __amdgpu_buffer_rsrc_t hres =
      __builtin_amdgcn_make_buffer_rsrc((void*)hin, (short)0, (int)(f.P * f.I * 2), kBufferRsrcWord3);
  const i32x4_t* work = reinterpret_cast<const i32x4_t*>(f.active + 4);
  const int64_t tile_stride_p = (int64_t)P2 * kPlaneTileBytes;
  const int64_t tile_stride_s = (int64_t)G * kTileRows;

  for (int item = worker; item < n_items; item += n_workers) {
    const int u = item / per_u;
    if (u >= U) break;
    const int rem = item % per_u;
    const int stripe = rem / ksplit, split = rem % ksplit;
    const i32x4_t w4 = work[u];
    const int e = w4[0], row0 = w4[1], n_e = w4[2];
    const uint8_t* blob = f.blob(e);
    if (!blob) continue;
    const bool valid = col < n_e;
    const float wcol = valid ? f.topk_weights[f.sorted_pairs[row0 + col]] : 0.f;
    const bool full = __ballot(valid && wcol >= tau) != 0;
    const uint32_t xoff = valid ? (uint32_t)((row0 + col) * f.I + 8 * kq) * 2u : kNoRow;
    // an empty K range (ksplit does not divide the plane tiles evenly) still writes its zero partials
    const int p0 = min(P2, split * ps_per), p1 = min(P2, p0 + ps_per);
    const int64_t poff = (int64_t)(RT * stripe) * P2 * kPlaneTileBytes + 16 * lane;
    const uint8_t* hip = blob + mo.hi2 + poff;
    const uint8_t* lop = blob + mo.lo2 + poff;
    const uint16_t* scales =
        reinterpret_cast<const uint16_t*>(blob + mo.sc2) + (int64_t)(RT * stripe) * G * kTileRows + 4 * kq;
    auto xfrag = [&](int g, int i) {
      return __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(hres, xoff + (uint32_t)(g * kGroup + 32 * i) * 2u, 0, 0));
    };
    auto xsum = [&](int g) {
      f32x4_t as = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) as = mfma16x16x32(ones, as_bf16x8(xfrag(g, i)), as);
      return as;
    };
    f32x4_t tot[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) tot[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (full)
      mat_stripe<true, RT, NB>(hip, lop, scales, tile_stride_p, tile_stride_s, P2, p0, p1, xfrag, xsum, tot);
    else
      mat_stripe<false, RT, NB>(hip, lop, scales, tile_stride_p, tile_stride_s, P2, p0, p1, xfrag, xsum, tot);
    if (valid) {
      float* yout = y + (int64_t)split * f.P * f.d + (int64_t)(row0 + col) * f.d;
#pragma unroll
      for (int r = 0; r < RT; ++r)
        *reinterpret_cast<f32x4_t*>(yout + kTileRows * (RT * stripe + r) + 4 * kq) = tot[r];
    }
  }
}

template <typename Kern>
static int mat_grid(Kern kern, int slot, int threads) {
  static int cached[4] = {0};
  if (!cached[slot]) {
    int dev = 0, cus = 0, per_cu = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0);
    cached[slot] = std::max(1, cus) * std::max(1, per_cu);
  }
  return cached[slot];
}

}  // namespace moe

using namespace moe;

extern "C" int moe_mat_layout_get(int d, int I, moe_mat_layout* out) {
  clear_error();
  MOE_CHECK_ARG(out != nullptr, MOE_ERR_INVALID_ARG, "moe_mat_layout_get: out is NULL");
  MOE_CHECK_ARG(d > 0 && I > 0, MOE_ERR_INVALID_ARG, "moe_mat_layout_get: d=%d I=%d", d, I);
  MOE_CHECK_ARG(d % kPlaneK == 0 && I % kPlaneK == 0, MOE_ERR_UNSUPPORTED_SHAPE,
                "moe_mat_layout_get: d=%d and I=%d must be multiples of 256", d, I);
  const MatOffsets m = mat_offsets(d, I);
  out->w13_hi = m.hi13;
  out->w13_lo = m.lo13;
  out->w13_scales = m.sc13;
  out->w2_hi = m.hi2;
  out->w2_lo = m.lo2;
  out->w2_scales = m.sc2;
  out->blob_bytes = (m.lo2 + (int64_t)d * I / 4 + 255) / 256 * 256;
  out->two_bit_bytes = m.lo13;
  return MOE_OK;
}

extern "C" int moe_mat_from_w4(const uint8_t* w4_bank, int64_t w4_stride, int E, int d, int I, uint8_t* mat_bank,
                               int64_t mat_stride, void* stream) {
  clear_error();
  MOE_CHECK_ARG(E > 0 && w4_bank && mat_bank, MOE_ERR_INVALID_ARG, "moe_mat_from_w4: bad arguments");
  moe_expert_layout v1;
  int rc = moe_expert_layout_get(d, I, &v1);
  if (rc) return rc;
  moe_mat_layout ml;
  rc = moe_mat_layout_get(d, I, &ml);
  if (rc) return rc;
  MOE_CHECK_ARG(w4_stride >= v1.blob_bytes && mat_stride >= ml.blob_bytes && w4_stride % 16 == 0 &&
                    mat_stride % 16 == 0 && ((uintptr_t)w4_bank % 16) == 0 && ((uintptr_t)mat_bank % 16) == 0,
                MOE_ERR_INVALID_ARG, "moe_mat_from_w4: strides %lld / %lld below the blob sizes or misaligned",
                (long long)w4_stride, (long long)mat_stride);
  hipStream_t s = (hipStream_t)stream;
  const int64_t ptiles13 = (int64_t)(2 * I / kTileRows) * (d / kPlaneK);
  const int64_t ptiles2 = (int64_t)(d / kTileRows) * (I / kPlaneK);
  const MatOffsets mo = mat_offsets(d, I);
  const int64_t waves = (ptiles13 + ptiles2) * E;
  hipLaunchKernelGGL(k_mat_convert, dim3((unsigned)ceil_div(waves, 4)), dim3(256), 0, s, w4_bank, w4_stride, mat_bank,
                     mat_stride, E, ptiles13, ptiles2, (int64_t)v1.w13_codes, (int64_t)v1.w2_codes, mo);
  rc = check_launch("moe_mat_from_w4");
  if (rc) return rc;
  // the scales are the same arrays
  const int64_t sc13 = (int64_t)2 * I * (d / kGroup) * 2, sc2 = (int64_t)d * (I / kGroup) * 2;
  hipError_t e1 = hipMemcpy2DAsync(mat_bank + mo.sc13, (size_t)mat_stride, w4_bank + v1.w13_scales, (size_t)w4_stride,
                                   (size_t)sc13, (size_t)E, hipMemcpyDeviceToDevice, s);
  hipError_t e2 = hipMemcpy2DAsync(mat_bank + mo.sc2, (size_t)mat_stride, w4_bank + v1.w2_scales, (size_t)w4_stride,
                                   (size_t)sc2, (size_t)E, hipMemcpyDeviceToDevice, s);
  MOE_CHECK_ARG(e1 == hipSuccess && e2 == hipSuccess, MOE_ERR_HIP, "moe_mat_from_w4: scale copy failed: %s",
                hipGetErrorString(e1 != hipSuccess ? e1 : e2));
  return MOE_OK;
}

extern "C" int moe_mat_grouped_ffn(const moe_ffn_args* a, float tau, void* stream) {
  clear_error();
  MOE_CHECK_ARG(a != nullptr, MOE_ERR_INVALID_ARG, "moe_mat_grouped_ffn: args is NULL");
  MOE_CHECK_ARG(a->T >= 0 && a->d > 0 && a->I > 0 && a->E > 0 && a->k > 0, MOE_ERR_INVALID_ARG,
                "moe_mat_grouped_ffn: bad sizes T=%d d=%d I=%d E=%d k=%d", a->T, a->d, a->I, a->E, a->k);
  MOE_CHECK_ARG(a->d % kPlaneK == 0 && a->I % kPlaneK == 0 && a->d <= 32 * kGroup && a->T <= 16 &&
                    a->E <= MOE_MAX_EXPERTS && a->k <= MOE_MAX_TOPK && a->k <= a->E,
                MOE_ERR_UNSUPPORTED_SHAPE,
                "moe_mat_grouped_ffn: unsupported shape T=%d d=%d I=%d E=%d k=%d (T <= 16, d <= 4096, d and I "
                "multiples of 256, k <= min(E,16))",
                a->T, a->d, a->I, a->E, a->k);
  if (a->T == 0) return MOE_OK;
  MOE_CHECK_ARG(a->x && a->topk_ids && a->topk_weights && a->sorted_pairs && a->pair_pos && a->active_experts &&
                    a->bank && a->workspace,
                MOE_ERR_INVALID_ARG, "moe_mat_grouped_ffn: null pointer");
  MOE_CHECK_ARG(!a->combine || a->out, MOE_ERR_INVALID_ARG, "moe_mat_grouped_ffn: combine needs out");
  moe_mat_layout ml;
  int rc = moe_mat_layout_get(a->d, a->I, &ml);
  if (rc) return rc;
  MOE_CHECK_ARG(a->bank_stride >= ml.blob_bytes && a->bank_stride % 256 == 0 && ((uintptr_t)a->bank % 256) == 0,
                MOE_ERR_INVALID_ARG,
                "moe_mat_grouped_ffn: bank must be 256-byte aligned with stride >= %lld (multiple of 256), got %lld",
                (long long)ml.blob_bytes, (long long)a->bank_stride);
  MOE_CHECK_ARG(((uintptr_t)a->x % 16) == 0 && ((uintptr_t)a->workspace % 256) == 0 &&
                    ((uintptr_t)a->active_experts % 16) == 0 && (!a->out || ((uintptr_t)a->out % 8) == 0),
                MOE_ERR_INVALID_ARG, "moe_mat_grouped_ffn: misaligned x, out or workspace");
  const int64_t need = moe_ffn_workspace_bytes(a->T, a->d, a->I, a->E, a->k, MOE_MODE_DECODE);
  MOE_CHECK_ARG(a->workspace_bytes >= need, MOE_ERR_WORKSPACE,
                "moe_mat_grouped_ffn: workspace %lld bytes < %lld needed (decode-mode size)",
                (long long)a->workspace_bytes, (long long)need);

  FfnDev f = {};
  f.x = a->x;
  f.T = a->T;
  f.d = a->d;
  f.I = a->I;
  f.E = a->E;
  f.k = a->k;
  f.P = (int64_t)a->T * a->k;
  f.umax = (int)std::min<int64_t>(a->E, f.P);
  f.topk_ids = a->topk_ids;
  f.topk_weights = a->topk_weights;  // the precision decision reads them
  f.offsets = a->expert_offsets;
  f.sorted_pairs = a->sorted_pairs;
  f.pair_pos = a->pair_pos;
  f.active = a->active_experts;
  f.bank = a->bank;
  f.bank_stride = a->bank_stride;
  f.slot_of_expert = a->slot_of_expert;
  const MatOffsets mo = mat_offsets(a->d, a->I);
  const FfnWorkspace w = ffn_workspace(a->T, a->d, a->I, a->E, a->k, MOE_MODE_DECODE, a->workspace);
  hipStream_t s = (hipStream_t)stream;
  const int G = a->d / kGroup;
  auto kgu = G <= 16 ? k_mat_gateup<16> : k_mat_gateup<32>;
  const int64_t items_gu = (int64_t)f.umax * (2 * a->I / (kTileRows * kMatRT));
  const int64_t grid_gu = std::min<int64_t>(mat_grid(kgu, G <= 16 ? 0 : 1, 512), ceil_div(items_gu, 8));
  const int64_t items_dn = (int64_t)f.umax * (a->d / (kTileRows * kMatRT)) * w.ksplit;
  const int64_t grid_dn = std::min<int64_t>(mat_grid(k_mat_down, 2, 256), ceil_div(items_dn, 4));
  timing_begin(K_GATEUP_MAT, s);
  hipLaunchKernelGGL(kgu, dim3((unsigned)grid_gu), dim3(512), 0, s, f, mo, tau, w.h);
  timing_end(K_GATEUP_MAT, s);
  timing_begin(K_DOWN_MAT, s);
  hipLaunchKernelGGL(k_mat_down, dim3((unsigned)grid_dn), dim3(256), 0, s, f, mo, tau, (const uint16_t*)w.h, w.y,
                     w.ksplit);
  timing_end(K_DOWN_MAT, s);
  rc = check_launch("grouped nested two/four-bit expert FFN");
  if (rc) return rc;
  if (a->combine) rc = launch_combine(f, w.y, w.ksplit, a->topk_weights, a->out, s);
  return rc;
}
