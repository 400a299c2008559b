// The grouped expert pass over unquantised BF16 experts: the same routing,
// permutation, work list and combine as the four-bit pass, with the expert
// weights read as bf16 straight from row-major [2I][d] (gate rows, then up rows)
// and [d][I] matrices.  It is the BF16 side of the page's W4-versus-BF16 decode
// comparison (ExactMoE, page "Every Expert Counts: ExactMoE for Memory-Efficient
// W4A16 Inference", Abstract: four-bit experts against the BF16 model), and moves
// 3.88x the bytes of the four-bit pass per expert.
//
// Contraction: v_mfma_f32_16x16x32_bf16 with weight rows on the 16-row side.  The
// A fragment of K step i for lane l is the eight bf16 weights at row l % 16,
// columns 32i + 8(l / 16) .. + 7 of a 128-wide group: one 16-byte load from the
// row-major matrix, and the four K steps of a group together read 256 contiguous
// bytes of each row.  Sums are fp32 over the whole K range (no scales).
//
// Work split: persistent wavefronts walk (active expert, stripe of 2 tiles, K
// split) items.  Gate/up stripes are 16 gate rows + the matching 16 up rows, so
// SwiGLU happens in registers; down stripes are 32 output rows, with K split over
// items when few experts are active (partials summed by the combine).  Each item
// runs the expert's pairs in blocks of 16 * NB columns, the weights of a group
// double-buffered in registers.
#include "ffn_common.hpp"

namespace moe {

constexpr int kB16RT = 2;  // row tiles per stripe

template <int NB, bool GATEUP>
__global__ __launch_bounds__(256) void k_bf16_ffn(FfnDev f, const uint16_t* __restrict__ hin,
                                                  uint16_t* __restrict__ hout, float* __restrict__ y, int ksplit) {
  const int K = GATEUP ? f.d : f.I;
  const int G = K / kGroup;
  const int n_stripes = GATEUP ? f.I / kTileRows : f.d / (kTileRows * kB16RT);
  const int per_u = n_stripes * ksplit;
  const int n_items = f.umax * per_u;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int col = lane & 15, kq = lane >> 4;
  const int worker = blockIdx.x * 4 + wave, n_workers = gridDim.x * 4;
  const int U = f.active[0];
  const int gs_per = (G + ksplit - 1) / ksplit;
  const uint32_t kNoRow = 0x7F000000u;  // past the end of any activation buffer: reads zeros
  const __amdgpu_buffer_rsrc_t xres =
      GATEUP ? __builtin_amdgcn_make_buffer_rsrc((void*)f.x, (short)0, (int)(f.T * f.d * 2), kBufferRsrcWord3)
             : __builtin_amdgcn_make_buffer_rsrc((void*)hin, (short)0, (int)(f.P * f.I * 2), kBufferRsrcWord3);
  const i32x4_t* work = reinterpret_cast<const i32x4_t*>(f.active + 4);

  for (int item = worker; item < n_items; item += n_workers) {
    const int u = item / per_u;
    if (u >= U) break;  // items are visited in increasing u: nothing active remains
    const int rem = item % per_u;
    const int stripe = rem / ksplit, split = rem % ksplit;
    const i32x4_t w4 = work[u];
    const int e = w4[0], row0 = w4[1], n_e = w4[2];
    const uint8_t* blob = f.blob(e);
    if (!blob) continue;
    const uint16_t* W = reinterpret_cast<const uint16_t*>(blob) + (GATEUP ? 0 : (int64_t)2 * f.I * f.d);
    const int trow0 = GATEUP ? kTileRows * stripe : kTileRows * kB16RT * stripe;
    const int trow1 = GATEUP ? f.I + kTileRows * stripe : trow0 + kTileRows;
    const uint16_t* wr0 = W + (int64_t)(trow0 + col) * K + 8 * kq;
    const uint16_t* wr1 = W + (int64_t)(trow1 + col) * K + 8 * kq;
    const int g0 = min(G, split * gs_per), g1 = min(G, g0 + gs_per);

    for (int tb = 0; tb < n_e; tb += 16 * NB) {
      uint32_t xoff[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int c = tb + 16 * b + col;
        xoff[b] = c >= n_e ? kNoRow
                           : (GATEUP ? (uint32_t)((f.sorted_pairs[row0 + c] / f.k) * f.d + 8 * kq) * 2u
                                     : (uint32_t)((row0 + c) * f.I + 8 * kq) * 2u);
      }
      f32x4_t acc[kB16RT][NB];
#pragma unroll
      for (int r = 0; r < kB16RT; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[r][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      // weights of group g into a register buffer; past g1 the loads repeat
      // group g1 - 1 and are not used
      u32x4_t wb[2][kB16RT][4];
      auto load_w = [&](int slot, int g) {
        const int gl = min(g, g1 - 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wb[slot][0][i] = *reinterpret_cast<const u32x4_t*>(wr0 + gl * kGroup + 32 * i);
          wb[slot][1][i] = *reinterpret_cast<const u32x4_t*>(wr1 + gl * kGroup + 32 * i);
        }
      };
      if (g0 < g1) load_w(0, g0);
      for (int g = g0; g < g1; g += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int gg = g + h;
          if (gg >= g1) break;
          load_w(h ^ 1, gg + 1);
          u32x4_t xb[NB][4];
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              xb[b][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                         xres, xoff[b] + (uint32_t)(gg * kGroup + 32 * i) * 2u, 0, 0));
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < kB16RT; ++r)
#pragma unroll
              for (int b = 0; b < NB; ++b)
                acc[r][b] = mfma16x16x32(as_bf16x8(wb[h][r][i]), as_bf16x8(xb[b][i]), acc[r][b]);
        }
      }

#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int c = tb + 16 * b + col;
        if (c >= n_e) continue;
        if (GATEUP) {
          float hf[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) hf[q] = silu_f32(acc[0][b][q]) * acc[1][b][q];
          const int hcol = kTileRows * stripe + 4 * kq;
          const u32x2_t o = pack_bf16x4(hf[0], hf[1], hf[2], hf[3]);
          *reinterpret_cast<u32x2_t*>(hout + (int64_t)(row0 + c) * f.I + hcol) = o;
        } else {
          float* yout = y + (int64_t)split * f.P * f.d + (int64_t)(row0 + c) * f.d;
#pragma unroll
          for (int r = 0; r < kB16RT; ++r)
            *reinterpret_cast<f32x4_t*>(yout + trow0 + kTileRows * r + 4 * kq) = acc[r][b];
        }
      }
    }
  }
}

template <typename Kern>
static int bf16_grid(Kern kern, int slot) {
  static int cached[4] = {0};
  if (!cached[slot]) {
    int dev = 0, cus = 0, per_cu = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0);
    cached[slot] = std::max(1, cus) * std::max(1, per_cu);
  }
  return cached[slot];
}

}  // namespace moe

using namespace moe;

extern "C" int64_t moe_bf16_expert_bytes(int d, int I) {
  if (d <= 0 || I <= 0) return -1;
  return (int64_t)6 * d * I;  // [2I][d] + [d][I] bf16
}

extern "C" int moe_bf16_pack(const uint16_t* w13, const uint16_t* w2, int E, int d, int I, uint8_t* bank,
                             int64_t bank_stride, void* stream) {
  clear_error();
  MOE_CHECK_ARG(E > 0 && d > 0 && I > 0, MOE_ERR_INVALID_ARG, "moe_bf16_pack: bad sizes E=%d d=%d I=%d", E, d, I);
  MOE_CHECK_ARG(w13 && w2 && bank, MOE_ERR_INVALID_ARG, "moe_bf16_pack: null pointer");
  const int64_t b13 = (int64_t)2 * I * d * 2, b2 = (int64_t)d * I * 2;
  MOE_CHECK_ARG(bank_stride >= b13 + b2, MOE_ERR_INVALID_ARG, "moe_bf16_pack: bank stride %lld < %lld",
                (long long)bank_stride, (long long)(b13 + b2));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e1 = hipMemcpy2DAsync(bank, (size_t)bank_stride, w13, (size_t)b13, (size_t)b13, (size_t)E,
                                   hipMemcpyDeviceToDevice, s);
  hipError_t e2 = hipMemcpy2DAsync(bank + b13, (size_t)bank_stride, w2, (size_t)b2, (size_t)b2, (size_t)E,
                                   hipMemcpyDeviceToDevice, s);
  MOE_CHECK_ARG(e1 == hipSuccess && e2 == hipSuccess, MOE_ERR_HIP, "moe_bf16_pack: copy failed: %s",
                hipGetErrorString(e1 != hipSuccess ? e1 : e2));
  return MOE_OK;
}

extern "C" int moe_bf16_grouped_ffn(const moe_ffn_args* a, void* stream) {
  clear_error();
  MOE_CHECK_ARG(a != nullptr, MOE_ERR_INVALID_ARG, "moe_bf16_grouped_ffn: args is NULL");
  MOE_CHECK_ARG(a->T >= 0 && a->d > 0 && a->I > 0 && a->E > 0 && a->k > 0, MOE_ERR_INVALID_ARG,
                "moe_bf16_grouped_ffn: bad sizes T=%d d=%d I=%d E=%d k=%d", a->T, a->d, a->I, a->E, a->k);
  MOE_CHECK_ARG(a->d % kGroup == 0 && a->I % kGroup == 0 && a->E <= MOE_MAX_EXPERTS && a->k <= MOE_MAX_TOPK &&
                    a->k <= a->E && (int64_t)a->T * a->k <= (1 << 24),
                MOE_ERR_UNSUPPORTED_SHAPE,
                "moe_bf16_grouped_ffn: unsupported shape d=%d I=%d E=%d k=%d T=%d (d, I multiples of 128, "
                "E <= 1024, k <= min(E,16))",
                a->d, a->I, a->E, a->k, a->T);
  if (a->T == 0) return MOE_OK;
  MOE_CHECK_ARG(a->x && a->topk_ids && a->topk_weights && a->expert_offsets && a->sorted_pairs && a->pair_pos &&
                    a->active_experts && a->bank && a->workspace,
                MOE_ERR_INVALID_ARG, "moe_bf16_grouped_ffn: null pointer");
  MOE_CHECK_ARG(!a->combine || a->out, MOE_ERR_INVALID_ARG, "moe_bf16_grouped_ffn: combine needs out");
  MOE_CHECK_ARG(a->bank_stride >= moe_bf16_expert_bytes(a->d, a->I) && a->bank_stride % 256 == 0 &&
                    ((uintptr_t)a->bank % 256) == 0,
                MOE_ERR_INVALID_ARG,
                "moe_bf16_grouped_ffn: bank must be 256-byte aligned with stride >= %lld (multiple of 256), got %lld",
                (long long)moe_bf16_expert_bytes(a->d, a->I), (long long)a->bank_stride);
  MOE_CHECK_ARG(((uintptr_t)a->x % 16) == 0 && ((uintptr_t)a->workspace % 256) == 0 &&
                    ((uintptr_t)a->active_experts % 16) == 0 && (!a->out || ((uintptr_t)a->out % 8) == 0),
                MOE_ERR_INVALID_ARG, "moe_bf16_grouped_ffn: misaligned x, out or workspace");
  // activations and h are addressed with 32-bit byte offsets by the buffer loads
  MOE_CHECK_ARG((int64_t)a->T * a->d * 2 < ((int64_t)1 << 31) && (int64_t)a->T * a->k * a->I * 2 < ((int64_t)1 << 31),
                MOE_ERR_UNSUPPORTED_SHAPE, "moe_bf16_grouped_ffn: T=%d too large for 32-bit activation offsets", a->T);
  const int64_t need = moe_ffn_workspace_bytes(a->T, a->d, a->I, a->E, a->k, MOE_MODE_DECODE);
  MOE_CHECK_ARG(a->workspace_bytes >= need, MOE_ERR_WORKSPACE,
                "moe_bf16_grouped_ffn: workspace %lld bytes < %lld needed (decode-mode size)",
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
  f.topk_weights = a->topk_weights;
  f.offsets = a->expert_offsets;
  f.sorted_pairs = a->sorted_pairs;
  f.pair_pos = a->pair_pos;
  f.active = a->active_experts;
  f.tile_offsets = a->tile_offsets;
  f.bank = a->bank;
  f.bank_stride = a->bank_stride;
  f.slot_of_expert = a->slot_of_expert;

  const FfnWorkspace w = ffn_workspace(a->T, a->d, a->I, a->E, a->k, MOE_MODE_DECODE, a->workspace);
  hipStream_t s = (hipStream_t)stream;
  // one 16-column block per expert when the step is small, else four
  const bool small = (double)a->T * a->k / a->E <= 16.0;
  auto kgu = small ? k_bf16_ffn<1, true> : k_bf16_ffn<4, true>;
  auto kdn = small ? k_bf16_ffn<1, false> : k_bf16_ffn<4, false>;
  const int64_t items_gu = (int64_t)f.umax * (a->I / kTileRows);
  const int64_t items_dn = (int64_t)f.umax * (a->d / (kTileRows * kB16RT)) * w.ksplit;
  const int64_t grid_gu = std::min<int64_t>(bf16_grid(kgu, small ? 0 : 1), ceil_div(items_gu, 4));
  const int64_t grid_dn = std::min<int64_t>(bf16_grid(kdn, small ? 2 : 3), ceil_div(items_dn, 4));
  timing_begin(K_GATEUP_BF16, s);
  hipLaunchKernelGGL(kgu, dim3((unsigned)grid_gu), dim3(256), 0, s, f, (const uint16_t*)nullptr, w.h,
                     (float*)nullptr, 1);
  timing_end(K_GATEUP_BF16, s);
  timing_begin(K_DOWN_BF16, s);
  hipLaunchKernelGGL(kdn, dim3((unsigned)grid_dn), dim3(256), 0, s, f, (const uint16_t*)w.h, (uint16_t*)nullptr, w.y,
                     w.ksplit);
  timing_end(K_DOWN_BF16, s);
  int rc = check_launch("grouped BF16 expert FFN");
  if (rc) return rc;
  if (a->combine) rc = launch_combine(f, w.y, w.ksplit, a->topk_weights, a->out, s);
  return rc;
}
