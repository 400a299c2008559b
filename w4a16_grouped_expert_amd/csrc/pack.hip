// pack_w4_g128: group-128 symmetric int4 quantisation of routed-expert weights
// and packing into layout v1 (ExactMoE, page "Every Expert Counts: ExactMoE for
// Memory-Efficient W4A16 Inference", Abstract: symmetric group-128 four-bit
// weights for the routed experts only).
//
// One wavefront produces one 16-row x 128-column tile (1024 bytes of codes and
// 16 bf16 scales).  Lane L owns row L % 16 and the 32 columns that its 16 output
// bytes hold (32i + 8(L/16) + m), so the loads, the quantisation and the single
// 16-byte store are all lane-local; only the group maximum needs the four lanes
// that share a row (XOR-16 and XOR-32 shuffles).
#include "common.hpp"

namespace moe {

__global__ __launch_bounds__(256) void k_pack_w4g128(const uint16_t* __restrict__ w, int E, int N, int K,
                                                     int interleave, uint8_t* __restrict__ codes,
                                                     int64_t codes_stride, uint8_t* __restrict__ scales,
                                                     int64_t scales_stride) {
  const int lane = lane_id();
  const int G = K / kGroup;
  const int NT = N / kTileRows;
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t tiles_per_expert = (int64_t)NT * G;
  if (tile >= tiles_per_expert * E) return;
  const int e = (int)(tile / tiles_per_expert);
  const int64_t t = tile % tiles_per_expert;
  const int nt = (int)(t / G);  // packed row tile
  const int kb = (int)(t % G);
  const int r = lane & 15, c = lane >> 4;

  int src_row;
  if (interleave) {
    const int I = N / 2;
    src_row = ((nt & 1) ? I : 0) + (nt >> 1) * kTileRows + r;
  } else {
    src_row = nt * kTileRows + r;
  }
  const uint16_t* src = w + ((int64_t)e * N + src_row) * K + (int64_t)kb * kGroup + 8 * c;

  // 32 values: word i holds columns 32i + 8c + m
  uint32_t v[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4_t q = *reinterpret_cast<const u32x4_t*>(src + 32 * i);
    v[i][0] = q[0]; v[i][1] = q[1]; v[i][2] = q[2]; v[i][3] = q[3];
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[i][j] & 0xFFFFu)));
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(v[i][j] >> 16)));
    }
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));

  // scale = bf16_rne(fl32(amax / 7)); the fp32 quotient is correctly rounded
  const uint32_t sbits = f32_to_bf16_bits(__fdiv_rn(amax, 7.0f));
  const float s = bf16_bits_to_f32(sbits);

  u32x4_t out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t u = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t hb = (m & 1) ? (v[i][m >> 1] >> 16) : (v[i][m >> 1] & 0xFFFFu);
      int q = 0;
      if (s > 0.f) {
        float qf = rintf(__fdiv_rn(bf16_bits_to_f32(hb), s));
        qf = fminf(fmaxf(qf, -8.f), 7.f);
        q = (int)qf;
      }
      u |= (uint32_t)(q + 8) << (4 * (m >> 1) + 16 * (m & 1));
    }
    out[i] = (u << 3) | (u >> 29);  // rotl32(u, 3)
  }
  uint8_t* dst = codes + (int64_t)e * codes_stride + t * kTileBytes + 16 * lane;
  *reinterpret_cast<u32x4_t*>(dst) = out;
  if (c == 0) {
    uint16_t* sdst = reinterpret_cast<uint16_t*>(scales + (int64_t)e * scales_stride) + t * kTileRows + r;
    *sdst = (uint16_t)sbits;
  }
}

}  // namespace moe

using namespace moe;

extern "C" int pack_w4_g128(const uint16_t* w, int E, int N, int K, int gateup_interleave, uint8_t* codes,
                            int64_t codes_stride, uint16_t* scales, int64_t scales_stride, void* stream) {
  clear_error();
  MOE_CHECK_ARG(E >= 0 && N >= 0 && K >= 0, MOE_ERR_INVALID_ARG, "pack_w4_g128: negative size");
  MOE_CHECK_ARG(N % kTileRows == 0 && K % kGroup == 0, MOE_ERR_UNSUPPORTED_SHAPE,
                "pack_w4_g128: N=%d must be a multiple of 16 and K=%d a multiple of 128", N, K);
  MOE_CHECK_ARG(!gateup_interleave || N % (2 * kTileRows) == 0, MOE_ERR_UNSUPPORTED_SHAPE,
                "pack_w4_g128: gate/up interleave needs N=%d to be a multiple of 32", N);
  if ((int64_t)E * N * K == 0) return MOE_OK;
  MOE_CHECK_ARG(w && codes && scales, MOE_ERR_INVALID_ARG, "pack_w4_g128: null pointer");
  const int64_t cbytes = (int64_t)N * K / 2, sbytes = (int64_t)N * (K / kGroup) * 2;
  MOE_CHECK_ARG(E == 1 || (codes_stride >= cbytes && scales_stride >= sbytes), MOE_ERR_INVALID_ARG,
                "pack_w4_g128: strides (%lld, %lld) smaller than one expert (%lld, %lld)",
                (long long)codes_stride, (long long)scales_stride, (long long)cbytes, (long long)sbytes);
  MOE_CHECK_ARG(((uintptr_t)w % 16) == 0 && ((uintptr_t)codes % 16) == 0 && (codes_stride % 16) == 0 &&
                    ((uintptr_t)scales % 2) == 0 && (scales_stride % 2) == 0,
                MOE_ERR_INVALID_ARG, "pack_w4_g128: misaligned pointer or stride");
  const int64_t tiles = (int64_t)E * (N / kTileRows) * (K / kGroup);
  const int64_t blocks = ceil_div(tiles, 4);
  MOE_CHECK_ARG(blocks < (1LL << 31), MOE_ERR_UNSUPPORTED_SHAPE, "pack_w4_g128: too many tiles");
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(k_pack_w4g128, dim3((unsigned)blocks), dim3(256), 0, s, w, E, N, K, gateup_interleave,
                     codes, codes_stride, reinterpret_cast<uint8_t*>(scales), scales_stride);
  return check_launch("pack_w4_g128");
}
