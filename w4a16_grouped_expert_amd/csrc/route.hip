// moe_route: BF16 router logits and unchanged top-k selection (ExactMoE, page
// "Every Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference",
// Abstract: the router stays BF16 and the top-k routing procedure is unchanged).
//
// Logits: products of bf16 values are exact, and the sum is kept in float64 so
// that the float32 logit is (to within one rounding of a float64 sum) the
// correctly rounded dot product; on MI355X an fp64 FMA issues at the same rate
// as a non-packed fp32 FMA, so the exactness costs nothing here.  A block of
// four wavefronts covers TB tokens x 16 experts; each wavefront owns four
// experts and its lanes stride through d in 16-byte chunks.
//
// Top-k: one wavefront per token holds the E logits in registers (lane l owns
// experts l, l+64, ...) and extracts the k largest with a wave-wide (value desc,
// index asc) argmax per step, then forms the softmax weights in float32.
#include "common.hpp"

namespace moe {

template <int TB>
__global__ __launch_bounds__(256) void k_route_logits(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ wr, int T, int d, int E,
                                                      float* __restrict__ logits) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TB;
  const int e0 = blockIdx.y * 16 + wave * 4;
  const int nch = d / 8;
  double acc[TB][4];
#pragma unroll
  for (int a = 0; a < TB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;

  for (int ch = lane; ch < nch; ch += 64) {
    double xv[TB][8];
#pragma unroll
    for (int a = 0; a < TB; ++a) {
      const int t = t0 + a;
      u32x4_t q = {0, 0, 0, 0};
      if (t < T) q = *reinterpret_cast<const u32x4_t*>(x + (int64_t)t * d + 8 * ch);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xv[a][2 * j] = (double)bf16_bits_to_f32(q[j] & 0xFFFFu);
        xv[a][2 * j + 1] = (double)bf16_bits_to_f32(q[j] >> 16);
      }
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int e = e0 + b;
      u32x4_t q = {0, 0, 0, 0};
      if (e < E) q = *reinterpret_cast<const u32x4_t*>(wr + (int64_t)e * d + 8 * ch);
      double wv[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wv[2 * j] = (double)bf16_bits_to_f32(q[j] & 0xFFFFu);
        wv[2 * j + 1] = (double)bf16_bits_to_f32(q[j] >> 16);
      }
#pragma unroll
      for (int a = 0; a < TB; ++a)
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[a][b] = fma(xv[a][m], wv[m], acc[a][b]);
    }
  }
#pragma unroll
  for (int a = 0; a < TB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      double v = acc[a][b];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      const int t = t0 + a, e = e0 + b;
      if (lane == 0 && t < T && e < E) logits[(int64_t)t * E + e] = (float)v;
    }
}

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int T, int E, int k,
                                                    int renormalize, int32_t* __restrict__ ids,
                                                    float* __restrict__ weights) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nper = (E + 63) / 64;  // <= 16
  float v[16];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    v[i] = (i < nper && e < E) ? logits[(int64_t)t * E + e] : 0.f;
  }
  float sel_v[16];
  int sel_i[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j >= k) break;
    float bv = 0.f;
    int bi = 0x7FFFFFFF;
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
    sel_v[j] = bv;
    sel_i[j] = bi;
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
  }
  const float lmax = sel_v[0];
  float den = 0.f;
  if (renormalize) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < k) den += expf(sel_v[j] - lmax);
  } else {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + 64 * i;
      if (i < nper && e < E) part += expf(v[i] - lmax);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    den = part;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < k && lane == j) {
      ids[(int64_t)t * k + j] = sel_i[j];
      weights[(int64_t)t * k + j] = expf(sel_v[j] - lmax) / den;
    }
  }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_route(const uint16_t* x, const uint16_t* w_router, int T, int d, int E, int k,
                         int renormalize, float* logits, int32_t* topk_ids, float* topk_weights, void* stream) {
  clear_error();
  MOE_CHECK_ARG(T >= 0 && d > 0 && E > 0 && k > 0, MOE_ERR_INVALID_ARG,
                "moe_route: bad sizes T=%d d=%d E=%d k=%d", T, d, E, k);
  MOE_CHECK_ARG(E <= MOE_MAX_EXPERTS && k <= MOE_MAX_TOPK && k <= E && d % 8 == 0, MOE_ERR_UNSUPPORTED_SHAPE,
                "moe_route: unsupported E=%d k=%d d=%d (E <= 1024, k <= min(E,16), d %% 8 == 0)", E, k, d);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(x && w_router && logits && topk_ids && topk_weights, MOE_ERR_INVALID_ARG,
                "moe_route: null pointer");
  MOE_CHECK_ARG(((uintptr_t)x % 16) == 0 && ((uintptr_t)w_router % 16) == 0, MOE_ERR_INVALID_ARG,
                "moe_route: x and w_router must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  timing_begin(K_ROUTE, s);
  if (T <= 64) {
    hipLaunchKernelGGL(k_route_logits<1>, dim3(T, ceil_div(E, 16)), dim3(256), 0, s, x, w_router, T, d, E, logits);
  } else {
    hipLaunchKernelGGL(k_route_logits<4>, dim3(ceil_div(T, 4), ceil_div(E, 16)), dim3(256), 0, s, x, w_router, T,
                       d, E, logits);
  }
  int rc = check_launch("moe_route (logits)");
  if (rc) return rc;
  hipLaunchKernelGGL(k_route_topk, dim3(ceil_div(T, 4)), dim3(256), 0, s, logits, T, E, k, renormalize, topk_ids,
                     topk_weights);
  timing_end(K_ROUTE, s);
  return check_launch("moe_route (top-k)");
}
