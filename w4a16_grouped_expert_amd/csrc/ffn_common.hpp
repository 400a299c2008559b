// Device-side view of one grouped FFN call, shared by the decode and prefill kernels.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace moe {

// Weight formats and precisions of the fused decode passes: four-bit blobs of
// layout v1, or nested two/four-bit blobs of layout m1 with every expert at four
// bits (tau <= 0), every expert at two bits (tau > 1), or each expert at four
// bits when the largest routing weight of its pairs reaches tau.
enum LayerPrec { kPrecW4 = 0, kPrecAll4 = 1, kPrecAll2 = 2, kPrecMixed = 3 };

struct FfnDev {
  const uint16_t* x;  // [T][d] bf16
  int T, d, I, E, k;
  int64_t P;          // T * k
  const int32_t* topk_ids;  // [T][k]
  const float* topk_weights;  // [T][k]
  int umax;           // upper bound on active experts: min(E, P)
  const int32_t* offsets;
  const int32_t* sorted_pairs;
  const int32_t* pair_pos;
  const int32_t* active;  // work list: [0] = U, entry u at 4 + 4u = {expert, row0, count, 0}
  const int32_t* tile_offsets;
  const uint8_t* bank;
  int64_t bank_stride;
  const int32_t* slot_of_expert;
  // layout v1: codes and scales; layout m1: high planes (as codes), scales and low planes
  int64_t off_w13_codes, off_w13_scales, off_w2_codes, off_w2_scales;
  int64_t off_w13_lo = 0, off_w2_lo = 0;
  float tau = 0.f;  // layout m1, mixed precision: an expert runs at four bits when a pair's weight reaches it
  // counters of the fused down + combine pass, zeroed by the gate/up pass before it
  int32_t* zero_ctr = nullptr;
  int n_zero_ctr = 0;

  // Blob of expert e, or nullptr when the expert is not part of this call.
  __device__ __forceinline__ const uint8_t* blob(int e) const {
    const int s = slot_of_expert ? slot_of_expert[e] : e;
    return s < 0 ? nullptr : bank + (int64_t)s * bank_stride;
  }
};

__device__ __forceinline__ void zero_down_counters(const FfnDev& f) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < f.n_zero_ctr; i += blockDim.x) f.zero_ctr[i] = 0;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// Workspace of one call: h [T*k][I] bf16, y [ksplit][T*k][d] fp32 (prefill:
// [T*k][d] bf16), for the prefill variant the group sums of x and h, and for
// steps of at most 16 tokens the partial sums and stripe counters of the fused
// down + combine pass.
struct FfnWorkspace {
  uint16_t* h;
  float* y;
  float* xsum;
  float* hsum;
  float* dc_part;       // [d / 32][32][512] fp32, or nullptr
  int32_t* dc_counters;  // [d / 32], or nullptr
  int ksplit;
};
FfnWorkspace ffn_workspace(int T, int d, int I, int E, int k, int mode, void* ws);
int launch_combine(const FfnDev& f, const float* y, int ksplit, const float* weights, uint16_t* out, hipStream_t s);

// out != nullptr (T <= 16, dc_part and dc_counters set): the down pass also
// performs the routing-weighted combine into out, and y is not written.
int launch_decode(const FfnDev& f, uint16_t* h, float* y, int ksplit, int nb, hipStream_t s,
                  uint16_t* out = nullptr, float* dc_part = nullptr, int32_t* dc_counters = nullptr);
// The fused down + combine pass alone (see launch_decode); pair: h rows in pair
// order and the active experts built from the routing table (the n_route_ctr
// counters at route_ctr zeroed).
void launch_down_combine(const FfnDev& f, const uint16_t* h, uint16_t* out, float* part, int32_t* counters,
                         int32_t* route_ctr, int n_route_ctr, hipStream_t s, bool pair);
// Units per wavefront of the fused down + combine pass, 0 if the step is too large for it.
int dc_units_per_wave(int umax, int G, int stripes);
// y: the per-pair outputs [P][d] in bf16 (combined by launch_combine_bf16)
int launch_prefill(const FfnDev& f, uint16_t* h, uint16_t* y, float* xsum, float* hsum, hipStream_t s);
int launch_combine_bf16(const FfnDev& f, const uint16_t* y, const float* weights, uint16_t* out, hipStream_t s);
int64_t prefill_extra_bytes(int T, int d, int I, int k);

}  // namespace moe
