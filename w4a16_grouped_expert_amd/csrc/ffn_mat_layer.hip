// moe_mat_decode_layer: the fused two-launch decode step (routing + gate/up +
// SwiGLU, then down + combine) on nested two/four-bit blobs (layout m1), each
// expert at four bits when the largest routing weight of its pairs reaches tau,
// else at two bits with the dropped bits replaced by their mean (page "MatMoE:
// Dynamic Mixed-Precision Quantization for Efficient MoE Inference", arXiv
// abstract: nested multi-precision experts, bit-widths from routing scores; the
// layer is ExactMoE's, page "Every Expert Counts: ExactMoE for Memory-Efficient
// W4A16 Inference", Abstract).  The kernels are those of moe_decode_layer with
// plane tiles as the K unit; at four bits every group's arithmetic is the same
// as on the layout v1 blob the nested one was made from.
//
// The precision rule fixes every expert when tau <= 0 (routing weights are never
// negative: four bits) or tau > 1 (a weight never exceeds 1: two bits); those
// calls use kernels whose loads do not wait for the routing.
#include <cmath>

#include "layer_gateup.hpp"

using namespace moe;

extern "C" int moe_mat_decode_layer(const moe_decode_layer_args* a, float tau, void* stream) {
  clear_error();
  MOE_CHECK_ARG(a != nullptr, MOE_ERR_INVALID_ARG, "moe_mat_decode_layer: args is NULL");
  MOE_CHECK_ARG(!std::isnan(tau), MOE_ERR_INVALID_ARG, "moe_mat_decode_layer: tau is NaN");
  MOE_CHECK_ARG(a->d <= 0 || a->I <= 0 || (a->d % kPlaneK == 0 && a->I % kPlaneK == 0), MOE_ERR_UNSUPPORTED_SHAPE,
                "moe_mat_decode_layer: d=%d and I=%d must be multiples of 256", a->d, a->I);
  moe_mat_layout ml = {};
  if (a->d > 0 && a->I > 0) {
    const int rc = moe_mat_layout_get(a->d, a->I, &ml);
    if (rc) return rc;
  }
  const LayerLayout lay = {ml.blob_bytes, ml.w13_hi, ml.w13_scales, ml.w2_hi, ml.w2_scales, ml.w13_lo, ml.w2_lo};
  const char* name = "moe_mat_decode_layer";
  if (tau <= 0.f) return decode_layer_launch<kPrecAll4>(a, lay, tau, name, stream);
  if (tau > 1.f) return decode_layer_launch<kPrecAll2>(a, lay, tau, name, stream);
  return decode_layer_launch<kPrecMixed>(a, lay, tau, name, stream);
}
