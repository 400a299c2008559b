// moe_decode_layer: the fused two-launch decode step on four-bit (layout v1) blobs.
#include "layer_gateup.hpp"

using namespace moe;

extern "C" int64_t moe_decode_layer_workspace_bytes(int T, int d, int I, int E, int k) {
  if (T < 0 || d <= 0 || I <= 0 || E <= 0 || k <= 0) return -1;
  return layer_ws_h(T, I, k) + align256((int64_t)(d / 32) * 32 * 512 * 4);
}

extern "C" int moe_decode_layer(const moe_decode_layer_args* a, void* stream) {
  clear_error();
  MOE_CHECK_ARG(a != nullptr, MOE_ERR_INVALID_ARG, "moe_decode_layer: args is NULL");
  // the layout of well-formed sizes (the launcher reports the others)
  moe_expert_layout el = {};
  if (a->d > 0 && a->I > 0 && a->d % kGroup == 0 && a->I % kGroup == 0) {
    const int rc = moe_expert_layout_get(a->d, a->I, &el);
    if (rc) return rc;
  }
  const LayerLayout lay = {el.blob_bytes, el.w13_codes, el.w13_scales, el.w2_codes, el.w2_scales, 0, 0};
  return decode_layer_launch<kPrecW4>(a, lay, INFINITY, "moe_decode_layer", stream);
}
