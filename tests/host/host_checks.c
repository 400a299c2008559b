/* Host-side paths of the W4A16 MoE library, for a build whose host code runs
 * under AddressSanitizer and UndefinedBehaviorSanitizer: layouts, workspace
 * sizes, status strings, and every entry point's argument checks.  No call here
 * reaches the GPU (each fails its host checks first or is a documented no-op),
 * so the program runs on a machine without one.  Exit status: the number of
 * checks that returned something else than expected. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "w4a16_moe.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: got %d, want %d (%s)\n", what, got, want, moe_last_error());
    ++failures;
  }
}

int main(void) {
  void* vp = (void*)256; /* never dereferenced */
  const uint16_t* hp = (const uint16_t*)vp;

  /* status strings and version */
  for (int s = -1; s <= 6; ++s) expect(moe_status_string(s) != NULL, 1, "status string");
  expect(moe_abi_version() > 0, 1, "abi version");

  /* layouts: 256-byte sections, sizes that grow with the expert */
  moe_expert_layout L;
  expect(moe_expert_layout_get(2048, 1024, &L), MOE_OK, "layout");
  expect(L.blob_bytes % 256 == 0 && L.w2_scales > L.w2_codes && L.w2_codes > L.w13_scales, 1, "layout order");
  expect(moe_expert_layout_get(100, 1024, &L), MOE_ERR_UNSUPPORTED_SHAPE, "layout d % 128");
  expect(moe_expert_layout_get(2048, 1024, NULL), MOE_ERR_INVALID_ARG, "layout null");
  moe_mat_layout M;
  expect(moe_mat_layout_get(2048, 1024, &M), MOE_OK, "mat layout");
  expect(M.two_bit_bytes > 0 && M.two_bit_bytes < M.blob_bytes, 1, "mat layout prefix");

  /* workspace sizes */
  expect(moe_ffn_workspace_bytes(16, 2048, 1024, 64, 8, 1) >= 16 * 8 * 1024 * 2 + 16 * 8 * 2048 * 4, 1, "ffn ws");
  expect((int)moe_ffn_workspace_bytes(-1, 2048, 1024, 64, 8, 0), -1, "ffn ws T < 0");
  expect(moe_decode_layer_workspace_bytes(16, 2048, 1024, 64, 8) > 0, 1, "layer ws");
  expect((int)moe_decode_layer_workspace_bytes(-1, 2048, 1024, 64, 8), -1, "layer ws T < 0");

  /* pack / route / align */
  expect(pack_w4_g128(hp, 1, 16, 100, 0, vp, 0, vp, 0, NULL), MOE_ERR_UNSUPPORTED_SHAPE, "pack K % 128");
  expect(pack_w4_g128(hp, 1, 48, 128, 1, vp, 0, vp, 0, NULL), MOE_ERR_UNSUPPORTED_SHAPE, "pack interleave N % 32");
  expect(pack_w4_g128(NULL, 1, 16, 128, 0, vp, 0, vp, 0, NULL), MOE_ERR_INVALID_ARG, "pack null");
  expect(pack_w4_g128(NULL, 0, 16, 128, 0, NULL, 0, NULL, 0, NULL), MOE_OK, "pack empty");
  expect(moe_route(hp, hp, 4, 64, 8, 9, 1, vp, vp, vp, NULL), MOE_ERR_UNSUPPORTED_SHAPE, "route k > E");
  expect(moe_route(hp, hp, 4, 64, 2000, 8, 1, vp, vp, vp, NULL), MOE_ERR_UNSUPPORTED_SHAPE, "route E > 1024");
  expect(moe_route(hp, hp, 4, 64, 8, 2, 1, NULL, vp, vp, NULL), MOE_ERR_INVALID_ARG, "route null");
  expect(moe_route(NULL, NULL, 0, 64, 8, 2, 1, NULL, NULL, NULL, NULL), MOE_OK, "route T = 0");
  expect(moe_align(vp, 4, 2, 1025, 0, vp, vp, vp, vp, NULL, NULL), MOE_ERR_UNSUPPORTED_SHAPE, "align E");
  expect(moe_align(vp, 4, 17, 64, 0, vp, vp, vp, vp, NULL, NULL), MOE_ERR_UNSUPPORTED_SHAPE, "align k");
  expect(moe_align(vp, 4, 2, 8, 64, vp, vp, vp, vp, NULL, NULL), MOE_ERR_INVALID_ARG, "align block_m");

  /* grouped FFN */
  expect(moe_w4a16_grouped_ffn(NULL, NULL), MOE_ERR_INVALID_ARG, "ffn null");
  moe_ffn_args a;
  memset(&a, 0, sizeof a);
  a.T = 4, a.d = 200, a.I = 512, a.E = 8, a.k = 2;
  expect(moe_w4a16_grouped_ffn(&a, NULL), MOE_ERR_UNSUPPORTED_SHAPE, "ffn d % 128");
  a.d = 256;
  expect(moe_w4a16_grouped_ffn(&a, NULL), MOE_ERR_INVALID_ARG, "ffn null pointers");
  a.x = hp, a.topk_ids = vp, a.topk_weights = vp, a.expert_offsets = vp, a.sorted_pairs = vp, a.pair_pos = vp;
  a.active_experts = vp, a.out = (uint16_t*)vp, a.bank = vp, a.bank_stride = 202752, a.workspace = vp;
  a.combine = 1, a.workspace_bytes = 16;
  expect(moe_w4a16_grouped_ffn(&a, NULL), MOE_ERR_WORKSPACE, "ffn workspace");
  a.bank_stride = 1000;
  expect(moe_w4a16_grouped_ffn(&a, NULL), MOE_ERR_INVALID_ARG, "ffn stride");
  expect(moe_bf16_grouped_ffn(NULL, NULL), MOE_ERR_INVALID_ARG, "bf16 ffn null");
  expect(moe_mat_grouped_ffn(NULL, 0.f, NULL), MOE_ERR_INVALID_ARG, "mat ffn null");
  expect(moe_w4a16_grouped_ffn_noalloc(NULL, NULL), MOE_ERR_INVALID_ARG, "noalloc null");
  memset(&a, 0, sizeof a);
  a.T = 4096, a.d = 2048, a.I = 1024, a.E = 64, a.k = 8, a.mode = 2;
  expect(moe_w4a16_grouped_ffn_noalloc(&a, NULL), MOE_ERR_WORKSPACE, "noalloc beyond the scratch");

  /* fused decode layers */
  moe_decode_layer_args l;
  memset(&l, 0, sizeof l);
  l.T = 17, l.d = 256, l.I = 512, l.E = 8, l.k = 2, l.renormalize = 1;
  expect(moe_decode_layer(&l, NULL), MOE_ERR_UNSUPPORTED_SHAPE, "layer T > 16");
  l.T = 4;
  expect(moe_decode_layer(&l, NULL), MOE_ERR_INVALID_ARG, "layer null pointers");
  expect(moe_mat_decode_layer(&l, NAN, NULL), MOE_ERR_INVALID_ARG, "mat layer NaN tau");
  l.x = hp, l.w_router = hp, l.bank = vp, l.logits = vp, l.topk_ids = vp, l.topk_weights = vp;
  l.out = (uint16_t*)vp, l.workspace = vp, l.counters = vp, l.bank_stride = 202752, l.workspace_bytes = 16;
  expect(moe_decode_layer(&l, NULL), MOE_ERR_WORKSPACE, "layer workspace");
  l.T = 0;
  expect(moe_decode_layer(&l, NULL), MOE_OK, "layer T = 0");

  /* slot cache and timing */
  moe_slot_cache* c = NULL;
  expect(moe_slot_cache_create(0, 16, 100, vp, vp, &c), MOE_ERR_INVALID_ARG, "cache E = 0");
  expect(moe_slot_cache_create(64, 16, 100, NULL, vp, &c), MOE_ERR_INVALID_ARG, "cache null store");
  expect(slot_cache_load(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL), MOE_ERR_INVALID_ARG, "cache load");
  expect(moe_slot_cache_configure(NULL, 0, 0.9, 1), MOE_ERR_INVALID_ARG, "cache configure");
  expect(slot_cache_begin_step(NULL, NULL), MOE_ERR_INVALID_ARG, "cache begin step");
  expect(moe_slot_cache_destroy(NULL), MOE_OK, "cache destroy null");
  expect(moe_timing_read(99, NULL, NULL), MOE_ERR_INVALID_ARG, "timing id");

  printf("host checks: %d failures\n", failures);
  return failures;
}
