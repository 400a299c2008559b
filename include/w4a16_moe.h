/*
 * w4a16_moe.h -- C ABI of the fused grouped W4A16 mixture-of-experts layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is the routed-expert part of ExactMoE (page "Every Expert Counts:
 * ExactMoE for Memory-Efficient W4A16 Inference", Abstract): routed experts'
 * weights are symmetric four-bit integers with one scale per group of 128 input
 * channels, activations and the router stay BF16, the top-k routing procedure
 * is unchanged, every selected expert runs (none pruned or substituted), the
 * quantised experts may live in pinned host memory and reach the GPU through a
 * configurable number of resident slots, and all selected experts of a step run
 * through one fused grouped pass.  Expert FFN = SwiGLU: h = silu(x Wg^T) *
 * (x Wu^T), y = h Wd^T; out[t] = sum_j w[t,j] * y[t,j].
 *
 * Conventions for every call
 *  - Pointers named *_dev / all tensor pointers are device pointers unless the
 *    parameter says "host".  bf16 values travel as uint16_t bit patterns.  All
 *    arrays are dense row-major with the shapes given; no hidden transposes.
 *  - The caller owns every buffer.  No call allocates device memory.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls only
 *    enqueue work; nothing synchronises except where stated.
 *  - Return value: MOE_OK (0) or a moe_status code.  Argument and shape checks
 *    run on the host before anything is enqueued; on failure nothing is
 *    enqueued and moe_last_error() (thread-local) describes the problem.
 *  - Inputs must be finite; NaN / Inf inputs give unspecified outputs.
 */
#ifndef W4A16_MOE_H
#define W4A16_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,      /* null pointer, negative size, bad enum */
  MOE_ERR_UNSUPPORTED_SHAPE = 2,/* K % 128 != 0, N % 16 != 0, E > 1024, k > 16, ... */
  MOE_ERR_WORKSPACE = 3,        /* workspace too small or misaligned */
  MOE_ERR_CAPACITY = 4,         /* slot cache: fewer slots than experts a token needs */
  MOE_ERR_HIP = 5               /* a HIP launch or copy failed */
};

#define MOE_GROUP 128           /* quantisation group along K (input channels) */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16

/* Status name of a code (static string). */
const char* moe_status_string(int status);
/* Message of the last failing call on this thread ("" if none).  With the
 * environment variable MOE_W4A16_LOG=1 each such message is also printed to
 * stderr when it is recorded; with 2, every moe_w4a16_grouped_ffn call also
 * prints the kernels it chose (decode or prefill variant, K split).  Read once. */
const char* moe_last_error(void);
/* ABI version of this library. */
int moe_abi_version(void);

/*
 * Byte layout of one packed expert ("blob"): w13 codes | w13 scales | w2 codes
 * | w2 scales, each section starting on a 256-byte boundary.  w13 is [2I, d]
 * (gate rows then up rows, packed with gate/up interleaving), w2 is [d, I].
 * A bank of experts (resident or slots) is an array of blobs at a fixed stride.
 */
typedef struct {
  int64_t w13_codes, w13_scales, w2_codes, w2_scales; /* byte offsets in the blob */
  int64_t blob_bytes;                                  /* total, multiple of 256 */
} moe_expert_layout;
int moe_expert_layout_get(int d, int I, moe_expert_layout* out);

/*
 * pack_w4_g128 -- quantise and pack E weight matrices (ExactMoE, Abstract:
 * symmetric group-128 four-bit routed-expert weights).
 *
 *  w       [E][N][K] bf16, device.
 *  scale of (row, group) = bf16_rne(amax / 7), amax = max |w| over the 128
 *  inputs of the group; q = clamp(rne(w / scale), -8, 7), q = 0 when scale = 0;
 *  stored code = q + 8 (4 bits).
 *  codes   device, expert e at codes + e * codes_stride (bytes), N*K/2 bytes each,
 *          packed layout v1: 16x128 tiles of 1024 bytes at (nb*K/128 + kb)*1024;
 *          lane L = 0..63 of a tile owns bytes 16L..16L+15 = row nb*16 + L%16,
 *          columns kb*128 + 32i + 8(L/16) + m in 32-bit word i; element m's code
 *          is the 4-bit field at bit (3 + 4(m/2) + 16(m%2)) mod 32 (wrapping).
 *  scales  device, expert e at (uint8_t*)scales + e * scales_stride (bytes),
 *          bf16 [N/16][K/128][16].
 *  gateup_interleave: 1 = W is [gate; up] (N = 2I); packed row tile 2j holds gate
 *          rows 16j.., tile 2j+1 up rows 16j.. (N % 32 == 0 required).
 *  Errors: MOE_ERR_UNSUPPORTED_SHAPE unless N % 16 == 0 and K % 128 == 0.
 *  Deterministic; bit-identical to the definition above (fp32 quotients are exact
 *  enough that every rounding decision equals the exact one).
 */
int pack_w4_g128(const uint16_t* w, int E, int N, int K, int gateup_interleave,
                 uint8_t* codes, int64_t codes_stride,
                 uint16_t* scales, int64_t scales_stride, void* stream);

/*
 * moe_route -- BF16 router and unchanged top-k (ExactMoE, Abstract).
 *
 *  x            [T][d] bf16 activations.  w_router [E][d] bf16.
 *  logits       [T][E] float32 output (required): sum_c x[t,c] * w_router[e,c],
 *               products exact, summed in float64, rounded once to float32 (the
 *               order of the float64 sum depends on the kernel T selects, so the
 *               last bit of a logit may too).
 *  topk_ids     [T][k] int32 output: experts ordered by (logit desc, index asc).
 *  topk_weights [T][k] float32 output: exp(l_j - l_max) / sum over the selected
 *               experts (renormalize = 1) or over all E (renormalize = 0).
 *  Limits: 1 <= k <= min(E, 16), E <= 1024, d % 8 == 0.  T == 0 is a no-op.
 */
int moe_route(const uint16_t* x, const uint16_t* w_router, int T, int d, int E, int k,
              int renormalize, float* logits, int32_t* topk_ids, float* topk_weights,
              void* stream);

/*
 * moe_align -- expert-sorted permutation of the T*k (token, slot) pairs that
 * feeds the grouped kernels.  Stable counting sort, pair p = t*k + j.
 * (ExactMoE, page "Every Expert Counts: ExactMoE for Memory-Efficient W4A16
 * Inference", Abstract: every selected expert of a step runs through fused
 * grouped MoE kernels; grouping a step's pairs by expert is what lets one grouped
 * pass stream each selected expert's weights once for all of its tokens.)
 *
 *  expert_offsets [E+1] int32: exclusive prefix sum of per-expert pair counts.
 *  sorted_pairs   [T*k] int32: pair ids grouped by expert, increasing within a group.
 *  pair_pos       [T*k] int32: position of pair p in sorted_pairs.
 *  active_experts [4 + 4E] int32, 16-byte aligned: the work list of the U experts
 *                 with >= 1 pair.  [0] = U, [1..3] = 0; entry u (ascending expert
 *                 id) at [4+4u .. 7+4u] = {expert id, expert_offsets[id], pair count, 0}.
 *  tile_offsets   [E+1] int32 or NULL: exclusive prefix sum of ceil(count / block_m)
 *                 (only when block_m > 0).
 *  Limits: E <= 1024, k <= 16, T*k <= 2^24.  Entries of topk_ids outside [0, E)
 *  are dropped: not counted, not placed, pair_pos = -1 (the combine skips them).
 *  Bit-exact: the output is unique.
 */
int moe_align(const int32_t* topk_ids, int T, int k, int E, int block_m,
              int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos,
              int32_t* active_experts, int32_t* tile_offsets, void* stream);

/*
 * moe_route_align -- moe_route followed by moe_align, in one launch for steps of
 * at most 128 tokens (the decode case); other steps (and T == 0) run the two
 * calls above.  Outputs are bit-identical to moe_route + moe_align.
 *
 *  Arguments: those of moe_route and moe_align, plus
 *  counters  MOE_ROUTE_ALIGN_COUNTERS int32 in device memory, owned by the
 *            caller: they must hold 0 before the first call and every call leaves
 *            them at 0.  Calls that share counters must not overlap (same stream,
 *            or otherwise ordered).
 *  Limits and errors: those of moe_route and moe_align; x, w_router and
 *  active_experts 16-byte aligned.
 */
#define MOE_ROUTE_ALIGN_COUNTERS 256
int moe_route_align(const uint16_t* x, const uint16_t* w_router, int T, int d, int E, int k,
                    int renormalize, int block_m, float* logits, int32_t* topk_ids,
                    float* topk_weights, int32_t* expert_offsets, int32_t* sorted_pairs,
                    int32_t* pair_pos, int32_t* active_experts, int32_t* tile_offsets,
                    int32_t* counters, void* stream);

/*
 * moe_w4a16_grouped_ffn -- the fused grouped expert pass (ExactMoE, Abstract:
 * all selected experts through fused grouped kernels): gate/up + SwiGLU, down,
 * routing-weighted combine, over the expert-sorted pairs from moe_align.
 */
/* MOE_MODE_AUTO: the decode kernels up to 20 expected pairs per expert (T k / E),
 * the MFMA-tiled prefill kernels above. */
enum moe_ffn_mode { MOE_MODE_AUTO = 0, MOE_MODE_DECODE = 1, MOE_MODE_PREFILL = 2 };

typedef struct {
  const uint16_t* x;              /* [T][d] bf16 */
  int T, d, I, E, k;
  const int32_t* topk_ids;        /* [T][k] from moe_route */
  const float* topk_weights;      /* [T][k] from moe_route */
  const int32_t* expert_offsets;  /* from moe_align */
  const int32_t* sorted_pairs;
  const int32_t* pair_pos;
  const int32_t* active_experts;  /* work list from moe_align */
  const int32_t* tile_offsets;    /* required for prefill mode with block_m = 128; else may be NULL */
  const uint8_t* bank;            /* expert blobs (moe_expert_layout), device */
  int64_t bank_stride;            /* bytes between blobs */
  const int32_t* slot_of_expert;  /* [E] device or NULL: blob index of each expert;
                                     -1 = skip the expert in this call */
  int mode;                       /* moe_ffn_mode */
  int combine;                    /* 1 = finish with the combine into `out`;
                                     0 = leave per-pair results in the workspace */
  uint16_t* out;                  /* [T][d] bf16 (written when combine = 1) */
  void* workspace;                /* device, 256-byte aligned */
  int64_t workspace_bytes;
} moe_ffn_args;

/* Workspace the call needs for these sizes and mode (bytes).
 * moe_w4a16_grouped_ffn: the experts of a token must be distinct (as moe_route
 * returns them).  Decode steps of at most 16 tokens called with combine = 1 and
 * slot_of_expert = NULL finish the combine inside the down pass (each group's
 * contribution scaled by its routing weight as it is accumulated, partial sums
 * added in a fixed order): the output is deterministic but is not bit-identical
 * to the two-pass combine, and no per-pair results are left in the workspace.
 * Calls with a slot table keep the two passes, so subsets of the experts can run
 * in separate calls with combine = 0 and the last one combines.  The per-pair
 * results of the two-pass combine are fp32 (decode mode) or rounded once to bf16
 * (prefill mode, which halves their write and read); the combine sums each
 * token's k rows in fp32 in slot order and rounds once to bf16. */
int64_t moe_ffn_workspace_bytes(int T, int d, int I, int E, int k, int mode);
int moe_w4a16_grouped_ffn(const moe_ffn_args* args, void* stream);

/*
 * moe_w4a16_grouped_ffn_noalloc -- moe_w4a16_grouped_ffn without a caller
 * workspace, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * workspace comes from a static device array of MOE_NOALLOC_SCRATCH_BYTES that
 * every GPU the library runs on holds until the process ends; the call makes no
 * allocation of any kind.
 *
 *  args  as for moe_w4a16_grouped_ffn, with workspace = NULL and
 *        workspace_bytes = 0 (MOE_ERR_INVALID_ARG otherwise).  Results are those
 *        of moe_w4a16_grouped_ffn on the same arguments (the same kernels on the
 *        same workspace layout), including combine = 0 rounds whose per-pair
 *        results stay in the scratch for a later call with combine = 1.
 *  Runs on the calling thread's current device; `stream` must belong to it.
 *  Errors: MOE_ERR_WORKSPACE when moe_ffn_workspace_bytes(T, d, I, E, k, mode)
 *  exceeds MOE_NOALLOC_SCRATCH_BYTES (checked on the host before anything is
 *  enqueued; e.g. OLMoE-shaped decode steps of 16 tokens use under 6 MiB, and
 *  OLMoE-shaped steps fit up to 819 tokens in decode mode and 1356 in prefill
 *  mode), MOE_ERR_HIP when the scratch address cannot be
 *  obtained, else those of moe_w4a16_grouped_ffn.
 *  All calls on one GPU share its scratch, which keeps the last call's contents:
 *  calls that overlap on one GPU (concurrent streams or threads) race and give
 *  undefined results; order them on one stream or by events.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64ll << 20)
int moe_w4a16_grouped_ffn_noalloc(const moe_ffn_args* args, void* stream);

/*
 * moe_decode_layer -- one decode step of the whole layer (router, top-k,
 * grouped gate/up + SwiGLU, grouped down, routing-weighted combine) for at most
 * 16 tokens, in two launches (ExactMoE, Abstract: the BF16 router with its
 * unchanged top-k and every selected expert through fused grouped kernels).
 * Routing overlaps the start of the weight stream; no expert-sorted permutation
 * is formed (h rows are kept in pair order).  logits, topk_ids and topk_weights
 * are bit-identical to moe_route_align; out equals moe_w4a16_grouped_ffn
 * (combine = 1, no slot table) on them bit for bit when that call accumulates
 * each gate/up item's K range in one wavefront (many active experts), else up
 * to the fp32 summation order (it splits K over two wavefronts when few experts
 * are active).
 *
 *  x [T][d] bf16, w_router [E][d] bf16 (16-byte aligned); bank: expert blobs
 *  (layout v1, 256-byte aligned, stride >= blob bytes, multiple of 256, below
 *  2^31); outputs logits [T][E] fp32, topk_ids [T][k], topk_weights [T][k], out
 *  [T][d] bf16; workspace of moe_decode_layer_workspace_bytes (256-byte
 *  aligned).  counters: MOE_DECODE_LAYER_COUNTERS int32 of device memory owned
 *  by the caller, all zero before the first call; every call leaves them zero,
 *  except counters[MOE_DECODE_LAYER_COUNTERS - 1], which a call sets to 1 if a
 *  workgroup gave up waiting for the routing (its results are then invalid).
 *  Calls sharing a counters buffer must not overlap.
 *  Limits: 1 <= T <= 16 (T == 0 is a no-op), d <= 4096, d and I multiples of
 *  128, E <= 1024, k <= min(E, 16); MOE_ERR_UNSUPPORTED_SHAPE otherwise.
 */
#define MOE_DECODE_LAYER_COUNTERS 1024
typedef struct {
  const uint16_t* x;
  const uint16_t* w_router;
  int T, d, I, E, k;
  int renormalize;
  const uint8_t* bank;
  int64_t bank_stride;
  float* logits;
  int32_t* topk_ids;
  float* topk_weights;
  uint16_t* out;
  void* workspace;
  int64_t workspace_bytes;
  int32_t* counters;
} moe_decode_layer_args;
int64_t moe_decode_layer_workspace_bytes(int T, int d, int I, int E, int k);
int moe_decode_layer(const moe_decode_layer_args* args, void* stream);

/*
 * BF16 experts: the same grouped pass over unquantised experts, the BF16 side of
 * the page's four-bit versus BF16 decode comparison (ExactMoE, Abstract: W4A16
 * experts against the BF16 model).
 *
 * moe_bf16_expert_bytes: bytes of one BF16 expert blob, 6 * d * I: W13 [2I][d]
 *   (gate rows 0..I-1, then up rows) followed by W2 [d][I], bf16 row-major.
 *   -1 for non-positive sizes.
 * moe_bf16_pack: copy E experts' w13 [E][2I][d] and w2 [E][d][I] (device bf16,
 *   contiguous) into a bank of blobs at bank_stride bytes (device-to-device
 *   copies on `stream`).  Errors: MOE_ERR_INVALID_ARG (sizes, NULL, stride below
 *   the blob size), MOE_ERR_HIP (copy could not be enqueued).
 * moe_bf16_grouped_ffn: gate/up + SwiGLU, down and combine as
 *   moe_w4a16_grouped_ffn, with `bank` holding BF16 blobs (256-byte aligned,
 *   stride >= moe_bf16_expert_bytes and a multiple of 256) and slot_of_expert /
 *   combine as there.  `mode` is ignored.  The workspace must hold
 *   moe_ffn_workspace_bytes(T, d, I, E, k, MOE_MODE_DECODE) bytes.  Limits: those
 *   of moe_w4a16_grouped_ffn, and T * d and T * k * I below 2^30.
 */
int64_t moe_bf16_expert_bytes(int d, int I);
int moe_bf16_pack(const uint16_t* w13, const uint16_t* w2, int E, int d, int I, uint8_t* bank,
                  int64_t bank_stride, void* stream);
int moe_bf16_grouped_ffn(const moe_ffn_args* args, void* stream);

/*
 * Nested two/four-bit experts (page "MatMoE: Dynamic Mixed-Precision
 * Quantization for Efficient MoE Inference", arXiv abstract: one nested
 * multi-precision representation, floor-and-compensation quantisation, each
 * expert's bit-width from its routing scores), built on the four-bit codes of
 * pack_w4_g128.
 *
 * Layout m1: each code c = q + 8 = 4h + l split into a high plane (h) and a low
 * plane (l); plane tiles of 16 rows x 256 columns (two groups, 1024 bytes) at
 * (row tile * K/256 + column tile) * 1024, rows in the gate/up interleaved order
 * of layout v1, the bf16 scales of layout v1; lane L of a wavefront owns 16 bytes
 * of each tile: 32-bit words j = 0..3 with K steps 2j, 2j+1 of row L % 16,
 * columns 32 i + 8 (L / 16) + m; element m of K step 2j + t has its 2-bit field
 * at bit (5 + 2 (4t + m/2) + 16 (m % 2)) mod 32.  Expert blob: w13 high plane |
 * w13 scales | w2 high plane | w2 scales | w13 low plane | w2 low plane, each
 * 256-byte aligned (moe_mat_layout_get; same blob size as layout v1): the first
 * two_bit_bytes hold everything an expert reads at two bits, so a two-bit load
 * of an expert is one copy of that prefix.
 *
 * moe_mat_layout_get: section offsets, blob bytes and the two-bit prefix for d, I
 *   (multiples of 256).
 * moe_mat_from_w4: rewrite E four-bit blobs (layout v1, from pack_w4_g128) as
 *   layout-m1 blobs (device to device on `stream`; same codes and scales).
 * moe_mat_grouped_ffn: the grouped pass with a per-expert precision: an expert
 *   runs at four bits, (4h + l - 8) * s = q * s, when the largest routing weight
 *   among its pairs in this step is >= tau, else at two bits with the dropped
 *   bits compensated by their mean, (4h + 1.5 - 8) * s, reading only the high
 *   plane.  Arguments as moe_w4a16_grouped_ffn with `bank` holding layout-m1
 *   blobs; `mode` ignored; workspace of moe_ffn_workspace_bytes(..., MOE_MODE_DECODE).
 *   Limits: T <= 16, d <= 4096, d and I multiples of 256 (decode steps;
 *   MOE_ERR_UNSUPPORTED_SHAPE otherwise), and those of moe_w4a16_grouped_ffn.
 */
typedef struct {
  int64_t w13_hi, w13_lo, w13_scales, w2_hi, w2_lo, w2_scales, blob_bytes;
  int64_t two_bit_bytes;  /* the two-bit part: bytes [0, two_bit_bytes) of the blob */
} moe_mat_layout;
int moe_mat_layout_get(int d, int I, moe_mat_layout* out);
int moe_mat_from_w4(const uint8_t* w4_bank, int64_t w4_stride, int E, int d, int I, uint8_t* mat_bank,
                    int64_t mat_stride, void* stream);
int moe_mat_grouped_ffn(const moe_ffn_args* args, float tau, void* stream);

/*
 * moe_mat_decode_layer: one decode step of the whole layer as moe_decode_layer
 *   (router, top-k, gate/up + SwiGLU, down, combine in two launches, same
 *   arguments, workspace, counters and limits) with `bank` holding layout-m1
 *   blobs (stride >= their blob bytes) and each expert's precision chosen as in
 *   moe_mat_grouped_ffn: four bits when the largest routing weight of its pairs
 *   in this step is >= tau, else two bits.  tau <= 0 puts every expert at four
 *   bits (out then equals moe_decode_layer on the layout-v1 blobs the nested ones
 *   were made from, bit for bit), tau > 1 every expert at two bits.  Limits: those
 *   of moe_decode_layer, with d and I multiples of 256; MOE_ERR_INVALID_ARG for a
 *   NaN tau.
 */
int moe_mat_decode_layer(const moe_decode_layer_args* args, float tau, void* stream);

/*
 * Expert slot cache (ExactMoE, Abstract: quantised experts in pinned host
 * memory, executed from a configurable GPU-resident slot cache).
 *
 * moe_slot_cache_create: host bookkeeping for E experts and S device slots.
 *   host_store   pinned host memory (hipHostMalloc), E blobs at blob_bytes stride.
 *   device_slots device memory, S blobs at blob_bytes stride.
 *   The cache allocates (once, here) a small ring of pinned host staging
 *   tables for the expert->slot map; nothing is allocated afterwards.
 * slot_cache_load: one round for the pending experts (host bitmask, ceil(E/64)
 *   words).  Takes the pending experts already resident (hits), then missing ones
 *   until the S slots are full; each miss replaces a slot not holding a hit.
 *   LRU policy (the default): misses in ascending id, victims least recently
 *   used (empty slots first, ties to the lower slot); moe_slot_cache_configure
 *   selects the cost-aware order instead.  On copy_stream, after wait_event (may be NULL; record it after the
 *   last kernel that read the slots), it enqueues the H2D copies of the misses,
 *   then the copy of the round's expert->slot table into slot_table_dev ([E]
 *   int32: slot of each expert of this round, -1 for every other expert), and
 *   records done_event (the grouped kernels wait on it).
 *   round_mask (host out, ceil(E/64) words) = experts of this round; the caller
 *   clears them from pending and calls again until nothing is pending (one round
 *   when the pending set fits in S).  n_hits / n_misses (host out, may be NULL).
 *   Errors: MOE_ERR_HIP when a copy cannot be enqueued; the slot it was meant
 *   for is then marked empty, so no slot is ever reported half-loaded.
 */
typedef struct moe_slot_cache moe_slot_cache;
int moe_slot_cache_create(int E, int S, int64_t blob_bytes, const void* host_store,
                          void* device_slots, moe_slot_cache** out);
int moe_slot_cache_destroy(moe_slot_cache* cache);
int slot_cache_load(moe_slot_cache* cache, const uint64_t* pending_mask, uint64_t* round_mask,
                    int32_t* slot_table_dev, int32_t* n_hits, int32_t* n_misses,
                    void* copy_stream, void* wait_event, void* done_event);
/* slot_cache_prefetch: copy experts expected to be needed soon (host bitmask
 *   `predicted`, ceil(E/64) words) ahead of their round, so that the copies
 *   overlap other work (the next-layer prefetch: issued while an earlier layer
 *   computes).  The predicted experts not resident, in ascending id and at most
 *   max_copies of them, go into victim slots chosen among the slots not holding a
 *   predicted expert (empty slots first, then least recently used, ties to the
 *   lower slot); they are then resident and count as hits when a round needs
 *   them.  Copies are enqueued on copy_stream after wait_event (may be NULL; pass
 *   an event recorded after the last kernel that read this cache's slots); the
 *   next slot_cache_load on the same copy stream is ordered after them.
 *   n_copies (host out, may be NULL).  Errors: MOE_ERR_INVALID_ARG, MOE_ERR_HIP
 *   (a copy could not be enqueued; its slot is then marked empty).
 */
int slot_cache_prefetch(moe_slot_cache* cache, const uint64_t* predicted_mask, int max_copies,
                        int32_t* n_copies, void* copy_stream, void* wait_event);

/*
 * moe_slot_cache_configure -- replacement policy and copy streams of a cache
 * (page "MoE-APEX: An Efficient MoE Inference System with Adaptive Precision
 * Expert Offloading", "Why it works": prefetching hides the transfer, a
 * cost-aware cache keeps the right experts resident).
 *  policy  MOE_SLOT_POLICY_LRU (the default, as described above) or
 *          MOE_SLOT_POLICY_COST: every expert carries an average u of "needed in
 *          a step" over the sequence (u <- decay * u + (1 - decay) * [needed],
 *          updated by slot_cache_begin_step); victims are empty slots first, then
 *          the lowest expected reload cost (u times the slot's bytes, the same for
 *          every slot), then least recently used, then the lower slot; misses enter
 *          a round in increasing u (ties ascending id) and prefetches in
 *          decreasing u (ties ascending id).
 *  decay   in [0, 1).
 *  copy_streams  1, or 2: the cache creates one stream of its own (default
 *          priority) and alternates the copies of a call between the caller's
 *          copy stream and it (two DMA engines share the host link); before its
 *          copies the second stream waits for wait_event, and the caller's copy
 *          stream waits for them before the slot table copy and done_event, so
 *          the ordering seen by the caller is unchanged.
 *  Errors: MOE_ERR_INVALID_ARG, MOE_ERR_HIP (stream or event creation).
 * slot_cache_begin_step -- the needed experts of a new step (host bitmask,
 *  ceil(E/64) words), before its first slot_cache_load: updates the usage
 *  averages (every policy keeps them; only MOE_SLOT_POLICY_COST uses them).
 */
enum moe_slot_policy { MOE_SLOT_POLICY_LRU = 0, MOE_SLOT_POLICY_COST = 1 };
int moe_slot_cache_configure(moe_slot_cache* cache, int policy, double decay, int copy_streams);
int slot_cache_begin_step(moe_slot_cache* cache, const uint64_t* needed_mask);

/*
 * Precision-aware loads (page "MoE-APEX: An Efficient MoE Inference System with
 * Adaptive Precision Expert Offloading", "This paper's idea": a cache-miss expert
 * that is less critical for the current tokens is loaded as a smaller
 * low-precision variant).  For stores of nested two/four-bit blobs (layout m1,
 * whose first two_bit_bytes hold everything an expert reads at two bits).
 * moe_slot_cache_set_prefix: declare that prefix (0 switches it off) while the
 *   cache is empty.  A slot then holds an expert's whole blob or only its prefix.
 * slot_cache_load_precision: slot_cache_load with full_mask (host bitmask,
 *   ceil(E/64) words): the pending experts needed at four bits (the others at two
 *   bits; moe_mat_grouped_ffn makes the same choice from the routing weights and
 *   tau, so the caller passes the experts whose largest routing weight in the step
 *   reaches tau).  Hits keep their slot; a resident expert holding only its
 *   prefix that is needed at four bits gets the rest of its blob copied into its
 *   slot; a miss copies the prefix (two bits) or the whole blob (four bits).  The
 *   cost-aware policy weighs usage by the bytes a slot holds.  bytes_copied (host
 *   out, may be NULL): bytes this round moved.  Errors: those of slot_cache_load,
 *   MOE_ERR_INVALID_ARG without a prefix.
 * moe_slot_cache_planes: [S] 1 where the slot holds the whole blob, the number of
 *   low-plane completions so far, and all bytes copied so far (outputs may be NULL).
 */
int moe_slot_cache_set_prefix(moe_slot_cache* cache, int64_t prefix_bytes);
int slot_cache_load_precision(moe_slot_cache* cache, const uint64_t* pending_mask, const uint64_t* full_mask,
                              uint64_t* round_mask, int32_t* slot_table_dev, int32_t* n_hits, int32_t* n_misses,
                              int64_t* bytes_copied, void* copy_stream, void* wait_event, void* done_event);
int moe_slot_cache_planes(const moe_slot_cache* cache, int32_t* slot_full, int64_t* upgrades,
                          int64_t* bytes_copied);
/* Current slot contents ([S] expert id or -1) and cumulative hit / miss counts. */
int moe_slot_cache_state(const moe_slot_cache* cache, int32_t* slot_expert,
                         int64_t* hits, int64_t* misses);

/*
 * Kernel timing: when enabled, each launch of the named kernel is bracketed by
 * hipEvents on its own stream.  moe_timing_read synchronises on the recorded
 * events and returns the summed duration and launch count since the last reset.
 * Kernel ids: 0 = gate/up (decode), 1 = down (decode), 2 = gate/up (prefill),
 * 3 = down (prefill), 4 = combine, 5 = route logits, 6 = align, 7 = gate/up
 * (BF16 experts), 8 = down (BF16 experts), 9 = gate/up (nested two/four-bit),
 * 10 = down (nested two/four-bit).
 */
int moe_timing_enable(int on);
int moe_timing_reset(void);
int moe_timing_read(int kernel_id, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* W4A16_MOE_H */
