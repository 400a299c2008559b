// GPU-resident expert slot cache over a pinned-host expert store (ExactMoE, page
// "Every Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference",
// Abstract: quantised experts stored in pinned host memory and executed through
// a configurable GPU-resident slot cache).  Host-side bookkeeping only: the
// policy (hits first, then misses in ascending id; victims = empty slots, then
// least recently used, ties to the lower slot) runs on the CPU and the data
// moves by hipMemcpyAsync on the caller's copy stream.
#include <cstdlib>
#include <cstring>
#include <vector>

#include "common.hpp"

struct moe_slot_cache {
  int E = 0, S = 0;
  int64_t blob_bytes = 0;
  const uint8_t* host_store = nullptr;
  uint8_t* device_slots = nullptr;
  std::vector<int> slot_expert;    // [S] expert in slot or -1
  std::vector<int64_t> slot_stamp; // [S] last round that used the slot, -1 if never
  std::vector<int> expert_slot;    // [E] slot of expert or -1
  int64_t clock = 0, hits = 0, misses = 0, prefetches = 0;
  // ring of pinned staging tables for the per-round expert->slot map
  static constexpr int kRing = 8;
  int32_t* tables = nullptr;       // [kRing][E], pinned
  hipEvent_t table_ev[kRing] = {};
  bool table_used[kRing] = {};
  int ring_next = 0;
  int fail_after = -1;             // test hook: copies allowed before an injected failure
};

using namespace moe;

extern "C" int moe_slot_cache_create(int E, int S, int64_t blob_bytes, const void* host_store, void* device_slots,
                                     moe_slot_cache** out) {
  clear_error();
  MOE_CHECK_ARG(out != nullptr, MOE_ERR_INVALID_ARG, "moe_slot_cache_create: out is NULL");
  *out = nullptr;
  MOE_CHECK_ARG(E > 0 && E <= MOE_MAX_EXPERTS && S > 0 && blob_bytes > 0, MOE_ERR_INVALID_ARG,
                "moe_slot_cache_create: bad sizes E=%d S=%d blob_bytes=%lld", E, S, (long long)blob_bytes);
  MOE_CHECK_ARG(host_store && device_slots, MOE_ERR_INVALID_ARG, "moe_slot_cache_create: null store or slots");
  auto* c = new moe_slot_cache();
  c->E = E;
  c->S = S;
  c->blob_bytes = blob_bytes;
  c->host_store = static_cast<const uint8_t*>(host_store);
  c->device_slots = static_cast<uint8_t*>(device_slots);
  c->slot_expert.assign(S, -1);
  c->slot_stamp.assign(S, -1);
  c->expert_slot.assign(E, -1);
  if (hipHostMalloc(reinterpret_cast<void**>(&c->tables), sizeof(int32_t) * E * moe_slot_cache::kRing,
                    hipHostMallocDefault) != hipSuccess) {
    delete c;
    set_error("moe_slot_cache_create: pinned staging allocation failed");
    return MOE_ERR_HIP;
  }
  for (int i = 0; i < moe_slot_cache::kRing; ++i) {
    if (hipEventCreateWithFlags(&c->table_ev[i], hipEventDisableTiming) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(c->table_ev[j]);
      (void)hipHostFree(c->tables);
      delete c;
      set_error("moe_slot_cache_create: event creation failed");
      return MOE_ERR_HIP;
    }
  }
  if (const char* f = getenv("MOE_SLOT_CACHE_FAIL_AFTER")) c->fail_after = atoi(f);
  *out = c;
  return MOE_OK;
}

extern "C" int moe_slot_cache_destroy(moe_slot_cache* c) {
  clear_error();
  if (!c) return MOE_OK;
  for (int i = 0; i < moe_slot_cache::kRing; ++i) {
    if (c->table_used[i]) (void)hipEventSynchronize(c->table_ev[i]);
    (void)hipEventDestroy(c->table_ev[i]);
  }
  (void)hipHostFree(c->tables);
  delete c;
  return MOE_OK;
}

extern "C" int slot_cache_load(moe_slot_cache* c, const uint64_t* pending_mask, uint64_t* round_mask,
                               int32_t* slot_table_dev, int32_t* n_hits, int32_t* n_misses, void* copy_stream,
                               void* wait_event, void* done_event) {
  clear_error();
  MOE_CHECK_ARG(c && pending_mask && round_mask && slot_table_dev && done_event, MOE_ERR_INVALID_ARG,
                "slot_cache_load: null argument");
  hipStream_t s = (hipStream_t)copy_stream;
  const int E = c->E, S = c->S, words = (E + 63) / 64;

  std::vector<int> hits, miss_all;
  for (int e = 0; e < E; ++e) {
    if (!((pending_mask[e >> 6] >> (e & 63)) & 1ull)) continue;
    if (c->expert_slot[e] >= 0)
      hits.push_back(e);
    else
      miss_all.push_back(e);
  }
  const int n_m = std::min<int>((int)miss_all.size(), S - (int)hits.size());
  std::vector<char> hit_slot(S, 0);
  for (int e : hits) hit_slot[c->expert_slot[e]] = 1;
  std::vector<int> victims;
  for (int sl = 0; sl < S; ++sl)
    if (!hit_slot[sl]) victims.push_back(sl);
  std::stable_sort(victims.begin(), victims.end(),
                   [&](int a, int b) { return c->slot_stamp[a] < c->slot_stamp[b]; });

  if (wait_event) {
    if (hipStreamWaitEvent(s, (hipEvent_t)wait_event, 0) != hipSuccess) {
      set_error("slot_cache_load: hipStreamWaitEvent failed");
      return MOE_ERR_HIP;
    }
  }
  std::vector<int> loaded;
  int rc = MOE_OK;
  for (int i = 0; i < n_m; ++i) {
    const int e = miss_all[i], sl = victims[i];
    const int old = c->slot_expert[sl];
    if (old >= 0) c->expert_slot[old] = -1;
    c->slot_expert[sl] = -1;
    c->slot_stamp[sl] = -1;
    hipError_t err = hipSuccess;
    if (c->fail_after == 0) {
      err = hipErrorInvalidValue;
    } else {
      if (c->fail_after > 0) --c->fail_after;
      err = hipMemcpyAsync(c->device_slots + (int64_t)sl * c->blob_bytes, c->host_store + (int64_t)e * c->blob_bytes,
                           c->blob_bytes, hipMemcpyHostToDevice, s);
    }
    if (err != hipSuccess) {
      set_error("slot_cache_load: H2D copy of expert %d into slot %d failed: %s", e, sl, hipGetErrorString(err));
      rc = MOE_ERR_HIP;
      break;
    }
    c->slot_expert[sl] = e;
    c->expert_slot[e] = sl;
    loaded.push_back(e);
  }
  if (rc) return rc;

  c->clock += 1;
  for (int e : hits) c->slot_stamp[c->expert_slot[e]] = c->clock;
  for (int e : loaded) c->slot_stamp[c->expert_slot[e]] = c->clock;
  c->hits += (int64_t)hits.size();
  c->misses += (int64_t)loaded.size();

  for (int w = 0; w < words; ++w) round_mask[w] = 0;
  const int slot_idx = c->ring_next;
  c->ring_next = (c->ring_next + 1) % moe_slot_cache::kRing;
  if (c->table_used[slot_idx]) (void)hipEventSynchronize(c->table_ev[slot_idx]);
  int32_t* table = c->tables + (int64_t)slot_idx * E;
  for (int e = 0; e < E; ++e) table[e] = -1;
  for (int e : hits) {
    table[e] = c->expert_slot[e];
    round_mask[e >> 6] |= 1ull << (e & 63);
  }
  for (int e : loaded) {
    table[e] = c->expert_slot[e];
    round_mask[e >> 6] |= 1ull << (e & 63);
  }
  if (hipMemcpyAsync(slot_table_dev, table, sizeof(int32_t) * E, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipEventRecord(c->table_ev[slot_idx], s) != hipSuccess || hipEventRecord((hipEvent_t)done_event, s) != hipSuccess) {
    set_error("slot_cache_load: slot table copy failed");
    return MOE_ERR_HIP;
  }
  c->table_used[slot_idx] = true;
  if (n_hits) *n_hits = (int32_t)hits.size();
  if (n_misses) *n_misses = (int32_t)loaded.size();
  return MOE_OK;
}

extern "C" int slot_cache_prefetch(moe_slot_cache* c, const uint64_t* predicted_mask, int max_copies,
                                   int32_t* n_copies, void* copy_stream, void* wait_event) {
  clear_error();
  MOE_CHECK_ARG(c && predicted_mask && max_copies >= 0, MOE_ERR_INVALID_ARG, "slot_cache_prefetch: bad argument");
  hipStream_t s = (hipStream_t)copy_stream;
  const int E = c->E, S = c->S;
  std::vector<int> want;
  std::vector<char> keep(S, 0);
  for (int e = 0; e < E; ++e) {
    if (!((predicted_mask[e >> 6] >> (e & 63)) & 1ull)) continue;
    if (c->expert_slot[e] >= 0)
      keep[c->expert_slot[e]] = 1;
    else
      want.push_back(e);
  }
  std::vector<int> victims;
  for (int sl = 0; sl < S; ++sl)
    if (!keep[sl]) victims.push_back(sl);
  std::stable_sort(victims.begin(), victims.end(),
                   [&](int a, int b) { return c->slot_stamp[a] < c->slot_stamp[b]; });
  const int n = std::min<int>(std::min<int>((int)want.size(), (int)victims.size()), max_copies);
  if (n > 0 && wait_event && hipStreamWaitEvent(s, (hipEvent_t)wait_event, 0) != hipSuccess) {
    set_error("slot_cache_prefetch: hipStreamWaitEvent failed");
    return MOE_ERR_HIP;
  }
  c->clock += 1;
  int done = 0;
  for (int i = 0; i < n; ++i) {
    const int e = want[i], sl = victims[i];
    const int old = c->slot_expert[sl];
    if (old >= 0) c->expert_slot[old] = -1;
    c->slot_expert[sl] = -1;
    c->slot_stamp[sl] = -1;
    hipError_t err = hipSuccess;
    if (c->fail_after == 0) {
      err = hipErrorInvalidValue;
    } else {
      if (c->fail_after > 0) --c->fail_after;
      err = hipMemcpyAsync(c->device_slots + (int64_t)sl * c->blob_bytes, c->host_store + (int64_t)e * c->blob_bytes,
                           c->blob_bytes, hipMemcpyHostToDevice, s);
    }
    if (err != hipSuccess) {
      set_error("slot_cache_prefetch: H2D copy of expert %d into slot %d failed: %s", e, sl, hipGetErrorString(err));
      if (n_copies) *n_copies = done;
      return MOE_ERR_HIP;
    }
    c->slot_expert[sl] = e;
    c->expert_slot[e] = sl;
    c->slot_stamp[sl] = c->clock;
    ++done;
  }
  c->prefetches += done;
  if (n_copies) *n_copies = done;
  return MOE_OK;
}

extern "C" int moe_slot_cache_state(const moe_slot_cache* c, int32_t* slot_expert, int64_t* hits, int64_t* misses) {
  clear_error();
  MOE_CHECK_ARG(c != nullptr, MOE_ERR_INVALID_ARG, "moe_slot_cache_state: cache is NULL");
  if (slot_expert)
    for (int s = 0; s < c->S; ++s) slot_expert[s] = c->slot_expert[s];
  if (hits) *hits = c->hits;
  if (misses) *misses = c->misses;
  return MOE_OK;
}
