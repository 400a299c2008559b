// GPU-resident expert slot cache over a pinned-host expert store (ExactMoE, page
// "Every Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference",
// Abstract: quantised experts stored in pinned host memory and executed through
// a configurable GPU-resident slot cache).  Host-side bookkeeping only: the
// policy runs on the CPU and the data moves by hipMemcpyAsync on the caller's
// copy stream (and, when configured, a second stream of the cache's own, so two
// copy engines share the host link).
// Policies: LRU (hits first, then misses in ascending id; victims = empty slots,
// then least recently used, ties to the lower slot) and cost-aware (page
// "MoE-APEX: An Efficient MoE Inference System with Adaptive Precision Expert
// Offloading", "Why it works": a sequence-level cache keeps resident the experts
// whose reload would cost most): every expert carries an exponential average of
// "needed in this step" over the sequence; victims go by expected reload cost
// (that average times the slot's bytes), then least recently used, then lower
// slot; misses enter a round in increasing expected cost, so the experts likely
// needed again are loaded last and stay.
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
  int policy = MOE_SLOT_POLICY_LRU;
  double decay = 0.9;
  std::vector<double> usage;       // [E] cost-aware: average of "needed in a step"
  int64_t prefix_bytes = 0;        // > 0: precision-aware, a blob's first prefix_bytes are its two-bit part
  std::vector<char> slot_full;     // [S] the slot holds the whole blob (else only the prefix)
  int64_t upgrades = 0, bytes_copied = 0;
  hipStream_t aux = nullptr;       // second copy stream (copy_streams = 2)
  hipEvent_t aux_done = nullptr;   // the aux stream's copies, joined into the caller's copy stream
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
  c->usage.assign(E, 0.0);
  c->slot_full.assign(S, 0);
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
  if (c->aux) {
    (void)hipStreamSynchronize(c->aux);
    (void)hipStreamDestroy(c->aux);
    (void)hipEventDestroy(c->aux_done);
  }
  (void)hipHostFree(c->tables);
  delete c;
  return MOE_OK;
}

extern "C" int moe_slot_cache_configure(moe_slot_cache* c, int policy, double decay, int copy_streams) {
  clear_error();
  MOE_CHECK_ARG(c != nullptr, MOE_ERR_INVALID_ARG, "moe_slot_cache_configure: cache is NULL");
  MOE_CHECK_ARG(policy == MOE_SLOT_POLICY_LRU || policy == MOE_SLOT_POLICY_COST, MOE_ERR_INVALID_ARG,
                "moe_slot_cache_configure: unknown policy %d", policy);
  MOE_CHECK_ARG(decay >= 0.0 && decay < 1.0, MOE_ERR_INVALID_ARG, "moe_slot_cache_configure: decay %g not in [0, 1)",
                decay);
  MOE_CHECK_ARG(copy_streams == 1 || copy_streams == 2, MOE_ERR_INVALID_ARG,
                "moe_slot_cache_configure: copy_streams must be 1 or 2, got %d", copy_streams);
  if (copy_streams == 2 && !c->aux) {
    if (hipStreamCreateWithFlags(&c->aux, hipStreamNonBlocking) != hipSuccess) {
      c->aux = nullptr;
      set_error("moe_slot_cache_configure: stream creation failed");
      return MOE_ERR_HIP;
    }
    if (hipEventCreateWithFlags(&c->aux_done, hipEventDisableTiming) != hipSuccess) {
      (void)hipStreamDestroy(c->aux);
      c->aux = nullptr;
      set_error("moe_slot_cache_configure: event creation failed");
      return MOE_ERR_HIP;
    }
  } else if (copy_streams == 1 && c->aux) {
    (void)hipStreamSynchronize(c->aux);
    (void)hipStreamDestroy(c->aux);
    (void)hipEventDestroy(c->aux_done);
    c->aux = nullptr;
    c->aux_done = nullptr;
  }
  c->policy = policy;
  c->decay = decay;
  return MOE_OK;
}

extern "C" int slot_cache_begin_step(moe_slot_cache* c, const uint64_t* needed_mask) {
  clear_error();
  MOE_CHECK_ARG(c && needed_mask, MOE_ERR_INVALID_ARG, "slot_cache_begin_step: null argument");
  for (int e = 0; e < c->E; ++e) {
    const double need = ((needed_mask[e >> 6] >> (e & 63)) & 1ull) ? 1.0 : 0.0;
    c->usage[e] = c->decay * c->usage[e] + (1.0 - c->decay) * need;
  }
  return MOE_OK;
}

namespace {

// victim order over the candidate slots: empty first; cost-aware: expected reload
// cost (usage; every slot reloads the same bytes), then last use, then slot;
// LRU: last use, then slot
void order_victims(const moe_slot_cache* c, std::vector<int>& v) {
  if (c->policy == MOE_SLOT_POLICY_COST) {
    // precision-aware: usage times the bytes the slot holds (its reload would copy them)
    auto cost = [&](int sl) {
      const int e = c->slot_expert[sl];
      if (c->prefix_bytes <= 0) return c->usage[e];
      return c->usage[e] * (double)(c->slot_full[sl] ? c->blob_bytes : c->prefix_bytes);
    };
    std::sort(v.begin(), v.end(), [&](int a, int b) {
      const int ea = c->slot_expert[a], eb = c->slot_expert[b];
      if ((ea >= 0) != (eb >= 0)) return ea < 0;
      if (ea >= 0 && cost(a) != cost(b)) return cost(a) < cost(b);
      if (c->slot_stamp[a] != c->slot_stamp[b]) return c->slot_stamp[a] < c->slot_stamp[b];
      return a < b;
    });
  } else {
    std::stable_sort(v.begin(), v.end(), [&](int a, int b) { return c->slot_stamp[a] < c->slot_stamp[b]; });
  }
}

// the copy of expert e into slot sl: the i-th copy of a call goes to the caller's
// stream (even i) or the cache's second stream (odd i, when configured)
hipError_t copy_expert(moe_slot_cache* c, int e, int sl, int i, hipStream_t s, int64_t off = 0, int64_t bytes = -1) {
  if (bytes < 0) bytes = c->blob_bytes - off;
  if (c->fail_after == 0) return hipErrorInvalidValue;
  if (c->fail_after > 0) --c->fail_after;
  hipStream_t cs = (c->aux && (i & 1)) ? c->aux : s;
  c->bytes_copied += bytes;
  return hipMemcpyAsync(c->device_slots + (int64_t)sl * c->blob_bytes + off,
                        c->host_store + (int64_t)e * c->blob_bytes + off, bytes, hipMemcpyHostToDevice, cs);
}

// before the copies: the second stream waits for what the caller's stream waits for
hipError_t aux_wait(moe_slot_cache* c, hipStream_t s, void* wait_event) {
  if (!c->aux) return hipSuccess;
  if (wait_event) return hipStreamWaitEvent(c->aux, (hipEvent_t)wait_event, 0);
  // no event: order the aux stream after the work already on the caller's stream
  hipError_t e = hipEventRecord(c->aux_done, s);
  return e == hipSuccess ? hipStreamWaitEvent(c->aux, c->aux_done, 0) : e;
}

// after the copies: the caller's stream waits for the second stream's copies
hipError_t aux_join(moe_slot_cache* c, hipStream_t s, int n_copies) {
  if (!c->aux || n_copies < 2) return hipSuccess;
  hipError_t e = hipEventRecord(c->aux_done, c->aux);
  return e == hipSuccess ? hipStreamWaitEvent(s, c->aux_done, 0) : e;
}

}  // namespace

// One round (slot_cache_load / slot_cache_load_precision).  full_mask NULL: every
// pending expert needs its whole blob.
static int load_round(moe_slot_cache* c, const uint64_t* pending_mask, const uint64_t* full_mask,
                      uint64_t* round_mask, int32_t* slot_table_dev, int32_t* n_hits, int32_t* n_misses,
                      int64_t* bytes_out, hipStream_t s, void* wait_event, void* done_event, const char* fn) {
  const int E = c->E, S = c->S, words = (E + 63) / 64;
  const bool mixed = c->prefix_bytes > 0;
  auto needs_full = [&](int e) { return !mixed || !full_mask || ((full_mask[e >> 6] >> (e & 63)) & 1ull); };
  const int64_t bytes0 = c->bytes_copied;

  std::vector<int> hits, miss_all, upgrade;
  for (int e = 0; e < E; ++e) {
    if (!((pending_mask[e >> 6] >> (e & 63)) & 1ull)) continue;
    if (c->expert_slot[e] >= 0) {
      hits.push_back(e);
      if (needs_full(e) && !c->slot_full[c->expert_slot[e]]) upgrade.push_back(e);
    } else {
      miss_all.push_back(e);
    }
  }
  if (c->policy == MOE_SLOT_POLICY_COST)
    std::stable_sort(miss_all.begin(), miss_all.end(), [&](int a, int b) { return c->usage[a] < c->usage[b]; });
  const int n_m = std::min<int>((int)miss_all.size(), S - (int)hits.size());
  std::vector<char> hit_slot(S, 0);
  for (int e : hits) hit_slot[c->expert_slot[e]] = 1;
  std::vector<int> victims;
  for (int sl = 0; sl < S; ++sl)
    if (!hit_slot[sl]) victims.push_back(sl);
  order_victims(c, victims);

  const int n_copies = (int)upgrade.size() + n_m;
  // also with nothing to copy: the slot table copy below must not overtake the
  // kernels that still read the previous table
  if (wait_event) {
    if (hipStreamWaitEvent(s, (hipEvent_t)wait_event, 0) != hipSuccess) {
      set_error("%s: hipStreamWaitEvent failed", fn);
      return MOE_ERR_HIP;
    }
  }
  if (n_copies > 1 && aux_wait(c, s, wait_event) != hipSuccess) {
    set_error("%s: second copy stream could not be ordered", fn);
    return MOE_ERR_HIP;
  }
  int rc = MOE_OK, issued = 0;
  // resident two-bit experts needed at four bits: their low planes into the same slot
  for (int e : upgrade) {
    const int sl = c->expert_slot[e];
    const hipError_t err = copy_expert(c, e, sl, issued, s, c->prefix_bytes);
    if (err != hipSuccess) {
      set_error("%s: H2D copy of expert %d's low planes into slot %d failed: %s", fn, e, sl, hipGetErrorString(err));
      rc = MOE_ERR_HIP;
      break;
    }
    ++issued;
    c->slot_full[sl] = 1;
    ++c->upgrades;
  }
  std::vector<int> loaded;
  for (int i = 0; i < n_m && !rc; ++i) {
    const int e = miss_all[i], sl = victims[i];
    const int old = c->slot_expert[sl];
    if (old >= 0) c->expert_slot[old] = -1;
    c->slot_expert[sl] = -1;
    c->slot_stamp[sl] = -1;
    c->slot_full[sl] = 0;
    const bool full = needs_full(e);
    const hipError_t err = copy_expert(c, e, sl, issued, s, 0, full ? c->blob_bytes : c->prefix_bytes);
    if (err != hipSuccess) {
      set_error("%s: H2D copy of expert %d into slot %d failed: %s", fn, e, sl, hipGetErrorString(err));
      rc = MOE_ERR_HIP;
      break;
    }
    ++issued;
    c->slot_expert[sl] = e;
    c->expert_slot[e] = sl;
    c->slot_full[sl] = full ? 1 : 0;
    loaded.push_back(e);
  }
  if (aux_join(c, s, issued) != hipSuccess && !rc) {
    set_error("%s: second copy stream could not be joined", fn);
    rc = MOE_ERR_HIP;
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
    set_error("%s: slot table copy failed", fn);
    return MOE_ERR_HIP;
  }
  c->table_used[slot_idx] = true;
  if (n_hits) *n_hits = (int32_t)hits.size();
  if (n_misses) *n_misses = (int32_t)loaded.size();
  if (bytes_out) *bytes_out = c->bytes_copied - bytes0;
  return MOE_OK;
}

extern "C" int slot_cache_load(moe_slot_cache* c, const uint64_t* pending_mask, uint64_t* round_mask,
                               int32_t* slot_table_dev, int32_t* n_hits, int32_t* n_misses, void* copy_stream,
                               void* wait_event, void* done_event) {
  clear_error();
  MOE_CHECK_ARG(c && pending_mask && round_mask && slot_table_dev && done_event, MOE_ERR_INVALID_ARG,
                "slot_cache_load: null argument");
  return load_round(c, pending_mask, nullptr, round_mask, slot_table_dev, n_hits, n_misses, nullptr,
                    (hipStream_t)copy_stream, wait_event, done_event, "slot_cache_load");
}

extern "C" int slot_cache_load_precision(moe_slot_cache* c, const uint64_t* pending_mask, const uint64_t* full_mask,
                                         uint64_t* round_mask, int32_t* slot_table_dev, int32_t* n_hits,
                                         int32_t* n_misses, int64_t* bytes_copied, void* copy_stream,
                                         void* wait_event, void* done_event) {
  clear_error();
  MOE_CHECK_ARG(c && pending_mask && full_mask && round_mask && slot_table_dev && done_event, MOE_ERR_INVALID_ARG,
                "slot_cache_load_precision: null argument");
  MOE_CHECK_ARG(c->prefix_bytes > 0, MOE_ERR_INVALID_ARG,
                "slot_cache_load_precision: the cache has no two-bit prefix (moe_slot_cache_set_prefix)");
  return load_round(c, pending_mask, full_mask, round_mask, slot_table_dev, n_hits, n_misses, bytes_copied,
                    (hipStream_t)copy_stream, wait_event, done_event, "slot_cache_load_precision");
}

extern "C" int moe_slot_cache_set_prefix(moe_slot_cache* c, int64_t prefix_bytes) {
  clear_error();
  MOE_CHECK_ARG(c != nullptr, MOE_ERR_INVALID_ARG, "moe_slot_cache_set_prefix: cache is NULL");
  MOE_CHECK_ARG(prefix_bytes >= 0 && prefix_bytes < c->blob_bytes, MOE_ERR_INVALID_ARG,
                "moe_slot_cache_set_prefix: prefix %lld not in [0, %lld)", (long long)prefix_bytes,
                (long long)c->blob_bytes);
  for (int sl = 0; sl < c->S; ++sl)
    MOE_CHECK_ARG(c->slot_expert[sl] < 0, MOE_ERR_INVALID_ARG, "moe_slot_cache_set_prefix: the cache is not empty");
  c->prefix_bytes = prefix_bytes;
  return MOE_OK;
}

extern "C" int moe_slot_cache_planes(const moe_slot_cache* c, int32_t* slot_full, int64_t* upgrades,
                                     int64_t* bytes_copied) {
  clear_error();
  MOE_CHECK_ARG(c != nullptr, MOE_ERR_INVALID_ARG, "moe_slot_cache_planes: cache is NULL");
  if (slot_full)
    for (int sl = 0; sl < c->S; ++sl) slot_full[sl] = c->slot_full[sl];
  if (upgrades) *upgrades = c->upgrades;
  if (bytes_copied) *bytes_copied = c->bytes_copied;
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
  if (c->policy == MOE_SLOT_POLICY_COST)
    std::stable_sort(want.begin(), want.end(), [&](int a, int b) { return c->usage[a] > c->usage[b]; });
  std::vector<int> victims;
  for (int sl = 0; sl < S; ++sl)
    if (!keep[sl]) victims.push_back(sl);
  order_victims(c, victims);
  const int n = std::min<int>(std::min<int>((int)want.size(), (int)victims.size()), max_copies);
  if (n > 0 && wait_event && hipStreamWaitEvent(s, (hipEvent_t)wait_event, 0) != hipSuccess) {
    set_error("slot_cache_prefetch: hipStreamWaitEvent failed");
    return MOE_ERR_HIP;
  }
  if (n > 1 && aux_wait(c, s, wait_event) != hipSuccess) {
    set_error("slot_cache_prefetch: second copy stream could not be ordered");
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
    c->slot_full[sl] = 0;
    const hipError_t err = copy_expert(c, e, sl, i, s);
    if (err != hipSuccess) {
      set_error("slot_cache_prefetch: H2D copy of expert %d into slot %d failed: %s", e, sl, hipGetErrorString(err));
      (void)aux_join(c, s, done);
      if (n_copies) *n_copies = done;
      return MOE_ERR_HIP;
    }
    c->slot_expert[sl] = e;
    c->expert_slot[e] = sl;
    c->slot_stamp[sl] = c->clock;
    c->slot_full[sl] = 1;
    ++done;
  }
  if (aux_join(c, s, done) != hipSuccess) {
    set_error("slot_cache_prefetch: second copy stream could not be joined");
    if (n_copies) *n_copies = done;
    return MOE_ERR_HIP;
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
