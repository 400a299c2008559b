// Host runtime of the W4A16 MoE library: error state, status strings, blob
// layout, and the per-kernel event timing used by the benchmark.
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"

namespace moe {

static thread_local std::string g_last_error;

// MOE_W4A16_LOG: 0 or unset silent, 1 errors to stderr, 2 also each grouped
// call's choices (read once, at the first message)
int log_level() {
  static const int level = [] {
    const char* v = std::getenv("MOE_W4A16_LOG");
    return v ? std::atoi(v) : 0;
  }();
  return level;
}

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  if (log_level() >= 1) std::fprintf(stderr, "[w4a16_moe] error: %s\n", buf);
}

void log_info(const char* fmt, ...) {
  if (log_level() < 2) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[w4a16_moe] %s\n", buf);
}

void clear_error() { g_last_error.clear(); }

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

// ---------------------------------------------------------------- timing

struct TimedLaunch {
  hipEvent_t start, stop;
};

static std::mutex g_timing_mu;
static bool g_timing_on = false;
static std::vector<TimedLaunch> g_pending[K_NUM];
static std::vector<hipEvent_t> g_event_pool;
static double g_total_ms[K_NUM];
static int64_t g_launches[K_NUM];
static int g_open[K_NUM];
static hipEvent_t g_open_start[K_NUM];

static hipEvent_t pool_get() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void timing_begin(int id, hipStream_t s) {
  if (!g_timing_on) return;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  hipEvent_t e = pool_get();
  if (!e) return;
  if (hipEventRecord(e, s) != hipSuccess) return;  // no interval opened
  g_open_start[id] = e;
  g_open[id] = 1;
}

void timing_end(int id, hipStream_t s) {
  if (!g_timing_on) return;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (!g_open[id]) return;
  hipEvent_t e = pool_get();
  if (!e) return;
  if (hipEventRecord(e, s) != hipSuccess) {  // the interval is dropped
    g_open[id] = 0;
    return;
  }
  g_pending[id].push_back({g_open_start[id], e});
  g_open[id] = 0;
}

static void drain_locked() {
  for (int id = 0; id < K_NUM; ++id) {
    for (auto& tl : g_pending[id]) {
      (void)hipEventSynchronize(tl.stop);  // on failure the elapsed-time query fails too and the sample is skipped
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, tl.start, tl.stop) == hipSuccess) {
        g_total_ms[id] += ms;
        g_launches[id] += 1;
      }
      g_event_pool.push_back(tl.start);
      g_event_pool.push_back(tl.stop);
    }
    g_pending[id].clear();
  }
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "MOE_ERR_UNSUPPORTED_SHAPE";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_CAPACITY: return "MOE_ERR_CAPACITY";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_abi_version(void) { return 1; }

int moe_expert_layout_get(int d, int I, moe_expert_layout* out) {
  clear_error();
  MOE_CHECK_ARG(out != nullptr, MOE_ERR_INVALID_ARG, "moe_expert_layout_get: out is NULL");
  MOE_CHECK_ARG(d > 0 && I > 0, MOE_ERR_INVALID_ARG, "moe_expert_layout_get: d=%d I=%d", d, I);
  MOE_CHECK_ARG(d % kGroup == 0 && I % kGroup == 0, MOE_ERR_UNSUPPORTED_SHAPE,
                "moe_expert_layout_get: d=%d and I=%d must be multiples of 128", d, I);
  auto up = [](int64_t v) { return (v + 255) / 256 * 256; };
  int64_t o = 0;
  out->w13_codes = o;
  o = up(o + (int64_t)2 * I * d / 2);
  out->w13_scales = o;
  o = up(o + (int64_t)2 * I * (d / kGroup) * 2);
  out->w2_codes = o;
  o = up(o + (int64_t)d * I / 2);
  out->w2_scales = o;
  o = up(o + (int64_t)d * (I / kGroup) * 2);
  out->blob_bytes = o;
  return MOE_OK;
}

int moe_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing_on = on != 0;
  return MOE_OK;
}

int moe_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  drain_locked();
  for (int i = 0; i < K_NUM; ++i) {
    g_total_ms[i] = 0;
    g_launches[i] = 0;
  }
  return MOE_OK;
}

int moe_timing_read(int kernel_id, double* total_ms, int64_t* launches) {
  clear_error();
  MOE_CHECK_ARG(kernel_id >= 0 && kernel_id < K_NUM, MOE_ERR_INVALID_ARG,
                "moe_timing_read: kernel id %d out of range", kernel_id);
  std::lock_guard<std::mutex> lk(g_timing_mu);
  drain_locked();
  if (total_ms) *total_ms = g_total_ms[kernel_id];
  if (launches) *launches = g_launches[kernel_id];
  return MOE_OK;
}

}  // extern "C"
