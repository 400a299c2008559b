// moe_w4a16_grouped_ffn: host dispatch of the fused grouped expert pass and the
// routing-weighted combine (ExactMoE, page "Every Expert Counts: ExactMoE for
// Memory-Efficient W4A16 Inference", Abstract: every selected expert executes
// through fused grouped kernels; none is pruned or substituted).
//
// Workspace: h [T*k][I] bf16 (SwiGLU output, expert-sorted rows) followed by
// y [ksplit][T*k][d] fp32 (down-projection partials, expert-sorted rows).
// The combine reads y through pair_pos, sums the K-split partials in a fixed
// order and the k routed outputs in slot order, in fp32, and rounds once to bf16.
#include <mutex>

#include "ffn_common.hpp"

namespace moe {

void log_info(const char* fmt, ...);  // runtime.hip: printed to stderr at MOE_W4A16_LOG >= 2

__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y, int ksplit, int64_t P, int d, int k,
                                                 const int32_t* __restrict__ pair_pos,
                                                 const float* __restrict__ w, uint16_t* __restrict__ out,
                                                 int nchunks) {
  const int64_t t = blockIdx.x / nchunks;
  const int n = ((blockIdx.x % nchunks) * 256 + threadIdx.x) * 4;
  if (n >= d) return;
  // every position and weight first, then every row slice: two dependent round
  // trips per thread instead of two per routed slot
  int64_t pos[MOE_MAX_TOPK];
  float wj[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    pos[j] = j < k ? pair_pos[t * k + j] : -1;  // -1: pair dropped by moe_align (expert id out of range)
    wj[j] = j < k ? w[t * k + j] : 0.f;
  }
  f32x4_t v[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j)
    v[j] = pos[j] >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(y + pos[j] * d + n))
                       : f32x4_t{0.f, 0.f, 0.f, 0.f};  // (y is read once: streaming loads)
  for (int s = 1; s < ksplit; ++s) {
    f32x4_t p[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      p[j] = pos[j] >= 0 ? *reinterpret_cast<const f32x4_t*>(y + ((int64_t)s * P + pos[j]) * d + n)
                         : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      v[j][0] += p[j][0];
      v[j][1] += p[j][1];
      v[j][2] += p[j][2];
      v[j][3] += p[j][3];
    }
  }
  // the k routed outputs in slot order, fp32, one bf16 rounding
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (pos[j] < 0) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = fmaf(wj[j], v[j][r], acc[r]);
  }
  const u32x2_t o = pack_bf16x4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<u32x2_t*>(out + t * d + n) = o;
}

// The combine of the prefill path: per-pair rows in bf16, one K part.  Same
// order and arithmetic as k_combine: the k routed outputs in slot order, fp32,
// one bf16 rounding.
__global__ __launch_bounds__(256) void k_combine_bf16(const uint16_t* __restrict__ y, int d, int k,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ w, uint16_t* __restrict__ out,
                                                      int nchunks) {
  const int64_t t = blockIdx.x / nchunks;
  const int n = ((blockIdx.x % nchunks) * 256 + threadIdx.x) * 4;
  if (n >= d) return;
  int64_t pos[MOE_MAX_TOPK];
  float wj[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    pos[j] = j < k ? pair_pos[t * k + j] : -1;  // -1: pair dropped by moe_align (expert id out of range)
    wj[j] = j < k ? w[t * k + j] : 0.f;
  }
  u32x2_t v[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j)
    v[j] = pos[j] >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(y + pos[j] * d + n))
                       : u32x2_t{0u, 0u};
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (pos[j] < 0) continue;
    const float r4[4] = {__uint_as_float(v[j][0] << 16), __uint_as_float(v[j][0] & 0xFFFF0000u),
                         __uint_as_float(v[j][1] << 16), __uint_as_float(v[j][1] & 0xFFFF0000u)};
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = fmaf(wj[j], r4[r], acc[r]);
  }
  const u32x2_t o = pack_bf16x4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<u32x2_t*>(out + t * d + n) = o;
}

// Automatic choice: the decode kernels up to 20 expected pairs per expert, the
// MFMA-tiled prefill kernels above (measured crossover: at 16 pairs per expert
// decode is 12 % (OLMoE) to 33 % (d = 4096, I = 14336) faster, at 24 prefill 6 %,
// at 32 to 48 prefill 5 % to 80 %).
static int resolve_mode(int T, int E, int k, int mode) {
  if (mode == MOE_MODE_DECODE || mode == MOE_MODE_PREFILL) return mode;
  const double per_expert = (double)T * k / E;  // expected pairs per expert
  return per_expert <= 20.0 ? MOE_MODE_DECODE : MOE_MODE_PREFILL;
}

// token blocks of 16 per pass of the decode kernels (grouped FFN, more than 16 tokens)
static int decode_token_blocks(int T, int E, int k) { return (double)T * k / E <= 8.0 ? 1 : 2; }

static int down_ksplit(int T, int d, int I, int E, int k, int mode) {
  if (mode == MOE_MODE_PREFILL) return 1;
  const int64_t umax = std::min<int64_t>(E, (int64_t)T * k);
  if (decode_token_blocks(T, E, k) <= 1) {  // down blocks own 64 output rows, a quarter split each wavefront
    const int64_t blocks = umax * (d / 64);
    const int max_split = std::max(1, (I / kGroup) / 4);
    int ks = 1;
    while (ks * 2 <= max_split && blocks * ks < 2048) ks *= 2;
    return ks;
  }
  const int64_t blocks = umax * ceil_div(d, 256);  // down blocks own 4 x 64 output rows
  const int max_split = std::max(1, (I / kGroup) / 8);  // more than 8 groups per split
  int ks = 1;
  while (ks * 2 <= max_split && blocks * ks < 1024) ks *= 2;
  return ks;
}

static int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

struct WsLayout {
  int64_t h_off, y_off, xsum_off, hsum_off, dc_part_off, dc_ctr_off, total;
};

// fused down + combine (steps of at most 16 tokens): up to 32 chunks x 512
// partial values per 32-row output stripe, and one counter per stripe
static int64_t dc_part_bytes(int d) { return (int64_t)(d / 32) * 32 * 512 * 4; }

static WsLayout ws_layout(int T, int d, int I, int E, int k, int mode) {
  const int64_t P = (int64_t)T * k;
  const int ks = down_ksplit(T, d, I, E, k, mode);
  WsLayout L;
  L.h_off = 0;
  L.y_off = align256(P * I * 2);
  // per-pair outputs: fp32 K parts (decode), bf16 rows (prefill)
  L.xsum_off = L.y_off + align256(mode == MOE_MODE_PREFILL ? P * d * 2 : (int64_t)ks * P * d * 4);
  L.hsum_off = L.xsum_off;
  L.total = L.xsum_off;
  L.dc_part_off = L.dc_ctr_off = -1;
  if (mode == MOE_MODE_DECODE && T <= 16) {
    L.dc_part_off = L.total;
    L.dc_ctr_off = L.dc_part_off + align256(dc_part_bytes(d));
    L.total = L.dc_ctr_off + align256((int64_t)(d / 32) * 4);
  }
  if (mode == MOE_MODE_PREFILL) {
    L.hsum_off = L.xsum_off + align256((int64_t)T * (d / kGroup) * 4);
    L.total = L.hsum_off + align256(P * (I / kGroup) * 4);
  }
  return L;
}

FfnWorkspace ffn_workspace(int T, int d, int I, int E, int k, int mode, void* ws) {
  const WsLayout L = ws_layout(T, d, I, E, k, mode);
  uint8_t* b = static_cast<uint8_t*>(ws);
  FfnWorkspace w;
  w.h = reinterpret_cast<uint16_t*>(b + L.h_off);
  w.y = reinterpret_cast<float*>(b + L.y_off);
  w.xsum = reinterpret_cast<float*>(b + L.xsum_off);
  w.hsum = reinterpret_cast<float*>(b + L.hsum_off);
  w.dc_part = L.dc_part_off >= 0 ? reinterpret_cast<float*>(b + L.dc_part_off) : nullptr;
  w.dc_counters = L.dc_ctr_off >= 0 ? reinterpret_cast<int32_t*>(b + L.dc_ctr_off) : nullptr;
  w.ksplit = down_ksplit(T, d, I, E, k, mode);
  return w;
}

int launch_combine_bf16(const FfnDev& f, const uint16_t* y, const float* weights, uint16_t* out, hipStream_t s) {
  const int nchunks = (int)ceil_div(f.d, 1024);
  timing_begin(K_COMBINE, s);
  hipLaunchKernelGGL(k_combine_bf16, dim3((unsigned)(f.T * (int64_t)nchunks)), dim3(256), 0, s, y, f.d, f.k,
                     f.pair_pos, weights, out, nchunks);
  timing_end(K_COMBINE, s);
  return check_launch("combine");
}

int launch_combine(const FfnDev& f, const float* y, int ksplit, const float* weights, uint16_t* out, hipStream_t s) {
  const int nchunks = (int)ceil_div(f.d, 1024);
  timing_begin(K_COMBINE, s);
  hipLaunchKernelGGL(k_combine, dim3((unsigned)(f.T * (int64_t)nchunks)), dim3(256), 0, s, y, ksplit, f.P, f.d, f.k,
                     f.pair_pos, weights, out, nchunks);
  timing_end(K_COMBINE, s);
  return check_launch("combine");
}

}  // namespace moe

using namespace moe;

extern "C" int64_t moe_ffn_workspace_bytes(int T, int d, int I, int E, int k, int mode) {
  if (T < 0 || d <= 0 || I <= 0 || E <= 0 || k <= 0) return -1;
  return ws_layout(T, d, I, E, k, resolve_mode(T, E, k, mode)).total;
}

extern "C" int moe_w4a16_grouped_ffn(const moe_ffn_args* a, void* stream) {
  clear_error();
  MOE_CHECK_ARG(a != nullptr, MOE_ERR_INVALID_ARG, "moe_w4a16_grouped_ffn: args is NULL");
  MOE_CHECK_ARG(a->T >= 0 && a->d > 0 && a->I > 0 && a->E > 0 && a->k > 0, MOE_ERR_INVALID_ARG,
                "moe_w4a16_grouped_ffn: bad sizes T=%d d=%d I=%d E=%d k=%d", a->T, a->d, a->I, a->E, a->k);
  MOE_CHECK_ARG(a->mode >= 0 && a->mode <= 2, MOE_ERR_INVALID_ARG, "moe_w4a16_grouped_ffn: bad mode %d", a->mode);
  MOE_CHECK_ARG(a->d % kGroup == 0 && a->I % kGroup == 0 && a->E <= MOE_MAX_EXPERTS && a->k <= MOE_MAX_TOPK &&
                    a->k <= a->E && (int64_t)a->T * a->k <= (1 << 24),
                MOE_ERR_UNSUPPORTED_SHAPE,
                "moe_w4a16_grouped_ffn: unsupported shape d=%d I=%d E=%d k=%d T=%d (d, I multiples of 128, "
                "E <= 1024, k <= min(E,16))",
                a->d, a->I, a->E, a->k, a->T);
  if (a->T == 0) return MOE_OK;
  MOE_CHECK_ARG(a->x && a->topk_ids && a->topk_weights && a->expert_offsets && a->sorted_pairs && a->pair_pos &&
                    a->active_experts && a->bank && a->workspace,
                MOE_ERR_INVALID_ARG, "moe_w4a16_grouped_ffn: null pointer");
  MOE_CHECK_ARG(!a->combine || a->out, MOE_ERR_INVALID_ARG, "moe_w4a16_grouped_ffn: combine needs out");
  moe_expert_layout lay;
  int rc = moe_expert_layout_get(a->d, a->I, &lay);
  if (rc) return rc;
  MOE_CHECK_ARG(a->bank_stride >= lay.blob_bytes && a->bank_stride % 256 == 0 && ((uintptr_t)a->bank % 256) == 0,
                MOE_ERR_INVALID_ARG,
                "moe_w4a16_grouped_ffn: bank must be 256-byte aligned with stride >= %lld (multiple of 256), got %lld",
                (long long)lay.blob_bytes, (long long)a->bank_stride);
  MOE_CHECK_ARG(((uintptr_t)a->x % 16) == 0 && ((uintptr_t)a->workspace % 256) == 0 &&
                    ((uintptr_t)a->active_experts % 16) == 0 &&
                    (!a->out || ((uintptr_t)a->out % 8) == 0),
                MOE_ERR_INVALID_ARG, "moe_w4a16_grouped_ffn: misaligned x, out or workspace");
  const int mode = resolve_mode(a->T, a->E, a->k, a->mode);
  const WsLayout L = ws_layout(a->T, a->d, a->I, a->E, a->k, mode);
  MOE_CHECK_ARG(a->workspace_bytes >= L.total, MOE_ERR_WORKSPACE,
                "moe_w4a16_grouped_ffn: workspace %lld bytes < %lld needed", (long long)a->workspace_bytes,
                (long long)L.total);

  FfnDev f;
  f.x = a->x;
  f.T = a->T;
  f.d = a->d;
  f.I = a->I;
  f.E = a->E;
  f.k = a->k;
  f.P = (int64_t)a->T * a->k;
  f.umax = (int)std::min<int64_t>(a->E, f.P);
  f.topk_ids = a->topk_ids;
  f.topk_weights = a->topk_weights;
  f.offsets = a->expert_offsets;
  f.sorted_pairs = a->sorted_pairs;
  f.pair_pos = a->pair_pos;
  f.active = a->active_experts;
  f.tile_offsets = a->tile_offsets;
  f.bank = a->bank;
  f.bank_stride = a->bank_stride;
  f.slot_of_expert = a->slot_of_expert;
  f.off_w13_codes = lay.w13_codes;
  f.off_w13_scales = lay.w13_scales;
  f.off_w2_codes = lay.w2_codes;
  f.off_w2_scales = lay.w2_scales;

  const FfnWorkspace w = ffn_workspace(a->T, a->d, a->I, a->E, a->k, mode, a->workspace);
  hipStream_t s = (hipStream_t)stream;
  // every expert in the call and the combine requested: at most 16 tokens finish
  // the combine inside the down pass
  const bool fused = mode == MOE_MODE_DECODE && a->T <= 16 && a->combine && !a->slot_of_expert && w.dc_part &&
                     a->bank_stride < ((int64_t)1 << 31) && dc_units_per_wave(f.umax, a->I / kGroup, a->d / 32) > 0;
  log_info("moe_w4a16_grouped_ffn: T=%d d=%d I=%d E=%d k=%d: %s kernels%s, down K split %d, token blocks %d", a->T,
           a->d, a->I, a->E, a->k, mode == MOE_MODE_DECODE ? "decode" : "prefill (MFMA-tiled)",
           fused ? " with the combine in the down pass" : "", mode == MOE_MODE_DECODE ? w.ksplit : 1,
           mode == MOE_MODE_DECODE ? decode_token_blocks(a->T, a->E, a->k) : 0);
  if (mode == MOE_MODE_DECODE) {
    rc = launch_decode(f, w.h, w.y, w.ksplit, decode_token_blocks(a->T, a->E, a->k), s, fused ? a->out : nullptr, w.dc_part,
                       w.dc_counters);
  } else {
    rc = launch_prefill(f, w.h, reinterpret_cast<uint16_t*>(w.y), w.xsum, w.hsum, s);
  }
  if (rc) return rc;
  if (a->combine && !fused) {
    if (mode == MOE_MODE_PREFILL)
      rc = launch_combine_bf16(f, reinterpret_cast<const uint16_t*>(w.y), a->topk_weights, a->out, s);
    else
      rc = launch_combine(f, w.y, w.ksplit, a->topk_weights, a->out, s);
  }
  return rc;
}

// ---------------------------------------------------------------- no-allocation variant
//
// moe_w4a16_grouped_ffn_noalloc: the same pass with its workspace taken from a
// file-scope device array instead of a caller buffer, for callers that cannot
// allocate.  Each GPU the library runs on holds its own copy of the array until the
// process ends; host code addresses it only through the device pointer that
// hipGetSymbolAddress returns for that device (the array's name is a host-side
// stand-in).  Nothing in the workspace has to be zero when a call starts: the
// gate/up kernels clear the down pass's stripe counters on every call.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices] = {};

// device address of this device's scratch copy, looked up once per device
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
    set_error("moe_w4a16_grouped_ffn_noalloc: no usable current device (%s, device %d)", hipGetErrorString(e), dev);
    return MOE_ERR_HIP;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      set_error("moe_w4a16_grouped_ffn_noalloc: hipGetSymbolAddress of the scratch array failed on device %d: %s",
                dev, hipGetErrorString(e));
      return MOE_ERR_HIP;
    }
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}
}  // namespace

extern "C" int moe_w4a16_grouped_ffn_noalloc(const moe_ffn_args* a, void* stream) {
  clear_error();
  MOE_CHECK_ARG(a != nullptr, MOE_ERR_INVALID_ARG, "moe_w4a16_grouped_ffn_noalloc: args is NULL");
  MOE_CHECK_ARG(a->workspace == nullptr && a->workspace_bytes == 0, MOE_ERR_INVALID_ARG,
                "moe_w4a16_grouped_ffn_noalloc: workspace must be NULL with 0 bytes (the call uses its own scratch)");
  MOE_CHECK_ARG(a->T >= 0 && a->d > 0 && a->I > 0 && a->E > 0 && a->k > 0 && a->mode >= 0 && a->mode <= 2,
                MOE_ERR_INVALID_ARG, "moe_w4a16_grouped_ffn_noalloc: bad sizes T=%d d=%d I=%d E=%d k=%d mode=%d",
                a->T, a->d, a->I, a->E, a->k, a->mode);
  const int64_t need = moe_ffn_workspace_bytes(a->T, a->d, a->I, a->E, a->k, a->mode);
  MOE_CHECK_ARG(need >= 0 && need <= (int64_t)MOE_NOALLOC_SCRATCH_BYTES, MOE_ERR_WORKSPACE,
                "moe_w4a16_grouped_ffn_noalloc: this step needs %lld bytes of workspace, above the %lld-byte scratch "
                "(use moe_w4a16_grouped_ffn with a caller buffer)",
                (long long)need, (long long)MOE_NOALLOC_SCRATCH_BYTES);
  if (a->T == 0) return moe_w4a16_grouped_ffn(a, stream);
  void* ws = nullptr;
  const int rc = scratch_for_current_device(&ws);
  if (rc) return rc;
  moe_ffn_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = (int64_t)MOE_NOALLOC_SCRATCH_BYTES;
  return moe_w4a16_grouped_ffn(&b, stream);
}
