// moe_route: BF16 router logits and unchanged top-k selection (ExactMoE, page
// "Every Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference",
// Abstract: the router stays BF16 and the top-k routing procedure is unchanged).
//
// One kernel per call.  Logits: products of bf16 values are exact; they are
// summed in float64 and rounded once to float32 (on MI355X a non-packed fp64 FMA
// issues at the fp32 rate, so the near-exact sum costs nothing extra).  The
// selection orders by (logit desc, index asc); softmax weights in float32.
// Three launch shapes: one 1024-thread block per token for small T (latency),
// blocks of TB tokens x all experts for large T (router weights reused across
// the TB tokens; TB = 2 up to 512 tokens, 4 beyond), and for E <= 128 once there
// are as many 16-token blocks as CUs, the float64 matrix-core kernel.
#include "align_block.hpp"
#include "route_rank.hpp"

namespace moe {

constexpr int kRouteMaxTB = 4;

__device__ __forceinline__ double bf16_to_f64(uint32_t bits16) { return (double)bf16_bits_to_f32(bits16); }

// Top-k of one token's E logits (in LDS) by one wavefront: lane l owns experts
// l, l+64, ...; for E up to 128 every logit's rank in the (value desc, index asc)
// order is counted against the row and the k best land at their rank (s_sv, s_si:
// the wavefront's k slots in LDS); beyond that, k rounds of a wave-wide argmax.
__device__ __forceinline__ void topk_wave(const float* __restrict__ lg, int E, int k, int renormalize, int t,
                          int32_t* __restrict__ ids, float* __restrict__ weights, float* s_sv, int* s_si) {
  const int lane = lane_id();
  const int nper = (E + 63) / 64;  // <= 16
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    v[i] = (i < nper && e < E) ? lg[e] : -INFINITY;
  }
  float sel_v[MOE_MAX_TOPK];
  int sel_i[MOE_MAX_TOPK];
  if (E <= 128) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        const int rank = rank_in_row(lg, E, v[i], e);
        if (rank < k) {
          s_sv[rank] = v[i];
          s_si[rank] = e;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k) {
        sel_v[j] = s_sv[j];
        sel_i[j] = s_si[j];
      }
    }
  } else {
    uint32_t taken = 0;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j >= k) break;
      // sentinel below every finite logit: a real candidate always wins the reduction
      float bv = -INFINITY;
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
      bi = min(bi, E - 1);  // unreachable for finite logits; keeps ids in range regardless
      sel_v[j] = bv;
      sel_i[j] = bi;
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    }
  }
  const float lmax = sel_v[0];
  float den = 0.f;
  if (renormalize) {
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
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
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (j < k && lane == j) {
      ids[(int64_t)t * k + j] = sel_i[j];
      weights[(int64_t)t * k + j] = expf(sel_v[j] - lmax) / den;
    }
  }
}

// Few tokens: one 1024-thread block per token.  Thread (expert slot el = tid/16,
// d-lane r = tid%16) accumulates expert eb+el over the 16-byte chunks r, r+16, ...
// of d, so a wavefront reads four 256-byte runs of four router rows per load and
// the sixteen partial sums of an expert meet in one 16-lane row (four shuffle
// steps).  Each thread issues eight chunks of loads before its FMAs.  The top-k
// is a rank computation: every thread ranks one expert against all E logits in
// LDS (broadcast reads) and the k winners write themselves.
constexpr int kRouteBatch = 8;

__global__ __launch_bounds__(1024) void k_route_token(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ wr, int T, int d, int E, int k,
                                                      int renormalize, float* __restrict__ logits,
                                                      int32_t* __restrict__ ids, float* __restrict__ weights) {
  __shared__ float s_logit[MOE_MAX_EXPERTS];
  __shared__ float s_sel_v[MOE_MAX_TOPK];
  __shared__ int s_sel_i[MOE_MAX_TOPK];
  __shared__ float s_den;
  const int tid = threadIdx.x, r = tid & 15, el = tid >> 4;
  const int t = blockIdx.x;
  const int nch = d / 8;
  const uint16_t* xr = x + (int64_t)t * d;
  for (int eb = 0; eb < E; eb += 64) {
    const int e = eb + el;
    double acc = 0.0;
    for (int c0 = 0; c0 < nch; c0 += 16 * kRouteBatch) {
      u32x4_t xq[kRouteBatch], wq[kRouteBatch];
#pragma unroll
      for (int c = 0; c < kRouteBatch; ++c) {
        const int ch = c0 + r + 16 * c;
        xq[c] = ch < nch ? *reinterpret_cast<const u32x4_t*>(xr + 8 * ch) : u32x4_t{0u, 0u, 0u, 0u};
        wq[c] = (ch < nch && e < E) ? *reinterpret_cast<const u32x4_t*>(wr + (int64_t)e * d + 8 * ch)
                                    : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int c = 0; c < kRouteBatch; ++c)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc = fma(bf16_to_f64(xq[c][m] & 0xFFFFu), bf16_to_f64(wq[c][m] & 0xFFFFu), acc);
          acc = fma(bf16_to_f64(xq[c][m] >> 16), bf16_to_f64(wq[c][m] >> 16), acc);
        }
    }
    acc += __shfl_xor(acc, 8);
    acc += __shfl_xor(acc, 4);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 1);
    if (r == 0 && e < E) s_logit[e] = (float)acc;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    const float v = s_logit[e];
    logits[(int64_t)t * E + e] = v;
    const int rank = rank_in_row(s_logit, E, v, e);
    if (rank < k) {
      s_sel_v[rank] = v;
      s_sel_i[rank] = e;
    }
  }
  __syncthreads();
  const float lmax = s_sel_v[0];
  // the same sums, in the same order, as topk_wave
  if (tid < 64) {
    float part = 0.f;
    if (renormalize) {
      if (tid == 0)
        for (int j = 0; j < k; ++j) part += expf(s_sel_v[j] - lmax);
    } else {
      for (int e = tid; e < E; e += 64) part += expf(s_logit[e] - lmax);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    }
    if (tid == 0) s_den = part;
  }
  __syncthreads();
  if (tid < k) {
    ids[(int64_t)t * k + tid] = s_sel_i[tid];
    weights[(int64_t)t * k + tid] = expf(s_sel_v[tid] - lmax) / s_den;
  }
}

// Decode-sized steps, routing and alignment in one launch.  Every workgroup
// computes 16 logits of one token, one per wavefront (lane l takes the 16-byte
// chunks l, l + 64, ... of d; the float64 partial sums meet in a butterfly),
// releases them with device-coherent stores and counts itself done on its
// token's counter once they have completed.  The workgroup that completes a
// token reads that token's logits with device-coherent loads and runs its top-k
// and weights (tokens in parallel, on as many CUs), releases the ids the same
// way and counts the token done; the workgroup that completes the last token
// reads every id and runs the alignment (align_block).  Each counter is put back
// to zero by the workgroup that saw it complete.
constexpr int kRouteAlignMaxT = 128;

__global__ __launch_bounds__(kAlignThreads) void k_route_align(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int d, int E, int k, int renormalize,
    int block_m, int id_bits, float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ weights,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ active, int32_t* __restrict__ tile_offsets, int32_t* __restrict__ counters) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int e = blockIdx.x * kAlignWaves + wave, t = blockIdx.y;
  if (e < E) {
    const int nch = d / 8;
    const uint16_t* xr = x + (int64_t)t * d;
    const uint16_t* wrow = wr + (int64_t)e * d;
    double acc = 0.0;
    constexpr int kB = 4;
    for (int c0 = 0; c0 < nch; c0 += 64 * kB) {
      u32x4_t xq[kB], wq[kB];
#pragma unroll
      for (int c = 0; c < kB; ++c) {
        const int ch = c0 + lane + 64 * c;
        xq[c] = ch < nch ? *reinterpret_cast<const u32x4_t*>(xr + 8 * ch) : u32x4_t{0u, 0u, 0u, 0u};
        wq[c] = ch < nch ? *reinterpret_cast<const u32x4_t*>(wrow + 8 * ch) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int c = 0; c < kB; ++c)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc = fma(bf16_to_f64(xq[c][m] & 0xFFFFu), bf16_to_f64(wq[c][m] & 0xFFFFu), acc);
          acc = fma(bf16_to_f64(xq[c][m] >> 16), bf16_to_f64(wq[c][m] >> 16), acc);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    // device-coherent store (no L2 write-back of everything else needed)
    if (lane == 0) __hip_atomic_store(logits + (int64_t)t * E + e, (float)acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __shared__ int s_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wavefront's logit has reached device scope
  __syncthreads();
  if (tid == 0) {
    s_last = __hip_atomic_fetch_add(counters + 1 + t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (int)gridDim.x - 1;
    if (s_last) __hip_atomic_store(counters + 1 + t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;

  // this token's logits are complete at device scope: top-k by rank (each expert
  // counts the logits that beat it, value desc, index asc) and weights, with the
  // sums of topk_wave in the same order
  __shared__ float s_lg[MOE_MAX_EXPERTS];
  __shared__ float s_sel_v[MOE_MAX_TOPK];
  __shared__ int s_sel_i[MOE_MAX_TOPK];
  __shared__ int32_t s_ids[kRouteAlignMaxT * MOE_MAX_TOPK];
  for (int i = tid; i < E; i += kAlignThreads)
    s_lg[i] = __hip_atomic_load(logits + (int64_t)t * E + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  for (int i = tid; i < E; i += kAlignThreads) {
    const float v = s_lg[i];
    const int rank = rank_in_row(s_lg, E, v, i);
    if (rank < k) {
      s_sel_v[rank] = v;
      s_sel_i[rank] = i;
    }
  }
  __syncthreads();
  if (wave == 0) {
    // lane j < k holds the exponential of selection j; the renormalising sum runs
    // over j in order
    const float lmax = s_sel_v[0];
    const float ex = lane < k ? expf(s_sel_v[lane] - lmax) : 0.f;
    float den = 0.f;
    if (renormalize) {
      for (int j = 0; j < k; ++j) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
    } else {
      float part = 0.f;
      for (int i = lane; i < E; i += 64) part += expf(s_lg[i] - lmax);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
      den = part;
    }
    if (lane < k) {
      const int id = s_sel_i[lane];
      s_ids[lane] = id;  // used when this is the only token
      __hip_atomic_store(ids + (int64_t)t * k + lane, id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      weights[(int64_t)t * k + lane] = ex / den;
    }
  }
  if (T > 1) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this token's ids have reached device scope
    __syncthreads();
    if (tid == 0) {
      s_last = __hip_atomic_fetch_add(counters, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == T - 1;
      if (s_last) __hip_atomic_store(counters, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    // every token's ids are complete at device scope
    for (int i = tid; i < T * k; i += kAlignThreads)
      s_ids[i] = __hip_atomic_load(ids + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  align_block(s_ids, T * k, E, block_m, id_bits, offsets, sorted_pairs, pair_pos, active, tile_offsets);
}

template <int TB>
__global__ __launch_bounds__(256) void k_route(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                               int T, int d, int E, int k, int renormalize,
                                               float* __restrict__ logits, int32_t* __restrict__ ids,
                                               float* __restrict__ weights) {
  __shared__ float s_logit[TB][MOE_MAX_EXPERTS];
  __shared__ float s_sv[TB][MOE_MAX_TOPK];
  __shared__ int s_si[TB][MOE_MAX_TOPK];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TB;
  const int nch = d / 8;

  for (int eb = wave * 8; eb < E; eb += 32) {
    double acc[TB][8];
#pragma unroll
    for (int a = 0; a < TB; ++a)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[a][j] = 0.0;
    for (int ch = lane; ch < nch; ch += 64) {
      double xv[TB][8];
#pragma unroll
      for (int a = 0; a < TB; ++a) {
        u32x4_t q = {0u, 0u, 0u, 0u};
        if (t0 + a < T) q = *reinterpret_cast<const u32x4_t*>(x + (int64_t)(t0 + a) * d + 8 * ch);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          xv[a][2 * m] = bf16_to_f64(q[m] & 0xFFFFu);
          xv[a][2 * m + 1] = bf16_to_f64(q[m] >> 16);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = eb + j;
        u32x4_t q = {0u, 0u, 0u, 0u};
        if (e < E) q = *reinterpret_cast<const u32x4_t*>(wr + (int64_t)e * d + 8 * ch);
        double wv[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          wv[2 * m] = bf16_to_f64(q[m] & 0xFFFFu);
          wv[2 * m + 1] = bf16_to_f64(q[m] >> 16);
        }
#pragma unroll
        for (int a = 0; a < TB; ++a)
#pragma unroll
          for (int m = 0; m < 8; ++m) acc[a][j] = fma(xv[a][m], wv[m], acc[a][j]);
      }
    }
    // halving butterfly: after the xor-32/16/8 steps lane l holds the partial sum of
    // expert j = 4*b5 + 2*b4 + b3 (b = lane bits) over 8 lanes; xor-4/2/1 finish it.
#pragma unroll
    for (int a = 0; a < TB; ++a) {
      const bool h5 = lane & 32, h4 = lane & 16, h3 = lane & 8;
      double v4[4], v2[2], v1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double send = h5 ? acc[a][j] : acc[a][j + 4];
        const double keep = h5 ? acc[a][j + 4] : acc[a][j];
        v4[j] = keep + __shfl_xor(send, 32);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const double send = h4 ? v4[j] : v4[j + 2];
        const double keep = h4 ? v4[j + 2] : v4[j];
        v2[j] = keep + __shfl_xor(send, 16);
      }
      {
        const double send = h3 ? v2[0] : v2[1];
        const double keep = h3 ? v2[1] : v2[0];
        v1 = keep + __shfl_xor(send, 8);
      }
      v1 += __shfl_xor(v1, 4);
      v1 += __shfl_xor(v1, 2);
      v1 += __shfl_xor(v1, 1);
      const int j = (h5 ? 4 : 0) + (h4 ? 2 : 0) + (h3 ? 1 : 0);
      if ((lane & 7) == 0 && eb + j < E) s_logit[a][eb + j] = (float)v1;
    }
  }
  __syncthreads();

  for (int i = threadIdx.x; i < TB * E; i += 256) {
    const int a = i / E, e = i % E;
    if (t0 + a < T) logits[(int64_t)(t0 + a) * E + e] = s_logit[a][e];
  }

  if (wave >= TB || t0 + wave >= T) return;
  topk_wave(s_logit[wave], E, k, renormalize, t0 + wave, ids, weights, s_sv[wave], s_si[wave]);
}

// Many tokens, E <= 128: the logits of 16 tokens x 16 experts per wavefront on the
// float64 matrix cores (v_mfma_f64_16x16x4f64: the bf16 values converted exactly,
// products and sums in float64, rounded once to float32, as in k_route).  Lane l
// (r = l % 16, q = l / 16) loads 8 consecutive channels of router row eb + r and of
// token row t0 + r and feeds them to 8 MFMAs as K index q, so each MFMA sums four
// channels 8 apart; element i of its result is expert eb + q + 4i, token t0 + r.
// A block is 16 tokens x (4 expert blocks of 16) x KS parts of d; the parts meet
// in LDS in part order.  Then one wavefront per token runs the top-k.  The float64
// sums come out the same as k_route's on the evaluated shapes (0 ulp at T = 300 to
// 4096); both are within an ulp of the oracle's.
constexpr int kRouteMfmaTB = 16, kRouteMfmaMaxE = 128, kRouteMfmaKS = 4;
typedef double f64x4_t __attribute__((ext_vector_type(4)));

template <int KS>
__global__ __launch_bounds__(256 * KS) void k_route_mfma(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                         int T, int d, int E, int k, int renormalize,
                                                         float* __restrict__ logits, int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
  constexpr int kWaves = 4 * KS;
  __shared__ float s_logit[kRouteMfmaTB][kRouteMfmaMaxE];
  __shared__ f64x4_t s_part[KS > 1 ? kWaves : 1][64];
  __shared__ float s_sv[kWaves][MOE_MAX_TOPK];
  __shared__ int s_si[kWaves][MOE_MAX_TOPK];
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int xb = wave / KS, part = wave % KS;  // expert block (of 4) and part of d
  const int t0 = blockIdx.x * kRouteMfmaTB;
  const int nch = (d + 31) / 32;                // 32-channel chunks
  const int cpp = (nch + KS - 1) / KS;          // chunks per part
  const int c_lo = min(nch, part * cpp), c_hi = min(nch, c_lo + cpp);
  const bool t_ok = t0 + r < T;
  const uint16_t* xrow = x + (int64_t)(t_ok ? t0 + r : 0) * d;

  // every wavefront takes the same number of expert-block rounds (the rounds
  // hold barriers); a round past E leaves its wavefront's sums at zero
  const int rounds = (E + 63) / 64;
  for (int m = 0; m < rounds; ++m) {
    const int eb = 16 * xb + 64 * m;
    const bool e_ok = eb + r < E;
    const uint16_t* wrow = wr + (int64_t)(e_ok ? eb + r : 0) * d;
    f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
    constexpr int kRing = 4;
    u32x4_t bw[kRing], bx[kRing];
    // chunk c's 16-byte slices (zeros past d, past E or past T)
    auto load = [&](int j, int c) {
      const int ch = 32 * c + 8 * q;
      const bool in = c < c_hi && ch < d;
      bw[j] = in && e_ok ? *reinterpret_cast<const u32x4_t*>(wrow + ch) : u32x4_t{0u, 0u, 0u, 0u};
      bx[j] = in && t_ok ? *reinterpret_cast<const u32x4_t*>(xrow + ch) : u32x4_t{0u, 0u, 0u, 0u};
    };
    const int c_end = eb < E ? c_hi : c_lo;  // wave-uniform
#pragma unroll
    for (int j = 0; j < kRing - 1; ++j) load(j, c_lo + j);
    for (int c = c_lo; c < c_end; c += kRing) {
#pragma unroll
      for (int j = 0; j < kRing; ++j) {
        load((j + kRing - 1) % kRing, c + j + kRing - 1);
        const u32x4_t w4 = bw[j], x4 = bx[j];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t wb = (m & 1) ? (w4[m >> 1] >> 16) : (w4[m >> 1] & 0xFFFFu);
          const uint32_t xv = (m & 1) ? (x4[m >> 1] >> 16) : (x4[m >> 1] & 0xFFFFu);
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(bf16_to_f64(wb), bf16_to_f64(xv), acc, 0, 0, 0);
        }
      }
    }
    if constexpr (KS > 1) {
      s_part[wave][lane] = acc;
      __syncthreads();
      if (part == 0) {
#pragma unroll
        for (int p = 1; p < KS; ++p) {
          const f64x4_t o = s_part[wave + p][lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] += o[i];
        }
      }
      __syncthreads();  // s_part is free for the next expert block
    }
    if (part == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = eb + q + 4 * i;
        if (e < E) s_logit[r][e] = (float)acc[i];
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kRouteMfmaTB * E; i += 64 * kWaves) {
    const int a = i / E, e = i % E;
    if (t0 + a < T) logits[(int64_t)(t0 + a) * E + e] = s_logit[a][e];
  }
  for (int a = wave; a < kRouteMfmaTB; a += kWaves)
    if (t0 + a < T) topk_wave(s_logit[a], E, k, renormalize, t0 + a, ids, weights, s_sv[wave], s_si[wave]);
}

}  // namespace moe

using namespace moe;

static int route_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    cus = std::max(cus, 1);
  }
  return cus;
}

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
  if (T <= 256) {
    hipLaunchKernelGGL(k_route_token, dim3(T), dim3(1024), 0, s, x, w_router, T, d, E, k, renormalize, logits,
                       topk_ids, topk_weights);
  } else if (E <= kRouteMfmaMaxE && ceil_div(T, kRouteMfmaTB) >= route_cus()) {
    // float64 matrix cores once every CU has a 16-token block (a block's time is
    // fixed by its products on one CU, so fewer blocks leave CUs idle)
    hipLaunchKernelGGL(k_route_mfma<kRouteMfmaKS>, dim3((unsigned)ceil_div(T, kRouteMfmaTB)), dim3(256 * kRouteMfmaKS),
                       0, s, x, w_router, T, d, E, k, renormalize, logits, topk_ids, topk_weights);
  } else if (T <= 512) {
    // two tokens per block: twice the blocks of the four-token shape, which leaves
    // half the CUs idle below 1024 tokens (measured faster up to 512 tokens)
    hipLaunchKernelGGL(k_route<2>, dim3((unsigned)ceil_div(T, 2)), dim3(256), 0, s, x, w_router, T, d, E, k,
                       renormalize, logits, topk_ids, topk_weights);
  } else {
    hipLaunchKernelGGL(k_route<kRouteMaxTB>, dim3((unsigned)ceil_div(T, kRouteMaxTB)), dim3(256), 0, s, x, w_router,
                       T, d, E, k, renormalize, logits, topk_ids, topk_weights);
  }
  timing_end(K_ROUTE, s);
  return check_launch("moe_route");
}

extern "C" int moe_route_align(const uint16_t* x, const uint16_t* w_router, int T, int d, int E, int k,
                               int renormalize, int block_m, float* logits, int32_t* topk_ids, float* topk_weights,
                               int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                               int32_t* active_experts, int32_t* tile_offsets, int32_t* counters, void* stream) {
  clear_error();
  MOE_CHECK_ARG(T >= 0 && d > 0 && E > 0 && k > 0 && block_m >= 0, MOE_ERR_INVALID_ARG,
                "moe_route_align: bad sizes T=%d d=%d E=%d k=%d block_m=%d", T, d, E, k, block_m);
  if (T == 0 || T > kRouteAlignMaxT) {
    // nothing to route, or a step too large for one launch: the two separate calls
    int rc = moe_route(x, w_router, T, d, E, k, renormalize, logits, topk_ids, topk_weights, stream);
    if (rc) return rc;
    return moe_align(topk_ids, T, k, E, block_m, expert_offsets, sorted_pairs, pair_pos, active_experts,
                     tile_offsets, stream);
  }
  MOE_CHECK_ARG(E <= MOE_MAX_EXPERTS && k <= MOE_MAX_TOPK && k <= E && d % 8 == 0, MOE_ERR_UNSUPPORTED_SHAPE,
                "moe_route_align: unsupported E=%d k=%d d=%d (E <= 1024, k <= min(E,16), d %% 8 == 0)", E, k, d);
  MOE_CHECK_ARG(x && w_router && logits && topk_ids && topk_weights && expert_offsets && sorted_pairs && pair_pos &&
                    active_experts && counters,
                MOE_ERR_INVALID_ARG, "moe_route_align: null pointer");
  MOE_CHECK_ARG(block_m == 0 || tile_offsets, MOE_ERR_INVALID_ARG, "moe_route_align: block_m > 0 needs tile_offsets");
  MOE_CHECK_ARG(((uintptr_t)x % 16) == 0 && ((uintptr_t)w_router % 16) == 0 && ((uintptr_t)active_experts % 16) == 0,
                MOE_ERR_INVALID_ARG, "moe_route_align: x, w_router and active_experts must be 16-byte aligned");
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  hipStream_t s = (hipStream_t)stream;
  timing_begin(K_ROUTE, s);
  hipLaunchKernelGGL(k_route_align, dim3((unsigned)ceil_div(E, kAlignWaves), (unsigned)T), dim3(kAlignThreads), 0, s,
                     x, w_router, T, d, E, k, renormalize, block_m, bits, logits, topk_ids, topk_weights,
                     expert_offsets, sorted_pairs, pair_pos, active_experts, block_m > 0 ? tile_offsets : nullptr,
                     counters);
  timing_end(K_ROUTE, s);
  return check_launch("moe_route_align");
}
