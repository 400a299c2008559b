// Grouped W4A16 expert GEMMs for many tokens per expert (prefill), MFMA-tiled
// (ExactMoE, page "Every Expert Counts: ExactMoE for Memory-Efficient W4A16
// Inference", Abstract: all selected experts through fused grouped kernels on
// four-bit group-128 weights).
//
// A block of eight wavefronts computes a 256 (weight rows) x 128 (tokens of one
// expert) tile; wavefront w owns rows 64 (w % 4) .. + 63 and tokens 64 (w / 4) ..
// + 63 as 4 x 4 blocks of 16x16x32 bf16 MFMA.  Per K group of 128 the block
// stages, in a 3-stage LDS pipeline filled by LDS-DMA (buffer_load ... lds, no
// registers): the 128 activation rows (gathered through the permutation; 16-byte
// chunks XOR-swizzled so the MFMA B-fragment reads are bank-conflict free) and the
// 16 packed 16 x 128 weight tiles; the per-token activation sums ride one group
// ahead and the bf16 scales two, in rings of their own.  Weights are decoded in
// registers to bf16 1 + c/16.
//
// One accumulator per output carries the whole K loop.  With D_g the group's
// sum of (c - 8) x / 16 and e_g the group's scale (a zero scale replaced by the
// previous one: its group is all zero codes and adds nothing), the accumulator
// holds A_g = sum over g' <= g of D_g' e_g' / e_g, i.e.
//   A_g = A_{g-1} * (e_{g-1} / e_g) - 1.5 * sum_k x + MFMA sum of (1 + c/16) x,
// one fma per output per group, applied behind the last MFMAs of group g - 1
// (the last group's applies the factor 16 e_last, which gives the result).  The ratio of each row is computed once per group by the
// thread that owns the row and handed over in LDS.  sum_k x per token and group
// is precomputed (activations: a small pass; SwiGLU output: written by the
// gate/up epilogue, whose block covers exactly two groups of h).
//
// Blocks are persistent; the tile list (active expert, token tile, row tile) is
// built per block from the work list of moe_align and walked in an order that
// keeps the blocks resident on one XCD on the same expert, so its weights and
// activations are fetched into that XCD's L2 once.
#include "ffn_common.hpp"

namespace moe {

constexpr int kPBM = 128;                  // tokens per block tile
constexpr int kPBN = 256;                  // weight rows per block tile
constexpr int kPTiles = kPBN / kTileRows;  // packed 16-row tiles per block tile
constexpr int kPWaves = 8;                 // 4 row quarters x 2 token halves of the block tile
constexpr int kPThreads = 64 * kPWaves;
constexpr int kXcds = 8;

// xsum[t][g] = sum of x[t][128 g .. 128 g + 127] in fp32 (one wavefront per token).
__global__ __launch_bounds__(256) void k_group_sums(const uint16_t* __restrict__ x, int T, int d,
                                                    float* __restrict__ xsum) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int G = d / kGroup;
  for (int c0 = 0; c0 < d / 8; c0 += 64) {
    const int ch = c0 + lane;  // 16-byte chunk; a group is 16 chunks
    float s = 0.f;
    if (ch < d / 8) {
      const u32x4_t q = *reinterpret_cast<const u32x4_t*>(x + (int64_t)t * d + 8 * ch);
#pragma unroll
      for (int m = 0; m < 4; ++m) s += __uint_as_float(q[m] << 16) + __uint_as_float(q[m] & 0xFFFF0000u);
    }
    s += __shfl_xor(s, 8);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 1);
    if ((lane & 15) == 0 && ch < d / 8) xsum[(int64_t)t * G + ch / 16] = s;
  }
}

// ---------------------------------------------------------------- LDS DMA
// global_load_lds: each lane's 16 (or 4) bytes at `g` land in LDS at
// lds_base + 16 * lane (4 * lane), with no registers in between.  Written as
// inline asm with M0 saved and restored around it: the compiler neither sees
// these loads in its wait counts nor assumes anything about the LDS they fill,
// so every consumer waits explicitly (stage_barrier) and the stages are only
// filled through these calls and read with plain LDS reads.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(g), "s"(lds_base) : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(g), "s"(lds_base) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// The same through a buffer resource: the address is base + voff (per lane) + soff
// (wave-uniform), so advancing a stream by one K group costs no vector ALU work.
__device__ __forceinline__ i32x4_t raw_rsrc(const void* base) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4_t{__builtin_amdgcn_readfirstlane((int)(uint32_t)a), __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFF)),
                 -1, kBufferRsrcWord3};
}
__device__ __forceinline__ void buf_dma16(i32x4_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %4 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(rsrc), "s"(lds_base), "s"(soff) : "memory");
}
__device__ __forceinline__ void buf_dma4(i32x4_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %4 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(rsrc), "s"(lds_base), "s"(soff) : "memory");
}

// One stage of the LDS pipeline: the activations and weights of one K group.
struct PrefillStage {
  u32x4_t x[kPBM * 16];     // chunk kc of token t at slot 16 t + (kc ^ (t & 15))
  u32x4_t w[kPTiles * 64];  // packed tile j: lane l's 16 bytes at [64 j + l], as in HBM
};
constexpr int kStages = 3;

// Wait until at most N vector-memory operations of this wavefront are in flight
// (they retire in order; LDS-DMA included), finish its LDS operations, then meet
// the block.
template <int N>
__device__ __forceinline__ void stage_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// SiLU in fp32 with the hardware exp and reciprocal (a few ulp; h is rounded to bf16).
__device__ __forceinline__ float silu_fast(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

// Pipeline, in K groups g = 0 .. G-1 (a "top of g" is the block barrier that
// starts group g, after which batch g is resident):
//   batch k, issued during group k - 2: activations and weights of group k
//     (stage k % 3), the group sums of group k + 1 (ring of 4) and the scales of
//     group k + 2 (ring of 4);
//   at the top of k, the thread that owns row r turns the scales of group k + 2
//     into the ratio e_{k+1} / e_{k+2} (16 e_last once past the end), ring of 2;
//   during group g - 1 every lane reads the ratios and group sums it needs at the
//     top of g into registers, so group g starts with the rescale fma right away.
// Stages and rings are indexed by the workgroup's running group count (its tiles'
// groups one after another), so a tile's first batches may be issued while the
// previous tile still reads its last stage.
template <bool GATEUP>
__global__ __launch_bounds__(kPThreads) void k_prefill(
    FfnDev f, const uint16_t* __restrict__ act, const float* __restrict__ asum, uint16_t* __restrict__ hout,
    float* __restrict__ hsum_out, uint16_t* __restrict__ yout) {
  const int K = GATEUP ? f.d : f.I;
  const int N = GATEUP ? 2 * f.I : f.d;
  const int G = K / kGroup;
  const int NT = (N + kPBN - 1) / kPBN;
  const int GH = f.I / kGroup;  // groups of h = row tiles of gate/up

  __shared__ PrefillStage st[kStages];
  __shared__ float s_xs[4][kPBM];      // group sums of group g at [g % 4]: token 64 h + 16 b + c at [64 h + 4 c + b]
  __shared__ uint16_t s_sc[4][kPBN];   // bf16 scales of group g at [g % 4], row r of the block tile at [r]
  __shared__ float s_ratio[2][kPBN];   // e_{g-1} / e_g per row at [g % 2]; 16 e_last at [G % 2]
  __shared__ int s_row[2][kPBM];       // activation rows of this tile and the next (see fill_rows)
  __shared__ int s_pref[MOE_MAX_EXPERTS + 1];
  __shared__ uint16_t s_lpref[MOE_MAX_EXPERTS + 1];
  __shared__ float s_hs[4][kPBM];      // gate/up: per-token h sums of each row quarter's 32 columns
  __shared__ int s_wsum[kPWaves], s_wlsum[kPWaves];

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave & 3, wt = wave >> 2;  // rows 64 wr .. + 63, tokens 64 wt .. + 63 of the block tile
  const int col = lane & 15, kq = lane >> 4;
  const int U = f.active[0];
  const i32x4_t* work = reinterpret_cast<const i32x4_t*>(f.active + 4);

  // Tiles of active expert u: ceil(count / 128) token tiles x NT row tiles.  A
  // last token tile with at most 64 tokens (one token half busy) is a light tile;
  // the light tiles of every expert follow all the others, so the blocks that
  // get one tile more than the rest get light ones.  Exclusive prefixes in LDS:
  // s_pref of the other tiles, s_lpref of the experts with a light tile.
  if (tid == 0) {
    s_pref[0] = 0;
    s_lpref[0] = 0;
  }
  for (int base = 0; base < U; base += kPThreads) {
    __syncthreads();
    const int u = base + tid;
    const int n_e = u < U ? work[u][2] : 0;
    const int rem = n_e % kPBM;
    const int light = (rem > 0 && rem <= kPBM / 2) ? 1 : 0;
    int v = ((n_e + kPBM - 1) / kPBM - light) * NT, lv = light;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(v, off), ol = __shfl_up(lv, off);
      if (lane >= off) {
        v += o;
        lv += ol;
      }
    }
    if (lane == 63) s_wsum[wave] = v;
    if (lane == 63) s_wlsum[wave] = lv;
    __syncthreads();
    int add = s_pref[base], addl = s_lpref[base];
    for (int w = 0; w < wave; ++w) {
      add += s_wsum[w];
      addl += s_wlsum[w];
    }
    if (u < U) {
      s_pref[u + 1] = add + v;
      s_lpref[u + 1] = (uint16_t)(addl + lv);
    }
  }
  __syncthreads();
  const int total_main = s_pref[U];
  const int total = total_main + (int)s_lpref[U] * NT;

  // Workgroups are dealt to the XCDs round robin; renumber them so each XCD owns
  // a contiguous run of tile slots (consecutive tiles share an expert).
  const int nblk = gridDim.x;
  const int vb = (nblk % kXcds == 0) ? (blockIdx.x % kXcds) * (nblk / kXcds) + blockIdx.x / kXcds : blockIdx.x;

  const uint32_t kMask = vgpr_const(0x00780078u), kOne = vgpr_const(0x3F803F80u);

  auto active_of = [&](int t) {  // the active expert of tile t
    int lo = 0, hi = U;
    if (t < total_main) {  // s_pref[u] <= t < s_pref[u + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] <= t) lo = mid; else hi = mid;
      }
    } else {  // light tile j: s_lpref[u] <= j < s_lpref[u + 1]
      const int j = (t - total_main) / NT;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int)s_lpref[mid] <= j) lo = mid; else hi = mid;
      }
    }
    return lo;
  };
  struct Tile {
    int row0, n_e, mt, nt;
    const uint8_t* blob;
  };
  // token tile of tile t of active expert u with n_e tokens (row tiles fastest:
  // neighbours share the token tile; a light tile is the expert's last one)
  auto mt_of = [&](int t, int u, int n_e) {
    return t < total_main ? (t - s_pref[u]) / NT : (n_e + kPBM - 1) / kPBM - 1;
  };
  auto tile_of = [&](int t, int u, const i32x4_t& w) {
    Tile tl;
    tl.row0 = w[1];
    tl.n_e = w[2];
    tl.mt = mt_of(t, u, tl.n_e);
    tl.nt = t < total_main ? (t - s_pref[u]) % NT : (t - total_main) % NT;
    tl.blob = f.blob(w[0]);
    return tl;
  };
  // activation row of each of the tile's tokens (token for gate/up, sorted position
  // for down), -1 = none; thread tid < kPBM fills row tid
  auto fill_rows = [&](const Tile& tl, int* rows, int pair_val, bool have_pair) {
    if (tid < kPBM) {
      const int r = tl.mt * kPBM + tid;
      int row = -1;
      if (r < tl.n_e) row = GATEUP ? (have_pair ? pair_val : f.sorted_pairs[tl.row0 + r]) / f.k : tl.row0 + r;
      rows[tid] = row;
    }
  };

  // ---- this lane's DMA sources for a tile (group 0; group g adds g * stride)
  // Activations: instruction j of wavefront w fills slots s = 64 (4 w + j) + lane,
  // i.e. chunk (s % 16) ^ (t % 16) of token t = s / 16.  Rows are gathered tokens
  // for gate/up (byte offsets from x, below 4 GiB by the host check) and
  // consecutive sorted positions for down (offsets from the tile's first row);
  // padding tokens read the tile's first row and their outputs are dropped.
  // Weights: instruction j of wavefront w fills packed tile 2 w + j.  A last row
  // tile past N reads the final packed tile in place of the missing ones (those
  // rows are computed but not stored).
  // Scales (wavefront 0, two 4-byte instructions): word p = 64 j + lane holds rows
  // 2 (p % 8), + 1 of tile p / 8.  Group sums (wavefront 1, two instructions):
  // slot p = 64 j + lane holds token 64 j + 16 (p % 4) + (p % 64) / 4.
  const int last_tile = N / kTileRows - 1;
  uint32_t xoff[4], woff[2], aoff[2] = {0u, 0u};
  uint32_t astep = 0;  // bytes per group
  i32x4_t rs_x, rs_w, rs_a;
  auto setup_dma = [&](const Tile& tl, const int* rows) {
    const uint8_t* act_tile =
        reinterpret_cast<const uint8_t*>(GATEUP ? act : act + (int64_t)(tl.row0 + tl.mt * kPBM) * K);
    rs_x = raw_rsrc(act_tile);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sl = (wave * 4 + j) * 64 + lane;
      const int t = sl >> 4, kc = (sl & 15) ^ (t & 15);
      int row;
      if (GATEUP) row = rows[t] >= 0 ? rows[t] : rows[0];
      else row = rows[t] >= 0 ? t : 0;
      xoff[j] = ((uint32_t)row * (uint32_t)K + 8u * (uint32_t)kc) * 2u;
    }
    rs_w = raw_rsrc(tl.blob + (GATEUP ? f.off_w13_codes : f.off_w2_codes));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      woff[j] = (uint32_t)min(tl.nt * kPTiles + 2 * wave + j, last_tile) * (uint32_t)(G * kTileBytes) + 16u * lane;
    rs_a = raw_rsrc(wave == 0 ? (const void*)(tl.blob + (GATEUP ? f.off_w13_scales : f.off_w2_scales))
                              : (const void*)asum);
    if (wave == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int p = 64 * j + lane;
        aoff[j] = ((uint32_t)min(tl.nt * kPTiles + (p >> 3), last_tile) * (uint32_t)(G * kTileRows) + 2u * (p & 7)) * 2u;
      }
      astep = kTileRows * 2;
    } else if (wave == 1) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = 64 * j + 16 * (lane & 3) + (lane >> 2);
        const int r = rows[t] >= 0 ? rows[t] : rows[0];
        aoff[j] = (uint32_t)r * (uint32_t)(GATEUP ? G : GH) * 4u;
      }
      astep = 4;
    }
  };
  // The LDS rings are indexed by a running group count q = qb + g (mod 12: rings
  // of 2, 3 and 4), so a tile's first batches can land while the previous tile
  // still reads its last stage.
  auto issue_aux = [&](int g, int qbase) {  // scales (wave 0) or group sums (wave 1) of group g
    if (wave == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        buf_dma4(rs_a, aoff[j], (uint32_t)g * astep, lds_addr(&s_sc[(qbase + g) & 3][128 * j]));
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        buf_dma4(rs_a, aoff[j], (uint32_t)g * astep, lds_addr(&s_xs[(qbase + g) & 3][64 * j]));
    }
  };
  // Part `part` (0..3) of batch k: one activation instruction, a weight
  // instruction on parts 0 and 2, the scales / group sums on part 1.
  auto issue_part = [&](int k, int part, int qbase) {
    PrefillStage& S = st[(qbase + k) % kStages];
    buf_dma16(rs_x, xoff[part], (uint32_t)k * (kGroup * 2), lds_addr(&S.x[(wave * 4 + part) * 64]));
    if ((part & 1) == 0)
      buf_dma16(rs_w, woff[part >> 1], (uint32_t)k * kTileBytes, lds_addr(&S.w[(wave * 2 + (part >> 1)) * 64]));
    if (part == 1) {
      if (wave == 0 && k + 2 < G) issue_aux(k + 2, qbase);
      if (wave == 1 && k + 1 < G) issue_aux(k + 1, qbase);
    }
  };
  // DMA instructions of this wavefront in batch k (6, plus two for the scales /
  // group sums it carries)
  auto batch_has_aux = [&](int k) { return (wave == 0 && k + 2 < G) || (wave == 1 && k + 1 < G); };
  // prologue DMA of a tile: scales of groups 0, 1 and the group sums of group 0,
  // then batches 0 and 1
  auto issue_prologue = [&](int qbase) {
    if (wave == 0) {
      issue_aux(0, qbase);
      if (G > 1) issue_aux(1, qbase);
    } else if (wave == 1) {
      issue_aux(0, qbase);
    }
#pragma unroll
    for (int part = 0; part < 4; ++part) issue_part(0, part, qbase);
    if (G > 1) {
#pragma unroll
      for (int part = 0; part < 4; ++part) issue_part(1, part, qbase);
    }
  };
  auto bf16_at = [](uint16_t b) { return __uint_as_float((uint32_t)b << 16); };

  // The next tile's work record is requested at the start of a tile and (gate/up)
  // its gathered token ids at the top of the tile's second-to-last group.  Down
  // pass with G >= 4: the next tile's rows, DMA sources and prologue DMA are set
  // up at the top of the last group, so those round trips overlap the last group
  // and the epilogue (measured: 5 % off the down pass; the gate/up pass, whose
  // last group and epilogue carry more work, ran 3 % slower with it).
  int tile = vb;
  int un = tile < total ? active_of(tile) : 0;
  i32x4_t w4n = tile < total ? work[un] : i32x4_t{0, 0, 0, 0};
  int pair_next = 0, pair_tile = -1;  // thread tid < kPBM: sorted_pairs entry of its row in tile pair_tile
  bool ready = false;                 // this tile's setup and prologue DMA went out during the previous tile
  int qb = 0, rb = 0;                 // running group count (mod 12), this tile's s_row buffer
  for (; tile < total; tile += nblk) {
    const int u = un;
    const Tile cur = tile_of(tile, u, w4n);
    const int row0 = cur.row0, n_e = cur.n_e, mt = cur.mt, nt = cur.nt;
    const int next = tile + nblk;
    if (next < total) {
      un = active_of(next);
      w4n = work[un];
    }
    if (!cur.blob) {  // uniform over the block
      ready = false;
      continue;
    }
    if (!ready) {
      __syncthreads();  // the previous tile is done with every LDS buffer
      fill_rows(cur, s_row[rb], pair_next, pair_tile == tile);
      __syncthreads();
      setup_dma(cur, s_row[rb]);
      issue_prologue(qb);
    }
    bool next_ready = false;

    f32x4_t acc[4][4];
    // this wavefront's token half holds tokens of the tile (else it skips the
    // products of every group: the last tile of an expert is often half empty)
    const bool live = __builtin_amdgcn_readfirstlane(mt * kPBM + 64 * wt < n_e ? 1 : 0) != 0;
    float e_next = 1.f;  // scale chain of row `tid` (threads 0 .. 255): e of the newest group seen
    f32x4_t rn[4];       // this lane's ratios for the next group
    f32x4_t xsn;         // this lane's group sums for the next group

    // wavefronts 0 and 1 wait for their prologue loads only: at most n_after younger
    // operations (the batches, and any stores since) may stay in flight
    if (wave < 2) {
      const int n_after = 6 + (batch_has_aux(0) ? 2 : 0) + (G > 1 ? 6 + (batch_has_aux(1) ? 2 : 0) : 0);
      if (n_after == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      else if (n_after == 14) asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
      else if (n_after == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
      else if (n_after == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (tid < kPBN) {
      const float s0 = bf16_at(s_sc[qb & 3][tid]);
      const float e0 = s0 != 0.f ? s0 : 1.f;
      float out;
      if (G > 1) {
        const float s1 = bf16_at(s_sc[(qb + 1) & 3][tid]);
        e_next = s1 != 0.f ? s1 : e0;
        out = e0 * __builtin_amdgcn_rcpf(e_next);
      } else {
        e_next = e0;
        out = 16.f * e0;
      }
      s_ratio[(qb + 1) & 1][tid] = out;
    }

    for (int g = 0; g < G; ++g) {
      // batch g has landed (batch g + 1 may still be in flight); everyone is done with stage g - 1
      if (g + 1 < G) {
        if (batch_has_aux(g + 1)) stage_wait_barrier<8>(); else stage_wait_barrier<6>();
      } else {
        stage_wait_barrier<0>();
      }
      if (GATEUP && g == G - 2 && next < total && tid < kPBM) {
        const int rn_ = mt_of(next, un, w4n[2]) * kPBM + tid;
        if (rn_ < w4n[2]) pair_next = f.sorted_pairs[w4n[1] + rn_];
        pair_tile = next;
      }
      if (!GATEUP && G >= 4 && g == G - 1 && next < total) {
        const Tile nx = tile_of(next, un, w4n);
        if (nx.blob) {  // uniform over the block
          fill_rows(nx, s_row[rb ^ 1], pair_next, pair_tile == next);
          __syncthreads();
          setup_dma(nx, s_row[rb ^ 1]);
          issue_prologue((qb + G) % 12);
          next_ready = true;
        }
      }
      // Row tid's ratio two groups ahead (16 e_last once that is past the end).
      if (tid < kPBN && g + 2 <= G) {
        float out;
        if (g + 2 < G) {
          const float sn = bf16_at(s_sc[(qb + g + 2) & 3][tid]);
          const float en = sn != 0.f ? sn : e_next;
          out = e_next * __builtin_amdgcn_rcpf(en);
          e_next = en;
        } else {
          out = 16.f * e_next;
        }
        s_ratio[(qb + g) & 1][tid] = out;
      }

      const PrefillStage& S = st[(qb + g) % kStages];
      if (!live) {
        // a token half without tokens: no products, only its share of the batch's
        // DMA (its outputs are not stored; acc is set once so that they are defined)
        if (g == 0) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[t][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        if (g + 2 < G) {
#pragma unroll
          for (int i = 0; i < 4; ++i) issue_part(g + 2, i, qb);
        }
        continue;
      }
      // g = 0: acc = -1.5 sum_k x; later groups start from the rescale at the end of the previous one
      if (g == 0) {
        const f32x4_t xs = *reinterpret_cast<const f32x4_t*>(&s_xs[qb & 3][64 * wt + 4 * col]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float c = -1.5f * xs[b];
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[t][b] = f32x4_t{c, c, c, c};
        }
      }
      // applied at the end of this group: acc * (e_g / e_{g+1}) - 1.5 sum_k x of group g + 1,
      // or acc * 16 e_last after the last group (written at the top of g - 1, or of G - 2)
      float cn[4];
      {
        const float* rp = &s_ratio[(qb + g + 1) & 1][64 * wr];
#pragma unroll
        for (int t = 0; t < 4; ++t) rn[t] = *reinterpret_cast<const f32x4_t*>(&rp[16 * t + 4 * kq]);
        xsn = *reinterpret_cast<const f32x4_t*>(&s_xs[(qb + g + 1) & 3][64 * wt + 4 * col]);
        const bool more = g + 1 < G;
#pragma unroll
        for (int b = 0; b < 4; ++b) cn[b] = more ? -1.5f * xsn[b] : 0.f;
      }

      u32x4_t cw[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) cw[t] = S.w[(wr * 4 + t) * 64 + lane];
      const u32x4_t* xrow = &S.x[(wt * 64 + col) * 16];  // token block b adds 256 slots
      u32x4_t xb[4], xn[4];
      if (g + 2 < G) {
#pragma unroll
        for (int i = 0; i < 4; ++i) issue_part(g + 2, i, qb);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) xb[b] = xrow[b * 256 + (kq ^ col)];
      u32x4_t wa[4], wn[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) wa[t] = decode_word_biased(cw[t][0], kMask, kOne);
      auto dec1 = [&](uint32_t w, int j) -> uint32_t {
        const uint32_t v = j == 0 ? w : (j == 3 ? rotr32(w, 12) : (w >> (4 * j)));
        return (v & kMask) | kOne;
      };
      // Four K steps of 16 products.  Behind each product goes one word of the next
      // step's decode (steps 0 to 2) or the rescale of the product two places back
      // (step 3), in an order pinned by scheduling barriers: left to itself the
      // compiler puts the VALU work in front of each step's products, where it
      // cannot overlap them.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < 3) {
#pragma unroll
          for (int b = 0; b < 4; ++b) xn[b] = xrow[b * 256 + ((4 * (i + 1) + kq) ^ col)];
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          const int t = m & 3, b = m >> 2;
          acc[t][b] = mfma16x16x32(as_bf16x8(wa[t]), as_bf16x8(xb[b]), acc[t][b]);
          if (i < 3) {
            wn[m >> 2][m & 3] = dec1(cw[m >> 2][i + 1], m & 3);
          } else if (m >= 2) {
            const int t2 = (m - 2) & 3, b2 = (m - 2) >> 2;
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[t2][b2][q] = fmaf(acc[t2][b2][q], rn[t2][q], cn[b2]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (i < 3) {
#pragma unroll
          for (int b = 0; b < 4; ++b) xb[b] = xn[b];
#pragma unroll
          for (int t = 0; t < 4; ++t) wa[t] = wn[t];
        }
      }
#pragma unroll
      for (int m = 14; m < 16; ++m) {
        const int t2 = m & 3, b2 = m >> 2;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[t2][b2][q] = fmaf(acc[t2][b2][q], rn[t2][q], cn[b2]);
      }
    }

    if (GATEUP) {
      // tiles (0,1) and (2,3) of the wavefront are gate/up pairs: h columns nt*128 + wr*32 + 16p + 4kq + q
      float hs[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        hs[b] = 0.f;
        const int r = wt * 64 + b * 16 + col;
        const int pos = row0 + mt * kPBM + r;
        const bool ok = mt * kPBM + r < n_e;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          float hf[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) hf[q] = silu_fast(acc[2 * p][b][q]) * acc[2 * p + 1][b][q];
          const u32x2_t o = pack_bf16x4(hf[0], hf[1], hf[2], hf[3]);
#pragma unroll
          for (int w = 0; w < 2; ++w)  // the sum of the bf16 values that are stored
            hs[b] += __uint_as_float(o[w] << 16) + __uint_as_float(o[w] & 0xFFFF0000u);
          if (ok) {
            const int hcol = nt * 128 + wr * 32 + 16 * p + 4 * kq;
            *reinterpret_cast<u32x2_t*>(hout + (int64_t)pos * f.I + hcol) = o;
          }
        }
      }
      // per-token sum of this block's 128 h columns (one group of h): lanes kq, then the four row quarters
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        hs[b] += __shfl_xor(hs[b], 16);
        hs[b] += __shfl_xor(hs[b], 32);
        if (kq == 0) s_hs[wr][wt * 64 + b * 16 + col] = hs[b];
      }
      __syncthreads();
      if (tid < kPBM) {
        const int r = mt * kPBM + tid;
        if (r < n_e) hsum_out[(int64_t)(row0 + r) * GH + nt] = (s_hs[0][tid] + s_hs[1][tid]) + (s_hs[2][tid] + s_hs[3][tid]);
      }
    } else {
      // the pair's output row in bf16 (the combine sums the k rows in fp32)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int r = wt * 64 + b * 16 + col;
        if (mt * kPBM + r < n_e) {
          const int pos = row0 + mt * kPBM + r;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int n = nt * kPBN + wr * 64 + t * 16 + 4 * kq;
            const u32x2_t o = pack_bf16x4(acc[t][b][0], acc[t][b][1], acc[t][b][2], acc[t][b][3]);
            if (n < N) *reinterpret_cast<u32x2_t*>(yout + (int64_t)pos * f.d + n) = o;
          }
        }
      }
    }
    ready = next_ready;
    qb = (qb + G) % 12;
    rb ^= 1;
  }
}

template <typename Kern>
static int prefill_grid(Kern kern, int slot) {
  static int cached[2] = {0, 0};
  if (!cached[slot]) {
    int dev = 0, cus = 0, per_cu = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kPThreads, 0);
    cached[slot] = std::max(1, cus) * std::max(1, per_cu);
  }
  return cached[slot];
}

int64_t prefill_extra_bytes(int T, int d, int I, int k) {
  const int64_t P = (int64_t)T * k;
  return (int64_t)T * (d / kGroup) * 4 + P * (I / kGroup) * 4 + 512;
}

int launch_prefill(const FfnDev& f, uint16_t* h, uint16_t* y, float* xsum, float* hsum, hipStream_t s) {
  // the kernels address x, h and the group sums with 32-bit byte offsets
  if ((int64_t)f.T * f.d * 2 >= (int64_t(1) << 32) || f.P * f.I * 2 >= (int64_t(1) << 32)) {
    set_error("moe_w4a16_grouped_ffn: prefill needs T * d * 2 and T * k * I * 2 below 4 GiB (T=%d d=%d I=%d k=%d)", f.T,
              f.d, f.I, f.k);
    return MOE_ERR_UNSUPPORTED_SHAPE;
  }
  hipLaunchKernelGGL(k_group_sums, dim3((unsigned)ceil_div(f.T, 4)), dim3(256), 0, s, f.x, f.T, f.d, xsum);
  int rc = check_launch("activation group sums");
  if (rc) return rc;
  // upper bound of tiles: sum over experts of ceil(n_e / 128) <= P / 128 + U
  const int64_t mt_bound = f.P / kPBM + f.umax;
  const int64_t tiles_gu = mt_bound * ceil_div(2 * f.I, kPBN);
  const int64_t tiles_dn = mt_bound * ceil_div(f.d, kPBN);
  auto kgu = k_prefill<true>;
  auto kdn = k_prefill<false>;
  const int64_t grid_gu = std::min<int64_t>(prefill_grid(kgu, 0), tiles_gu);
  const int64_t grid_dn = std::min<int64_t>(prefill_grid(kdn, 1), tiles_dn);
  timing_begin(K_GATEUP_PREFILL, s);
  hipLaunchKernelGGL(kgu, dim3((unsigned)grid_gu), dim3(kPThreads), 0, s, f, f.x, (const float*)xsum, h, hsum,
                     (uint16_t*)nullptr);
  timing_end(K_GATEUP_PREFILL, s);
  rc = check_launch("grouped gate/up (prefill)");
  if (rc) return rc;
  timing_begin(K_DOWN_PREFILL, s);
  hipLaunchKernelGGL(kdn, dim3((unsigned)grid_dn), dim3(kPThreads), 0, s, f, (const uint16_t*)h, (const float*)hsum,
                     (uint16_t*)nullptr, (float*)nullptr, y);
  timing_end(K_DOWN_PREFILL, s);
  return check_launch("grouped down (prefill)");
}

}  // namespace moe
