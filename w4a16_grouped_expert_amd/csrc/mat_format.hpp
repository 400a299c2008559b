// Nested two/four-bit experts: the four-bit codes stored as two planes (high and
// low two bits) so that an expert can run at two bits by reading only the high
// plane, with the dropped bits replaced by their mean (floor and compensation),
// and each expert's precision in a step chosen from its routing weights (page
// "MatMoE: Dynamic Mixed-Precision Quantization for Efficient MoE Inference",
// arXiv abstract: nested multi-precision experts, floor-and-compensation
// quantisation, bit-widths allocated from routing scores; the four-bit codes are
// those of ExactMoE, page "Every Expert Counts: ExactMoE for Memory-Efficient
// W4A16 Inference", Abstract).
//
// Layout m1: plane tiles of 16 rows x 256 columns (two quantisation groups), rows
// in the gate/up interleaved order of layout v1, the scale array of layout v1; one
// 1024-byte tile per plane.  Lane L owns 16 bytes of each plane tile: 32-bit words
// j = 0..3 with K steps 2j and 2j + 1 of its MFMA A fragment (row L % 16, eight
// consecutive columns per K step; steps 0-3 are the first group, 4-7 the second).
// Element m of K step 2j + t has pair index p = 4t + m / 2 and its 2-bit field at
// bit (5 + 2p + 16 (m % 2)) mod 32: rotating the word right by 2p puts the pair at
// bits 5-6 and 21-22, the top mantissa bits of two bf16 with exponent 0.
//
// Decode of a pair: two bits, bf16(1 + h/4) = (rot(h) & 0x00600060) | 1.0 (one
// and-or after the rotation); four bits, bf16(1 + c/16) with c = 4h + l: the low
// plane rotated two places further lands at bits 3-4, so
// (rot(h) & 0x00600060) | (rot2(l) & 0x00180018) | 1.0 is the code of layout v1.
// With A = sum over a group of (decoded value) * x (exact products, fp32 sums)
// and X = sum x:
//   four bits:  sum (c - 8) x        = 16 A - 24 X
//   two bits:   sum (4h + 1.5 - 8) x = 16 A - 22.5 X
// each scaled once per group in fp32.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kPlaneTileBytes = 1024;
constexpr int kPlaneK = 256;  // columns per plane tile

struct MatOffsets {
  int64_t hi13, lo13, sc13, hi2, lo2, sc2;
};

// Sections of an m1 blob: the two-bit part first (w13 high plane, w13 scales, w2
// high plane, w2 scales), then the low planes (w13, w2), each 256-byte aligned, so
// loading an expert at two bits moves one prefix of the blob.
inline MatOffsets mat_offsets(int d, int I) {
  auto up = [](int64_t v) { return (v + 255) / 256 * 256; };
  MatOffsets m;
  int64_t o = 0;
  m.hi13 = o;
  o = up(o + (int64_t)2 * I * d / 4);
  m.sc13 = o;
  o = up(o + (int64_t)2 * I * (d / kGroup) * 2);
  m.hi2 = o;
  o = up(o + (int64_t)d * I / 4);
  m.sc2 = o;
  o = up(o + (int64_t)d * (I / kGroup) * 2);
  m.lo13 = o;
  o = up(o + (int64_t)2 * I * d / 4);
  m.lo2 = o;
  return m;
}

// K step t (0..1) of a plane word: bf16x8 operand from the high plane word (and,
// for four bits, the low plane word) holding it.  mhi = 0x00600060,
// mlo = 0x00180018, one = 0x3F803F80 (vgpr_const values let the compiler fuse
// each mask and or into one v_and_or_b32).
template <bool FULL>
__device__ __forceinline__ u32x4_t decode_step(uint32_t hw, uint32_t lw, int t, uint32_t mhi = 0x00600060u,
                                               uint32_t mlo = 0x00180018u, uint32_t one = 0x3F803F80u) {
  u32x4_t o;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    const int p = 4 * t + pp;
    const uint32_t rh = p ? __builtin_amdgcn_alignbit(hw, hw, 2 * p) : hw;
    uint32_t v = (rh & mhi) | one;
    if (FULL) {
      // an empty asm keeps the partial word opaque, so each field takes one
      // v_and_or_b32 (the compiler would otherwise fuse the three terms into
      // two ands and an or3); it emits no instruction
      asm("" : "+v"(v));
      v |= __builtin_amdgcn_alignbit(lw, lw, 2 * p + 2) & mlo;
    }
    o[pp] = v;
  }
  return o;
}

}  // namespace moe
