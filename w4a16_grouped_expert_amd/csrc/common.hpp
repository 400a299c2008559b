// Internal helpers shared by the HIP sources of the W4A16 MoE library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>

#include "w4a16_moe.h"

namespace moe {

// ---------------------------------------------------------------- host-side errors

void set_error(const char* fmt, ...);
void clear_error();

#define MOE_CHECK_ARG(cond, code, ...)      \
  do {                                       \
    if (!(cond)) {                           \
      ::moe::set_error(__VA_ARGS__);         \
      return (code);                         \
    }                                        \
  } while (0)

// Check the launch that was just enqueued.
int check_launch(const char* what);

// Timing hooks (see moe_timing_*): bracket one launch of `kernel_id`.
enum KernelId { K_GATEUP_DECODE = 0, K_DOWN_DECODE = 1, K_GATEUP_PREFILL = 2, K_DOWN_PREFILL = 3,
                K_COMBINE = 4, K_ROUTE = 5, K_ALIGN = 6, K_GATEUP_BF16 = 7, K_DOWN_BF16 = 8,
                K_GATEUP_MAT = 9, K_DOWN_MAT = 10, K_NUM = 11 };
void timing_begin(int kernel_id, hipStream_t s);
void timing_end(int kernel_id, hipStream_t s);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- device types

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;          // quantisation group along K
constexpr int kTileRows = 16;        // rows per packed tile
constexpr int kTileBytes = 1024;     // bytes per packed tile (16 x 128 x 4 bit)
// Word 3 of a raw (unswizzled, stride 0) buffer resource on gfx9: 32-bit data
// format; offsets at or past num_records read as zero.
constexpr int kBufferRsrcWord3 = 0x00020000;
// Cache-policy operand of the raw buffer builtins on gfx950: bit 1 = nt (streaming).
constexpr int kCacheNonTemporal = 2;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bf16 bits, round to nearest even (the conversion instruction of gfx950,
// v_cvt_pk_bf16_f32, which also keeps NaNs quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// two float32 values -> one word of two bf16 (lo in bits 0..15), one conversion instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){lo, hi}, b2_t));
}
// four float32 values -> four bf16 in two words, in order
__device__ __forceinline__ u32x2_t pack_bf16x4(float a, float b, float c, float d) {
  return u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

__device__ __forceinline__ uint32_t rotr32(uint32_t v, int n) {
  return __builtin_amdgcn_alignbit(v, v, n);
}

// 16x16x32 bf16 MFMA, fp32 accumulate: C[16 x 16] += A[16 x 32] * B[32 x 16].
// Lane l supplies A row (l % 16) and B column (l % 16), eight consecutive k each;
// C: lane l holds column l % 16, rows 4*(l / 16) + 0..3.
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// A constant the compiler cannot see through, materialised in a VGPR.  gfx9 VOP3
// encodings take no literal operand, so with visible constants the compiler
// splits (a & m) | o into v_and + v_or; with m and o in VGPRs it emits one
// v_and_or_b32 (and still tracks every hazard itself, as it is ordinary code).
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  uint32_t v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(c));
  return v;
}

// One 32-bit word of packed codes (8 elements) -> 8 bf16 values (1 + code/16).
// Element m's code sits at bit (3 + 4(m/2) + 16(m%2)) mod 32, so shifting right by
// 4p (rotating for p = 3, whose high field wraps to bits 0..2) puts elements 2p and
// 2p+1 at bits 3..6 and 19..22, i.e. straight into the top mantissa bits of two
// bf16 values with exponent 0 (0x3F80 = 1.0): seven VALU instructions per word.
// mask = 0x00780078, one = 0x3F803F80, passed as vgpr_const values by the caller.
__device__ __forceinline__ u32x4_t decode_word_biased(uint32_t w, uint32_t mask, uint32_t one) {
  u32x4_t r;
  r[0] = (w & mask) | one;
  r[1] = ((w >> 4) & mask) | one;
  r[2] = ((w >> 8) & mask) | one;
  r[3] = (rotr32(w, 12) & mask) | one;
  return r;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

}  // namespace moe
