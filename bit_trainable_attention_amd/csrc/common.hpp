// Device-side building blocks shared by the HIP kernels of the SageBwd-style INT8 attention.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA matrix cores.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sagebwd {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

enum { DT_FP16 = 0, DT_BF16 = 1 };

// ---------------------------------------------------------------- 16-bit storage <-> float
template <int DT> __device__ __forceinline__ float to_f32(unsigned short b);
template <> __device__ __forceinline__ float to_f32<DT_FP16>(unsigned short b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
template <> __device__ __forceinline__ float to_f32<DT_BF16>(unsigned short b) {
  return __uint_as_float(((unsigned)b) << 16);
}
// float -> 16-bit, round to nearest even (hardware conversions on gfx950).
template <int DT> __device__ __forceinline__ unsigned short from_f32(float x);
template <> __device__ __forceinline__ unsigned short from_f32<DT_FP16>(float x) {
  return __builtin_bit_cast(unsigned short, (_Float16)x);
}
template <> __device__ __forceinline__ unsigned short from_f32<DT_BF16>(float x) {
  return __builtin_bit_cast(unsigned short, (__bf16)x);
}

// ---------------------------------------------------------------- MFMA wrappers
// Layouts (checked on the hardware): for an M x M result with M = 32, lane l holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32 in register r (r = 0..15). Operand A: lane l
// holds row l%32 and contraction slots (l/32, s); operand B: lane l holds column l%32
// and the same contraction slots. A and B pair their slots identically, so any fixed
// assignment of contraction indices to (lane group, slot) is valid if both agree.
__device__ __forceinline__ i32x16 mfma_i8_32x32x32(i32x4 a, i32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
template <int DT> __device__ __forceinline__ f32x16 mfma_16b_32x32x16(u16x8 a, u16x8 b, f32x16 c);
template <> __device__ __forceinline__ f32x16 mfma_16b_32x32x16<DT_FP16>(u16x8 a, u16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mfma_16b_32x32x16<DT_BF16>(u16x8 a, u16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- small helpers
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Pack the low bytes of four 32-bit words into one word (byte i <- word i).
__device__ __forceinline__ unsigned pack4_lo_bytes(unsigned w0, unsigned w1, unsigned w2, unsigned w3) {
  unsigned lo = __builtin_amdgcn_perm(w1, w0, 0x0c0c0400u);
  unsigned hi = __builtin_amdgcn_perm(w3, w2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// INT8 code of x under inverse scale inv: round-to-nearest-even of fl(x * inv), for
// |x * inv| <= 127. The product is rounded to float32 first (no fused multiply-add);
// adding 1.5 * 2^23 then rounds it to an integer (nearest even) held in the low mantissa
// bits, whose low byte is the two's-complement code.
__device__ __forceinline__ unsigned quant_word(float x, float inv) {
#pragma clang fp contract(off)
  float t = x * inv;
  return __float_as_uint(t + 12582912.0f);
}

// In-kernel tile codes (P, dS): nearest-even integer of the exact product x * inv, rounded
// once by the fused multiply-add with 1.5 * 2^23 (|x * inv| <= 127.5); low byte = code.
__device__ __forceinline__ unsigned quant_word_fma(float x, float inv) {
  return __float_as_uint(__builtin_fmaf(x, inv, 12582912.0f));
}

}  // namespace sagebwd
