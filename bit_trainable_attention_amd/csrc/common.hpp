// Device-side building blocks shared by the HIP kernels of the SageBwd-style quantised attention.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA matrix cores.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sagebwd {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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

// 16 x 16 products (checked on the hardware): lane l, register r of the result hold row
// 4*(l/16) + r and column l%16. Operand A: lane l holds row l%16; operand B: column l%16;
// lane group l/16 supplies the same contraction slots to both (16 bytes for the INT8 form,
// 8 16-bit values for the 16-bit form).
__device__ __forceinline__ i32x4 mfma_i8_16x16x64(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
template <int DT> __device__ __forceinline__ f32x4 mfma_16b_16x16x32(u16x8 a, u16x8 b, f32x4 c);
template <> __device__ __forceinline__ f32x4 mfma_16b_16x16x32<DT_FP16>(u16x8 a, u16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mfma_16b_16x16x32<DT_BF16>(u16x8 a, u16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b8). Inside each group of 16 lanes, lanes 2i and 2i+1
// name the two 8-byte halves of "row" i (i = 0..7); lane j of the group receives byte j of
// every row: result byte i = byte (j % 8) at the address of lane 2i + j/8 (checked on the
// hardware). Reading a 16-byte column block of 8 rows thus hands each lane one column.
__device__ __forceinline__ i32x2 lds_read_tr8(const int8_t* p) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p);
}

// Transposing LDS read of 16-bit values (ds_read_b64_tr_b16). Inside each group of 16 lanes,
// lanes 4k .. 4k+3 name the four 8-byte quarters of "row" k (k = 0..3, 16 values per row) and
// lane j of the group receives value j of every row: result element k = value (j % 4) at the
// address of lane 4k + j/4 (checked on the hardware). Reading four rows of a row-major 16-bit
// tile thus hands each lane one column: the transposed operand of a 16-bit MFMA.
__device__ __forceinline__ u16x4 lds_read_tr16(const void* p) {
  typedef short s16x4 __attribute__((vector_size(8)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}

// ---------------------------------------------------------------- small helpers
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Max over the 64 lanes (wave-uniform result). Floats are compared as integers: flipping
// the magnitude bits of negative values makes signed-integer order equal float order (for
// everything but NaN), so each butterfly step is one v_max_i32 with a DPP source (quad swaps,
// then row rotations by 4 and 8) and needs no NaN canonicalisation. The four row maxima are
// read out with v_readlane and combined on the scalar unit.
__device__ __forceinline__ int float_order_key(float x) {
  const int b = __float_as_int(x);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
template <int CTRL>
__device__ __forceinline__ int imax_dpp(int v) {
  return max(v, __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_max(float x) {
  int v = float_order_key(x);
  v = imax_dpp<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v = imax_dpp<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v = imax_dpp<0x124>(v);  // row_ror:4
  v = imax_dpp<0x128>(v);  // row_ror:8 -> every lane of a row holds the row max
  const int m = max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
                    max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
  return __int_as_float(m ^ ((m >> 31) & 0x7FFFFFFF));
}
// Two independent wave maxima, their butterfly steps interleaved so that each chain's DPP
// wait states are filled by the other chain.
__device__ __forceinline__ void wave_max2(float& x, float& y) {
  int u = float_order_key(x), v = float_order_key(y);
  u = imax_dpp<0xB1>(u);  v = imax_dpp<0xB1>(v);
  u = imax_dpp<0x4E>(u);  v = imax_dpp<0x4E>(v);
  u = imax_dpp<0x124>(u); v = imax_dpp<0x124>(v);
  u = imax_dpp<0x128>(u); v = imax_dpp<0x128>(v);
  const int mu = max(max(__builtin_amdgcn_readlane(u, 0), __builtin_amdgcn_readlane(u, 16)),
                     max(__builtin_amdgcn_readlane(u, 32), __builtin_amdgcn_readlane(u, 48)));
  const int mv = max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
                     max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
  x = __int_as_float(mu ^ ((mu >> 31) & 0x7FFFFFFF));
  y = __int_as_float(mv ^ ((mv >> 31) & 0x7FFFFFFF));
}
// Two wave maxima of non-negative floats. The row steps are float max with a DPP operand
// (every source lane exists for these controls, so no lane reads the bound value); the four
// row maxima are combined as integers, which order non-negative floats like the floats.
template <int CTRL>
__device__ __forceinline__ float fmax_dpp(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true)));
}
__device__ __forceinline__ int rows_max(float v) {
  const int b = __float_as_int(v);
  return max(max(__builtin_amdgcn_readlane(b, 0), __builtin_amdgcn_readlane(b, 16)),
             max(__builtin_amdgcn_readlane(b, 32), __builtin_amdgcn_readlane(b, 48)));
}
__device__ __forceinline__ float wave_max_nonneg(float x) {
  x = fmax_dpp<0xB1>(x);
  x = fmax_dpp<0x4E>(x);
  x = fmax_dpp<0x124>(x);
  x = fmax_dpp<0x128>(x);
  return __int_as_float(rows_max(x));
}
__device__ __forceinline__ void wave_max2_nonneg(float& x, float& y) {
  x = fmax_dpp<0xB1>(x);  y = fmax_dpp<0xB1>(y);    // lane ^ 1
  x = fmax_dpp<0x4E>(x);  y = fmax_dpp<0x4E>(y);    // lane ^ 2
  x = fmax_dpp<0x124>(x); y = fmax_dpp<0x124>(y);   // row_ror:4
  x = fmax_dpp<0x128>(x); y = fmax_dpp<0x128>(y);   // row_ror:8
  x = __int_as_float(rows_max(x));
  y = __int_as_float(rows_max(y));
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

// ---------------------------------------------------------------- code formats
// The six quantised products take one-byte codes in one of two formats, with the same
// byte layouts everywhere: INT8 (codes in [-127, 127], scale absmax/127, int32 products)
// or FP8 e4m3 (OCP float8 e4m3fn, largest finite 448, scale absmax/448, float32 products).
enum { FMT_INT8 = 0, FMT_FP8 = 1 };

template <int FMT> struct Codes;

template <> struct Codes<FMT_INT8> {
  using acc4 = i32x4;
  using acc16 = i32x16;
  static constexpr float kMax = 127.0f;
  static constexpr float kLog2Max = 6.988684686772166f;   // log2(127)
  __device__ static __forceinline__ acc4 mma16(i32x4 a, i32x4 b, acc4 c) { return mfma_i8_16x16x64(a, b, c); }
  __device__ static __forceinline__ acc4 mma16x2(i32x4 a0, i32x4 a1, i32x4 b0, i32x4 b1, acc4 c) {
    return mfma_i8_16x16x64(a1, b1, mfma_i8_16x16x64(a0, b0, c));
  }
  __device__ static __forceinline__ acc16 mma32x2(i32x4 a0, i32x4 a1, i32x4 b0, i32x4 b1, acc16 c) {
    return mfma_i8_32x32x32(a1, b1, mfma_i8_32x32x32(a0, b0, c));
  }
};

// FP8 products. Each lane's 16 operand bytes of an INT8 product (one contraction slot per
// byte, paired identically in A and B) feed the FP8 forms unchanged: two 8-byte halves make
// two K = 32 (16 x 16) or K = 16 (32 x 32) products, or the 16 bytes of two consecutive
// INT8 chunks concatenate into the 32 bytes of one K = 128 / K = 64 scaled product (scale
// exponents 127 = 2^0, both operands e4m3). A and B see the same slot assignment in every
// case, so the sum over the contraction is unchanged. The hardware keeps subnormal codes;
// its float32 accumulation is not exact (errors near 2^-16 of the sum of |terms| were
// measured), unlike the exact int32 sums of the INT8 form.
template <> struct Codes<FMT_FP8> {
  using acc4 = f32x4;
  using acc16 = f32x16;
  static constexpr float kMax = 448.0f;
  static constexpr float kLog2Max = 8.807354922057604f;   // log2(448)
  __device__ static __forceinline__ long half(i32x4 v, int h) {
    return __builtin_bit_cast(long, i32x2{v[2 * h], v[2 * h + 1]});
  }
  __device__ static __forceinline__ acc4 mma16(i32x4 a, i32x4 b, acc4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(half(a, 0), half(b, 0), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(half(a, 1), half(b, 1), c, 0, 0, 0);
  }
  __device__ static __forceinline__ acc4 mma16x2(i32x4 a0, i32x4 a1, i32x4 b0, i32x4 b1, acc4 c) {
    const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    const i32x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
  // operands already held as 32 bytes per lane
  __device__ static __forceinline__ acc4 mma16w(i32x8 a, i32x8 b, acc4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
  __device__ static __forceinline__ acc16 mma32x2(i32x4 a0, i32x4 a1, i32x4 b0, i32x4 b1, acc16 c) {
    const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    const i32x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// e4m3 codes of four values already multiplied by the inverse scale (|x| < 464), round to
// nearest even (v_cvt_pk_fp8_f32), byte i <- x_i.
__device__ __forceinline__ unsigned fp8_word(float x0, float x1, float x2, float x3) {
  const unsigned w = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, (int)w, true);
}

// Codes of four values under inverse scale inv, the rule of the prologue: fl(x * inv)
// rounded to the format (nearest even); byte i <- x_i.
__device__ __forceinline__ unsigned code_word(bool fp8, float x0, float x1, float x2, float x3, float inv) {
#pragma clang fp contract(off)
  if (fp8) return fp8_word(x0 * inv, x1 * inv, x2 * inv, x3 * inv);
  return pack4_lo_bytes(quant_word(x0, inv), quant_word(x1, inv), quant_word(x2, inv), quant_word(x3, inv));
}

// In-kernel tile codes (P, dS): INT8 rounds the exact product x * inv once; FP8 rounds
// fl(x * inv) to e4m3.
template <int FMT>
__device__ __forceinline__ unsigned tile_code_word(float x0, float x1, float x2, float x3, float inv) {
  if constexpr (FMT == FMT_FP8) {
#pragma clang fp contract(off)
    return fp8_word(x0 * inv, x1 * inv, x2 * inv, x3 * inv);
  } else {
    return pack4_lo_bytes(quant_word_fma(x0, inv), quant_word_fma(x1, inv), quant_word_fma(x2, inv),
                          quant_word_fma(x3, inv));
  }
}

// ---------------------------------------------------------------- LDS staging helpers
// XOR swizzles of the 16-byte chunks of LDS rows: 8 consecutive rows read at the same
// logical chunk land in 8 different bank groups.
template <int ROWB>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (ROWB >= 128) return chunk ^ (row & 7);
  else if constexpr (ROWB == 64) return chunk ^ ((row >> 1) & 3);
  else return chunk;
}

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Direct buffer -> LDS copy (buffer_load ... lds): lane l reads 16 bytes at byte offset
// voff + soff of the buffer [base, base + bytes) (reads past the end return zeros) and the
// hardware writes them to LDS at lds + 16*l (the 4-byte form: 4 bytes at lds + 4*l). voff is
// the per-lane offset; soff and lds must be the same in every lane of the wave. The
// bodies are compiled for the device only:
// this compiler's host pass cannot type-check the LDS-DMA builtin and, instead of reporting
// it, silently omits the host launch stubs of kernels that reach it.
// CPOL: the load's cache policy bits; kCpolNT marks data read once (a stream), which the
// caches then keep from displacing data that is read again.
constexpr int kCpolNT = 2;
template <int CPOL = 0>
__device__ __forceinline__ void buffer_to_lds16(const void* base, uint32_t bytes, int8_t* lds, uint32_t voff,
                                                uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                                                      0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, CPOL);
#endif
}

__device__ __forceinline__ void buffer_to_lds4(const void* base, uint32_t bytes, int8_t* lds, uint32_t voff,
                                               uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                                                      0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
#endif
}

}  // namespace sagebwd
