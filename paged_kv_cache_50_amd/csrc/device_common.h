// Device helpers shared by the gfx950 kernels: bfloat16 and binary16
// conversions, DPP lane reductions, 16-byte vector types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Reinterpret a 32-bit word as two bfloat16 lanes.  Takes the word by value:
// applying __builtin_bit_cast directly to a vector-element subscript (v[i])
// reads element 0 with this compiler, so callers must go through here.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t x) { return __builtin_bit_cast(bf16x2_t, x); }

// bfloat16 -> float32 is exact: the 16 stored bits are the high half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bfloat16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// ---- IEEE binary16 (cache dtype fp16) <-> float32.  Widening is exact;
// narrowing rounds to nearest even (the default rounding mode), NaN stays a
// NaN and magnitudes past 65504 round to infinity.
__device__ __forceinline__ f16x2_t as_f16x2(uint32_t x) { return __builtin_bit_cast(f16x2_t, x); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// The two 16-bit formats of q, out and 16-bit caches, as the matrix-core
// kernels use them: F16 = false is bfloat16, true is binary16.  Both have a
// 16x16x32 MFMA with fp32 accumulation on gfx950.
template <bool F16>
struct Fmt16;

template <>
struct Fmt16<false> {
  typedef __bf16 elem;
  typedef bf16x8_t x8;
  typedef bf16x4_t x4;
  static __device__ __forceinline__ x8 as_x8(u32x4 v) { return __builtin_bit_cast(x8, v); }
  static __device__ __forceinline__ f32x4 mfma(x8 a, x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // the 16 x 16 x 16 product (K = 16: 4 operand values per lane)
  static __device__ __forceinline__ f32x4 mfma16(x4 a, x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return bf16_lo(w); }
  static __device__ __forceinline__ float hi(uint32_t w) { return bf16_hi(w); }
  static __device__ __forceinline__ uint32_t rne(float f) { return f32_to_bf16_rne(f); }
};

template <>
struct Fmt16<true> {
  typedef _Float16 elem;
  typedef f16x8_t x8;
  typedef f16x4_t x4;
  static __device__ __forceinline__ x8 as_x8(u32x4 v) { return __builtin_bit_cast(x8, v); }
  static __device__ __forceinline__ f32x4 mfma(x8 a, x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(x4 a, x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return f16_lo(w); }
  static __device__ __forceinline__ float hi(uint32_t w) { return f16_hi(w); }
  static __device__ __forceinline__ uint32_t rne(float f) { return f32_to_f16_rne(f); }
};

template <bool F16>
__device__ __forceinline__ uint32_t pack16x2(float lo, float hi) {
  return Fmt16<F16>::rne(lo) | (Fmt16<F16>::rne(hi) << 16);
}

// ---- e4m3 (OCP "fn" variant) <-> float32, with the gfx950 converters, which
// round to nearest even and handle subnormals (out-of-range inputs must be
// clamped first: they would become NaN).

// Two e4m3 codes (bytes 0, 1 of w, or 2, 3 with HI) -> two bfloat16 (low
// half first) in one instruction: the gfx950 scaled converter with scale 1.
// Exact, since every e4m3 value is a bfloat16; on the device it gives the
// same bits as converting to float32 (v_cvt_pk_f32_fp8) and keeping the high
// halves, for all 2^16 code pairs, NaNs included.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Sixteen e4m3 codes -> two 16-byte chunks of eight bfloat16.
__device__ __forceinline__ void e4m3x16_to_bf16x16(const u32x4 w, u32x4& c0, u32x4& c1) {
  c0 = u32x4{e4m3x2_to_bf16x2<false>(w[0]), e4m3x2_to_bf16x2<true>(w[0]),
             e4m3x2_to_bf16x2<false>(w[1]), e4m3x2_to_bf16x2<true>(w[1])};
  c1 = u32x4{e4m3x2_to_bf16x2<false>(w[2]), e4m3x2_to_bf16x2<true>(w[2]),
             e4m3x2_to_bf16x2<false>(w[3]), e4m3x2_to_bf16x2<true>(w[3])};
}

// Saturate to the finite e4m3 range; NaN passes through.
__device__ __forceinline__ float e4m3_sat(float t) {
  return t > 448.f ? 448.f : (t < -448.f ? -448.f : t);
}

// Four floats (already saturated) -> four e4m3 codes, nearest even; NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float t0, float t1, float t2, float t3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(t0, t1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(t2, t3, w, true);
  uint32_t u = (uint32_t)w;
  if (t0 != t0) u = (u & 0xFFFFFF00u) | 0x7Fu;
  if (t1 != t1) u = (u & 0xFFFF00FFu) | 0x7F00u;
  if (t2 != t2) u = (u & 0xFF00FFFFu) | 0x7F0000u;
  if (t3 != t3) u = (u & 0x00FFFFFFu) | 0x7F000000u;
  return u;
}

// One DPP move of a float within a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// DPP controls (GCN/CDNA encoding).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;      // row_mirror: lane i <-> 15-i within 16

// Sum over aligned groups of N lanes (N = 4, 8, 16, 32, 64); every lane of the
// group receives the total.  Within a row of 16 the butterfly is done with DPP.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  x += dpp_f<kDppQuadXor1>(x);
  x += dpp_f<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp_f<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_f<kDppMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float acc_log2(float x) { return log2f(x); }

// Sequence length actually used: clamped into what the block table row and
// the launch (max_seq_len) can address, so bad metadata never leads to an
// out-of-bounds access.
__device__ __forceinline__ int clamp_seq_len(int L, int max_seq_len, int max_blocks, int bs) {
  int cap = min(max_seq_len, max_blocks * bs);
  return min(max(L, 0), cap);
}

// Wave-uniform read of read-only metadata through the scalar cache.  Going
// through the constant address space makes the compiler emit s_load (waited
// on with lgkmcnt) instead of a vector load; a vector load here would make
// the next wait for it also drain every K/V load still in flight.
typedef __attribute__((address_space(4))) const int32_t const_i32;
__device__ __forceinline__ int32_t load_uniform_i32(const int32_t* p, int64_t i) {
  return ((const_i32*)(p))[i];
}

// s_waitcnt immediate (gfx9 encoding) waiting until at most n vector memory
// operations of this wave are outstanding; lgkm and exp counts are ignored.
constexpr int vmcnt_enc(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

__device__ __forceinline__ int clamp_i(int x, int lo, int hi) { return min(max(x, lo), hi); }

}  // namespace pkv
