// Device-side types and conversions shared by the HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Storage-type tags (what one element of a pool / tensor is).
struct F16 {
  static constexpr int kBytes = 2;
};
struct BF16 {
  static constexpr int kBytes = 2;
};
struct FP8 {
  static constexpr int kBytes = 1;
};

// ---- scalar conversions --------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// OCP E4M3 (e4m3fn) encode of an fp32 value: round to nearest, ties to even,
// saturate to +-448 (also for +-inf), NaN -> 0x7f with the sign kept.
// Normal range [2^-6, 448): the 23-bit fp32 mantissa is rounded to 3 bits;
// a carry out of the mantissa bumps the exponent, which is the right
// result. Below 2^-6 the value is a multiple of 2^-9: scale by 2^9 (exact)
// and round to an integer 0..8 (8 is the smallest normal, code 0x08).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;  // >= 448
  if (a < 0x3c800000u) {                      // < 2^-6
    const float f = __uint_as_float(a) * 512.0f;
    return sign | static_cast<uint32_t>(__builtin_rintf(f));
  }
  const uint32_t e = (a >> 23) - 120u;  // biased e4m3 exponent, 1..15
  uint32_t code = (e << 3) | ((a >> 20) & 7u);
  const uint32_t rem = a & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) ++code;
  return sign | code;
}

// Four E4M3 bytes packed in a dword -> bf16 pairs, by CDNA4's packed
// conversion (v_cvt_scalef32_pk_bf16_fp8, scale 1: exact, since every E4M3
// value is a bf16 value). word_sel picks bytes 0-1 or 2-3. Returns two
// dwords, each holding two bf16 (byte 0 in the low half of .x).
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Four E4M3 bytes -> four f16 values (v_cvt_scalef32_pk_f16_fp8, exact: f16
// holds every E4M3 value).
__device__ __forceinline__ u32x2 e4m3x4_to_f16x4(uint32_t w) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const h2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Four E4M3 bytes -> four fp32 values (v_cvt_pk_f32_fp8, exact).
__device__ __forceinline__ f32x4 e4m3x4_to_f32x4(uint32_t w) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  return f32x4{lo.x, lo.y, hi.x, hi.y};
}

// ---- wave-level reductions (wave64) ----------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ---- 16x16x32 MFMA on 8-element operands held as 4 dwords -----------------

template <typename T>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c);

template <>
__device__ __forceinline__ f32x4 mfma_16x16x32<BF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mfma_16x16x32<F16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                 0, 0);
}

// Output element conversion by runtime dtype code (0 f16, 1 bf16, 2 f32).
// Max / sum over the lane pairs (l, l ^ 16) and (l, l ^ 32) on the VALU.
// v_permlane16_swap / v_permlane32_swap exchange rows of 16 (32) lanes
// between two registers; given x in both, every lane ends with its own x
// in one and its partner's in the other, the order depending on the lane
// (checked on gfx950), so the max or sum of the two is the pair's, equal on
// both lanes (a + b = b + a). Same results as ds_swizzle / ds_bpermute,
// without their LDS round trips. Written as inline asm (an exchange of two
// registers, no memory access): the compiler's builtin folds max(r0, r1) of
// its two results to r0, which the hardware does not return. The s_nop
// gives the two wait states the compiler puts between a VALU write of an
// operand and these instructions.
__device__ __forceinline__ void pair_swap16(float x, float& a, float& b) {
  a = x;
  b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void pair_swap32(float x, float& a, float& b) {
  a = x;
  b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float pair16_max(float x) {
  float a, b;
  pair_swap16(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float pair32_max(float x) {
  float a, b;
  pair_swap32(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float pair16_sum(float x) {
  float a, b;
  pair_swap16(x, a, b);
  return a + b;
}
__device__ __forceinline__ float pair32_sum(float x) {
  float a, b;
  pair_swap32(x, a, b);
  return a + b;
}

__device__ __forceinline__ void store_out(void* out, int64_t idx, int dtype, float v) {
  if (dtype == 2) {
    static_cast<float*>(out)[idx] = v;
  } else if (dtype == 1) {
    static_cast<uint16_t*>(out)[idx] = static_cast<uint16_t>(f32_to_bf16_bits(v));
  } else {
    static_cast<uint16_t*>(out)[idx] = static_cast<uint16_t>(f32_to_f16_bits(v));
  }
}

// Eight consecutive output elements (16-byte aligned for 16-bit outputs,
// 32-byte aligned for fp32) by runtime dtype code.
__device__ __forceinline__ void store_out8(void* out, int64_t idx, int dtype, const float (&v)[8]) {
  if (dtype == 2) {
    float* o = static_cast<float*>(out) + idx;
    *reinterpret_cast<f32x4*>(o) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(o + 4) = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = dtype == 1 ? f32_to_bf16_bits(v[2 * i]) : f32_to_f16_bits(v[2 * i]);
      const uint32_t hi = dtype == 1 ? f32_to_bf16_bits(v[2 * i + 1]) : f32_to_f16_bits(v[2 * i + 1]);
      w[i] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + idx) = w;
  }
}

}  // namespace pa
