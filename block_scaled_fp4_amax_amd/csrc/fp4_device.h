// fp4_device.h -- device helpers for the gfx950 FP4 kernels: packed-type
// aliases, E2M1 / E4M3 / E8M0 conversions on the CDNA4 conversion units,
// Philox4x32-10, the 16-point Hadamard butterfly and cross-lane reductions.
//
// Format definitions: Ultralytics glossary page "FP4", section "Como funciona
// FP4" (E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; MXFP4 = 32 values under
// an E8M0 power-of-two scale; NVFP4 = 16 values under an E4M3 scale and an
// FP32 tensor scale).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4dev {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kFltMin = 1.17549435e-38f;   // smallest normal fp32
constexpr float kE4M3Max = 448.0f;           // largest finite OCP E4M3 ("fn")

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Power-of-two scale operand of the gfx950 scaled conversions: the hardware
// reads only the exponent field, so the E8M0 byte goes straight into it
// (byte 0 reads as 2^-127).
__device__ __forceinline__ float e8m0_scale_operand(uint32_t byte) {
  return __builtin_bit_cast(float, byte << 23);
}

// Round two fp32 values to E2M1 (nearest, ties to even, saturating at 6, sign
// kept) and place the pair in byte `SEL` of `old`: low nibble = a, high = b.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}
// Same for a bf16 pair divided by the power of two whose exponent is in `scale`.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2_bf16(uint32_t old, uint32_t bf16pair, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(bf16x2, bf16pair), scale, SEL);
}
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2_scaled(uint32_t old, float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}

// Decode the two codes in byte `SEL` of w to fp32 (exact), times the power of
// two in `scale`.
template <int SEL>
__device__ __forceinline__ f32x2 e2m1_unpack2(uint32_t w, float scale = 1.0f) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, SEL);
}
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_unpack2_bf16(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL));
}

// E4M3 ("fn") nearest-even encoding of s in [0, 448] (the caller clamps: the
// converter turns values above 464 into NaN) and its exact decoding.
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(s, 0.0f, 0u, false) & 0xffu;
}
__device__ __forceinline__ float e4m3_decode(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8(code, 0);
}

// MXFP4 block exponent: e = floor(log2(amax)) - 2 (block max lands in [4, 8),
// values above 6 saturate), clamped to [-127, 127]; amax = 0 or denormal
// gives -127. Returns the E8M0 byte e + 127.
__device__ __forceinline__ uint32_t e8m0_from_amax(float amax) {
  uint32_t ef = __builtin_bit_cast(uint32_t, amax) >> 23;  // amax >= 0
  int e = (ef == 0) ? -127 : (int)ef - 129;
  e = e < -127 ? -127 : e;
  return (uint32_t)(e + 127);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// two-multiplier S-box over a 128-bit counter, key bumped by the Weyl
// constants between rounds.
// Full 32 x 32 -> 64-bit product in one v_mad_u64_u32 (the compiler would
// otherwise often split it into separate low and high multiplies).
__device__ __forceinline__ uint64_t mul_wide_u32(uint32_t a, uint32_t b) {
  uint64_t p, carry;
  asm("v_mad_u64_u32 %0, %1, %2, %3, 0" : "=v"(p), "=s"(carry) : "v"(a), "v"(b));
  (void)carry;
  return p;
}

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; r++) {
    const uint64_t p0 = mul_wide_u32(0xD2511F53u, c.x), p1 = mul_wide_u32(0xCD9E8D57u, c.z);
    uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    c = u32x4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Stochastic rounding of q to E2M1 with the 16-bit random integer r: with
// a = |q| < 6 between grid neighbours lo < hi, round up iff
// r < (a - lo) / (hi - lo) * 2^16; a >= 6 saturates. Returns the 4-bit code.
// The fraction is read off the fp32 encoding of a: in [1, 6) the grid has two
// points per binade, so (a - lo) / (hi - lo) * 2^16 is the mantissa's low 22
// bits / 2^6; in [0.5, 1) it is the mantissa / 2^7; below 0.5 it is a * 2^17,
// exact in fp32. Each test is the exact comparison of the definition.
// For a >= 1 the encoding's bits 22 and up are 2 * (binade + 127) plus the
// half-binade bit, which is the round-down code + 252; adding
// 2^22 - 1 - r * 2^6 carries into bit 22 exactly when the low 22 bits exceed
// r * 2^6, so the sum's bits 22 and up give the rounded code + 252. From
// a = 6 on that code is 7 or more (at most 260), so a min saturates it.
__device__ __forceinline__ uint32_t e2m1_sr(float q, uint32_t r16) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, q);
  const uint32_t sign = (bits >> 28) & 8u;
  const uint32_t ab = bits & 0x7fffffffu;
  const uint32_t mant = ab & 0x7fffffu;
  const uint32_t c_hi = ((ab + (0x3fffffu - (r16 << 6))) >> 22) - 252u;
  const uint32_t c_mid = 1u + ((r16 << 7) < mant);
  const uint32_t c_lo = (float)r16 < __builtin_fabsf(q) * 131072.0f;
  const uint32_t m = ab >= 0x3f800000u ? (c_hi < 7u ? c_hi : 7u) : (ab >= 0x3f000000u ? c_mid : c_lo);
  return sign | m;
}

// 16-point randomized Hadamard transform of v (in place): negate where the
// sign mask has a bit, Walsh-Hadamard butterflies in stages 1, 2, 4, 8, then
// multiply by 1/4.
__device__ __forceinline__ void rht16(float v[16], uint32_t signs) {
#pragma unroll
  for (int i = 0; i < 16; i++) v[i] = ((signs >> i) & 1u) ? -v[i] : v[i];
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; j++) {
      if (j & h) continue;
      float a = v[j], b = v[j + h];
      v[j] = a + b;
      v[j + h] = a - b;
    }
  }
#pragma unroll
  for (int i = 0; i < 16; i++) v[i] = v[i] * 0.25f;
}

__device__ __forceinline__ float max_abs16(const float v[16]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i++) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
  return m;
}

// v of lane (lane ^ MASK). Masks 1 and 2 are a DPP quad permutation of the
// source operand, 4, 8 and 16 a ds_swizzle in bit mode (xor within each half
// of the wave), both without the per-lane address arithmetic of a general
// cross-lane read; 32 falls back to that. Every lane of an exchanging group
// must be active.
template <int MASK>
__device__ __forceinline__ float xor_shfl(float v) {
  const int x = __builtin_bit_cast(int, v);
  int r;
  if constexpr (MASK == 1) {
    r = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad_perm [1, 0, 3, 2]
  } else if constexpr (MASK == 2) {
    r = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad_perm [2, 3, 0, 1]
  } else if constexpr (MASK == 4 || MASK == 8 || MASK == 16) {
    r = __builtin_amdgcn_ds_swizzle(x, (MASK << 10) | 0x1F);  // and 0x1F, or 0, xor MASK
  } else {
    r = __shfl_xor(x, MASK, 64);
  }
  return __builtin_bit_cast(float, r);
}

}  // namespace fp4dev
