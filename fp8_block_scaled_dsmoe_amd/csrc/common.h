// Device-side building blocks shared by the dsmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsmoe {

constexpr int kWave = 64;
constexpr int kTile = 128;  // quantisation tile / promotion interval

// ---------------------------------------------------------------------------
// bf16 <-> f32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Two floats to two bf16 (a in the low half), round to nearest, ties to
// even, by gfx950's packed conversion (one VALU instruction; subnormals are
// kept, as the kernels run with float32 denormals on).
typedef float f32x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{a, b}, bf16x2_v));
}

// ---------------------------------------------------------------------------
// OCP E4M3FN encoder: round to nearest, ties to even, saturate at +-448,
// sign of zero kept.  Integer-only apart from the exact scaling of the
// subnormal range, so it is bit-exact by construction:
//   |v| >= 448           -> 0x7E
//   |v| <  2^-6          -> n = rne(|v| * 2^9), code n (n = 8 is 0x08)
//   otherwise            -> keep 3 mantissa bits, round on the 20 dropped
//                           bits; a carry out of the mantissa increments the
//                           exponent field through the plain addition.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t mag = bits & 0x7FFFFFFFu;
  if (mag >= 0x43E00000u) return sign | 0x7Eu;            // >= 448 (and Inf/NaN)
  if (mag < 0x3C800000u) {                                // < 2^-6
    const float t = __uint_as_float(mag) * 512.0f;        // exact power-of-2 scaling
    return sign | static_cast<uint32_t>(__builtin_rintf(t));
  }
  const uint32_t e = (mag >> 23) - 127u + 7u;             // 1..15
  const uint32_t m = mag & 0x7FFFFFu;
  uint32_t keep = m >> 20;
  const uint32_t rest = m & 0xFFFFFu;
  keep += (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
  return sign | ((e << 3) + keep);
}

// E4M3 codes of two values (low byte: a, next byte: b) with gfx950's packed
// conversion, which rounds to nearest even like e4m3_encode and gives the same
// code for every float with |v| <= 464; past that it gives NaN where
// e4m3_encode saturates, so the values are clamped to +-448 first (the two
// then agree on every input but NaN).
__device__ __forceinline__ uint32_t e4m3_encode2(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

// E4M3 codes (low byte, next byte) of the IEEE quotients a / sa and b / sb
// from reciprocals ra = fl(1 / sa) and rb = fl(1 / sb) (IEEE divisions):
// q = fl(a * ra) is within 2^-23 (relative) of a / sa, so the quotient lies
// strictly between fl(q * (1 - 2^-22)) and fl(q * (1 + 2^-22)) (for q a
// normal float; a smaller q and its quotient both encode to a signed zero).
// The encoder is monotone, so where both ends give one code it is the
// quotient's; the function returns the lower end's codes and sets `unsure`
// where the ends differ (a few ulps from a rounding point, or across zero)
// or a reciprocal overflowed: there the caller encodes the quotient itself.
__device__ __forceinline__ uint32_t e4m3_encode2_recip(float a, float b, float ra, float rb, bool& unsure) {
  constexpr float kBelow = 1.0f - 0x1p-22f, kAbove = 1.0f + 0x1p-22f;
  const float qa = a * ra, qb = b * rb;
  const uint32_t lo = e4m3_encode2(qa * kBelow, qb * kBelow);
  const uint32_t hi = e4m3_encode2(qa * kAbove, qb * kAbove);
  unsure = unsure || lo != hi || !(ra < 0x1p127f) || !(rb < 0x1p127f);
  return lo;
}

// ---------------------------------------------------------------------------
// Wave helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max_width(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, width));
  return v;
}

// Maximum of non-negative values (or NaN) over each aligned group of 16
// lanes (one DPP row), left in every lane of the group: swap neighbours, swap
// pairs (quad permutations), then mirror within each 8-lane half and within
// the row.  For non-negative floats the order of the bit patterns is the
// order of the values, so an unsigned max does it without canonicalising
// moves; there is no LDS round trip (a cross-lane shuffle goes through the
// LDS crossbar).
__device__ __forceinline__ float row16_max_nonneg(float v) {
  uint32_t b = __float_as_uint(v);
  b = max(b, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b), 0xB1, 0xF, 0xF, false)));
  b = max(b, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b), 0x4E, 0xF, 0xF, false)));
  b = max(b, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b), 0x141, 0xF, 0xF, false)));
  b = max(b, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b), 0x140, 0xF, 0xF, false)));
  return __uint_as_float(b);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace dsmoe
