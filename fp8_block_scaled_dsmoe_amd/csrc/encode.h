// Loads and E4M3 codes shared by the quantisers (quant.hip, granularity.hip).
//
// Every quantiser computes q = E4M3(fl32(v / s)) with fl32 the IEEE float32
// division (the build asks for correctly rounded division), s = fl32(amax /
// 448).  A multiply by fl32(1 / s), checked against the division's rounding
// interval and dividing only where that interval straddles an E4M3 rounding
// point, gives the same codes (checked bit for bit on the GPU) but was no
// faster on MI355X: 18.6 against 19.0 us for 4096 x 7168 bf16 in 1x128 tiles,
// and slower per row (25.6 against 21.9 us), so the kernels divide.
#pragma once

#include "common.h"

namespace dsmoe {

template <bool kF32>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float (&v)[8]) {
  if constexpr (kF32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    const float4 a = p[0];
    const float4 b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

__device__ __forceinline__ float scale_from_amax(float amax) {
  return amax == 0.0f ? 1.0f : amax / 448.0f;
}

// Codes of v / s for 8 values, two per byte pair, as a little-endian uint2.
// |v / s| <= 448 (1 + 2^-23) for the scales used here, well inside the range
// where the packed hardware conversion gives e4m3_encode's code.
__device__ __forceinline__ uint2 encode8(const float (&v)[8], float s) {
  const uint32_t c01 = e4m3_encode2(v[0] / s, v[1] / s), c23 = e4m3_encode2(v[2] / s, v[3] / s);
  const uint32_t c45 = e4m3_encode2(v[4] / s, v[5] / s), c67 = e4m3_encode2(v[6] / s, v[7] / s);
  return make_uint2(c01 | (c23 << 16), c45 | (c67 << 16));
}

}  // namespace dsmoe
