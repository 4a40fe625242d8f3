// Coarser FP8 scaling granularities, for comparison with the fine-grained
// recipe: one E4M3 scale per tensor, or one per row over the whole row (per
// token for an activation, per output channel for a weight stored [N][K]).
// Source: infra answer (51itzy.com "DeepSeek-V3 ... infra"), FP8 paragraph:
// a single outlier under per-tensor scaling stretches the scale of everything
// else, the recipe answers with 1x128 / 128x128 tiles, and per-token x
// per-channel scaling is left undiscussed; V3 notes §6.1 for the recipe.
//
// Every scale follows the recipe's rule, s = fl32(amax / 448) (IEEE division,
// 1 for amax = 0), q = E4M3(fl32(x / s)), so the three granularities differ
// only in the set of values an amax is taken over.  The GEMM then runs on the
// block-scaled kernel unchanged: a per-tensor or per-row scale is broadcast
// into the 1x128 / 128x128 layouts, and a per-output-channel weight scale,
// which no 128x128 layout can hold, is applied to the finished output.
#include "common.h"
#include "encode.h"
#include "kernels.h"

namespace dsmoe {
namespace {


__device__ __forceinline__ float amax8(const float (&v)[8], float m) {
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
  return m;
}

// Maximum of non-negative values over the 256 threads of a block, left in
// every thread.
__device__ __forceinline__ float block256_max(float m, float* red) {
  m = wave_max_width(m, kWave);
  if (lane_id() == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

constexpr int kRowVecs = 16;  // 8-element vectors per thread: rows of up to 256*16*8 = 32768

// 8 input elements as loaded: one 16-byte word of bf16, or two of float32.
template <bool kF32>
struct Raw8 {
  uint4 u;
};
template <>
struct Raw8<true> {
  float4 a, b;
};

template <bool kF32>
__device__ __forceinline__ Raw8<kF32> load_raw8(const void* base, int64_t idx) {
  Raw8<kF32> r;
  if constexpr (kF32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    r.a = p[0];
    r.b = p[1];
  } else {
    r.u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
  }
  return r;
}

template <bool kF32>
__device__ __forceinline__ void unpack8(const Raw8<kF32>& r, float (&v)[8]) {
  if constexpr (kF32) {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
  } else {
    const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

// One 256-thread block per row.  Thread t holds vectors t, t+256, ... of the
// row in registers as loaded (bf16 stays packed: 4 VGPRs per 8 elements), so
// the row is read from HBM once: amax over the block, then the codes from the
// held values.
template <bool kF32>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ x, int64_t cols,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
  __shared__ float red[4];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * cols;
  const int nvec = static_cast<int>(cols >> 3);
  Raw8<kF32> raw[kRowVecs];
#pragma unroll
  for (int i = 0; i < kRowVecs; ++i) {
    const int j = threadIdx.x + 256 * i;
    if (j < nvec) raw[i] = load_raw8<kF32>(x, base + 8 * j);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kRowVecs; ++i) {
    const int j = threadIdx.x + 256 * i;
    if (j < nvec) {
      float v[8];
      unpack8<kF32>(raw[i], v);
      amax = amax8(v, amax);
    }
  }
  // opaque to the compiler: the codes unpack the held words again instead of
  // keeping the first unpacking's floats live (twice the registers) across
  // the block reduction
  if constexpr (!kF32) {
#pragma unroll
    for (int i = 0; i < kRowVecs; ++i)
      asm volatile("" : "+v"(raw[i].u.x), "+v"(raw[i].u.y), "+v"(raw[i].u.z), "+v"(raw[i].u.w));
  }
  const float s = scale_from_amax(block256_max(amax, red));
#pragma unroll
  for (int i = 0; i < kRowVecs; ++i) {
    const int j = threadIdx.x + 256 * i;
    if (j < nvec) {
      float v[8];
      unpack8<kF32>(raw[i], v);
      *reinterpret_cast<uint2*>(q + base + 8 * j) = encode8(v, s);
    }
  }
  if (threadIdx.x == 0) scale[blockIdx.x] = s;
}

// Partial maxima of the per-tensor amax pass: kAmaxSlots slots, each on its
// own 128-byte line.  Blocks merge into slot (block mod kAmaxSlots), so no
// line takes more than gridDim / kAmaxSlots atomics: device-scope atomics on
// one address serialise (2048 of them on one slot cost about 19 us on a
// 4096 x 7168 tensor, against 12 us for the whole pass with 64 slots).
constexpr int kAmaxSlots = 64;
constexpr int kSlotStride = 32;  // floats
static_assert(kAmaxSlots == kWave, "one slot per lane of the reducing wave");

// The amax slots of one per-tensor quantisation to 0 (when given) and the
// offsets {0, m} of a one-group GEMM (when given).
__global__ void prep_kernel(float* slots, int32_t* offsets, int32_t m) {
  if (slots && threadIdx.x < kAmaxSlots) slots[kSlotStride * threadIdx.x] = 0.0f;
  if (offsets && threadIdx.x == 0) {
    offsets[0] = 0;
    offsets[1] = m;
  }
}

constexpr int kStreamBlocks = 2048;  // 8 blocks of 256 threads per CU
constexpr int kStreamUnroll = 8;     // 16-byte loads a thread of the amax pass issues before using any

// amax over the whole tensor: grid-stride over 8-element vectors with up to
// kStreamUnroll loads in flight per thread, one maximum per block, merged
// with an unsigned atomic max on the bit patterns (the order of non-negative
// floats): exact and independent of order.
template <bool kF32>
__global__ __launch_bounds__(256) void tensor_amax_kernel(const void* __restrict__ x, int64_t nvec,
                                                          float* __restrict__ slots) {
  __shared__ float red[4];
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  float m = 0.0f;
  for (int64_t j0 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; j0 < nvec;
       j0 += kStreamUnroll * stride) {
    float v[kStreamUnroll][8];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u)
      if (j0 + u * stride < nvec) load8<kF32>(x, 8 * (j0 + u * stride), v[u]);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u)
      if (j0 + u * stride < nvec) m = amax8(v[u], m);
  }
  m = block256_max(m, red);
  if (threadIdx.x == 0)
    atomicMax(reinterpret_cast<unsigned int*>(slots + kSlotStride * (blockIdx.x % kAmaxSlots)),
              __float_as_uint(m));
}

// Codes of the whole tensor under the one scale.  Each wave reduces the
// slots itself (lane l reads slot l); block 0 publishes the total in slot 0
// (a concurrent reader of slot 0 sees the partial or the total, and both give
// the same maximum) and the scale.
template <bool kF32>
__global__ __launch_bounds__(256) void tensor_encode_kernel(const void* __restrict__ x, int64_t nvec,
                                                            float* __restrict__ slots,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  const float amax = wave_max_width(slots[kSlotStride * lane_id()], kWave);
  const float s = scale_from_amax(amax);
  // four loads ahead, then one at a time: with eight ahead, as in the amax
  // pass, this read-and-write pass took 24.6 instead of 20.2 us on MI355X
  // (4096 x 7168 bf16)
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  for (; j + 3 * stride < nvec; j += 4 * stride) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8<kF32>(x, 8 * (j + u * stride), v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<uint2*>(q + 8 * (j + u * stride)) = encode8(v[u], s);
  }
  for (; j < nvec; j += stride) {
    float v[8];
    load8<kF32>(x, 8 * j, v);
    *reinterpret_cast<uint2*>(q + 8 * j) = encode8(v, s);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    slots[0] = amax;
    *scale = s;
  }
}

// dst[r][t] = src[r * src_stride] (t < tiles), or 1 when src is null.
__global__ __launch_bounds__(256) void broadcast_scale_kernel(float* __restrict__ dst, int64_t rows,
                                                              int64_t tiles,
                                                              const float* __restrict__ src,
                                                              int64_t src_stride) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * tiles) return;
  const int64_t r = i / tiles;
  dst[i] = src ? src[r * src_stride] : 1.0f;
}

// c[m][n] *= col[n] for float32 c [M][N], four columns per thread.
__global__ __launch_bounds__(256) void scale_cols_kernel(float* __restrict__ c, int64_t m, int64_t n,
                                                         const float* __restrict__ col) {
  const int64_t n4 = n >> 2;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < m * n4; i += stride) {
    const int64_t j = i % n4;
    float4 v = reinterpret_cast<float4*>(c)[i];
    const float4 s = reinterpret_cast<const float4*>(col)[j];
    v.x *= s.x; v.y *= s.y; v.z *= s.z; v.w *= s.w;
    reinterpret_cast<float4*>(c)[i] = v;
  }
}

unsigned stream_blocks(int64_t nvec) {
  const int64_t need = (nvec + 255) / 256;
  return static_cast<unsigned>(need < 1 ? 1 : (need < kStreamBlocks ? need : kStreamBlocks));
}

}  // namespace

int64_t quant_rows_max_cols() { return 256LL * kRowVecs * 8; }

hipError_t launch_quant_rows(const void* x, bool x_f32, int64_t rows, int64_t cols, uint8_t* q,
                             float* scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(rows));
  if (x_f32)
    quant_rows_kernel<true><<<grid, 256, 0, s>>>(x, cols, q, scale);
  else
    quant_rows_kernel<false><<<grid, 256, 0, s>>>(x, cols, q, scale);
  return hipGetLastError();
}

int64_t quant_tensor_scratch_floats() { return static_cast<int64_t>(kAmaxSlots) * kSlotStride; }

hipError_t launch_quant_tensor(const void* x, bool x_f32, int64_t n, uint8_t* q, float* scale,
                               float* amax_scratch, hipStream_t s) {
  const int64_t nvec = n >> 3;
  prep_kernel<<<1, kAmaxSlots, 0, s>>>(amax_scratch, nullptr, 0);
  const dim3 grid(stream_blocks(nvec));
  if (x_f32) {
    tensor_amax_kernel<true><<<grid, 256, 0, s>>>(x, nvec, amax_scratch);
    tensor_encode_kernel<true><<<grid, 256, 0, s>>>(x, nvec, amax_scratch, q, scale);
  } else {
    tensor_amax_kernel<false><<<grid, 256, 0, s>>>(x, nvec, amax_scratch);
    tensor_encode_kernel<false><<<grid, 256, 0, s>>>(x, nvec, amax_scratch, q, scale);
  }
  return hipGetLastError();
}

hipError_t launch_prep_offsets(int32_t* offsets, int32_t m, hipStream_t s) {
  prep_kernel<<<1, kAmaxSlots, 0, s>>>(nullptr, offsets, m);
  return hipGetLastError();
}

hipError_t launch_broadcast_scale(float* dst, int64_t rows, int64_t tiles, const float* src,
                                  int64_t src_stride, hipStream_t s) {
  const int64_t n = rows * tiles;
  if (n == 0) return hipSuccess;
  broadcast_scale_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(dst, rows, tiles, src,
                                                                               src_stride);
  return hipGetLastError();
}

hipError_t launch_scale_cols(float* c, int64_t m, int64_t n, const float* col, hipStream_t s) {
  if (m == 0) return hipSuccess;
  scale_cols_kernel<<<stream_blocks(m * n / 4), 256, 0, s>>>(c, m, n, col);
  return hipGetLastError();
}

}  // namespace dsmoe
