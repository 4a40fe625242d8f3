// Decode-serving variant of the layer: redundant copies ("slots") of hot
// experts and the shared expert run as a 9th routed expert.
// Source: V3 notes (xutianle.me "DeepSeek-V3 技术报告" walk-through) §8, the
// deployment section: in decode the shared expert is a routed expert every
// token takes; hot experts get redundant copies, re-chosen periodically from
// loads observed online.  Infra answer (51itzy.com), inference paragraph:
// decode over 256 experts plus 64 copies of hot ones.
//
// Readings (the pages fix neither rule):
// - plan: extra slots go one at a time to the expert with the largest load
//   per slot c_e / n_e (exact integer comparison, lowest index on ties);
//   an expert's slots are consecutive;
// - split: the rows of expert e (tokens ascending) are cut into n_e
//   contiguous chunks, chunk j starting at offsets[e] + floor(j c_e / n_e),
//   so the permutation is untouched and only the group offsets change.
#include "common.h"
#include "kernels.h"

namespace dsmoe {
namespace {

constexpr int kPlanMaxExperts = 1024;  // the ABI's expert limit
constexpr int kPlanPerLane = kPlanMaxExperts / kWave;

// a = (ca, na, ea) carries more load per slot than b, or the same with a lower
// index; lanes with no expert carry e = INT32_MAX, c = 0, n = 1 and lose
// against every real expert of equal load.
__device__ __forceinline__ bool plan_better(int32_t ca, int32_t na, int32_t ea, int32_t cb,
                                            int32_t nb, int32_t eb) {
  const int64_t l = static_cast<int64_t>(ca) * nb, r = static_cast<int64_t>(cb) * na;
  return l > r || (l == r && ea < eb);
}

// One wave.  Lane l holds experts l, l+64, ..., so every greedy step is a scan
// of the lane's own experts and a wave argmax, without LDS or barriers.
__global__ __launch_bounds__(kWave) void plan_replicas_kernel(const int32_t* __restrict__ counts,
                                                              int32_t E, int32_t n_extra,
                                                              int32_t* __restrict__ slot_first,
                                                              int32_t* __restrict__ slot_expert) {
  const int lane = lane_id();
  int32_t c[kPlanPerLane], n[kPlanPerLane];
#pragma unroll
  for (int i = 0; i < kPlanPerLane; ++i) {
    const int e = lane + kWave * i;
    c[i] = e < E ? counts[e] : 0;
    n[i] = 1;
  }
  for (int32_t r = 0; r < n_extra; ++r) {
    int32_t bc = 0, bn = 1, be = INT32_MAX;
#pragma unroll
    for (int i = 0; i < kPlanPerLane; ++i) {
      const int e = lane + kWave * i;
      if (e < E && plan_better(c[i], n[i], e, bc, bn, be)) {
        bc = c[i];
        bn = n[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      const int32_t oc = __shfl_xor(bc, o), on = __shfl_xor(bn, o), oe = __shfl_xor(be, o);
      if (plan_better(oc, on, oe, bc, bn, be)) {
        bc = oc;
        bn = on;
        be = oe;
      }
    }
    // every lane now holds the winner; its owner adds the slot
#pragma unroll
    for (int i = 0; i < kPlanPerLane; ++i)
      if (lane + kWave * i == be) ++n[i];
  }
  // slot_first: exclusive prefix sum of n over experts 0..E-1, 64 at a time
  int32_t carry = 0;
#pragma unroll
  for (int i = 0; i < kPlanPerLane; ++i) {
    const int e = lane + kWave * i;
    int32_t v = e < E ? n[i] : 0;
    int32_t incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int32_t t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    const int32_t first = carry + incl - v;
    if (e < E) {
      slot_first[e] = first;
      for (int32_t j = 0; j < v; ++j) slot_expert[first + j] = e;
    }
    carry += __shfl(incl, kWave - 1);
  }
  if (lane == 0) slot_first[E] = carry;
}

// phys[s] for slots s < S from the experts' offsets; phys[S] = offsets[E];
// phys[S + 1] = offsets[E] + extra_rows when extra_rows >= 0 (the shared
// expert's rows after the routed ones).  A slot whose plan entries are not
// those of a plan (expert out of range, no slots, position outside the
// expert's slots) gets offsets[E]: the results are then wrong, but every
// offset stays inside the rows, so the GEMMs stay in bounds.
__global__ __launch_bounds__(256) void slot_offsets_kernel(const int32_t* __restrict__ offsets, int32_t E,
                                                           const int32_t* __restrict__ slot_first,
                                                           const int32_t* __restrict__ slot_expert,
                                                           int32_t S, int64_t extra_rows,
                                                           int32_t* __restrict__ phys) {
  const int32_t s = static_cast<int32_t>(blockIdx.x) * 256 + threadIdx.x;
  if (s < S) {
    const int32_t e = slot_expert[s];
    int32_t v = offsets[E];
    if (e >= 0 && e < E) {
      const int32_t j = s - slot_first[e];
      const int32_t ne = slot_first[e + 1] - slot_first[e];
      const int32_t cnt = offsets[e + 1] - offsets[e];
      if (ne >= 1 && j >= 0 && j < ne && cnt >= 0)
        v = offsets[e] + static_cast<int32_t>(static_cast<int64_t>(j) * cnt / ne);
    }
    phys[s] = v;
  } else if (s == S) {
    phys[S] = offsets[E];
    if (extra_rows >= 0) phys[S + 1] = offsets[E] + static_cast<int32_t>(extra_rows);
  }
}

// Slot s receives matrix slot_expert[s] and its block scales: a gather copy
// in 16-byte words, blockIdx.y = slot.  A slot naming no expert in [0, E) is
// left as it was.
__global__ __launch_bounds__(256) void place_slots_kernel(const uint4* __restrict__ src, int64_t mat_words,
                                                          const float* __restrict__ src_scale,
                                                          int64_t mat_scales,
                                                          const int32_t* __restrict__ slot_expert,
                                                          int32_t E, uint4* __restrict__ dst,
                                                          float* __restrict__ dst_scale) {
  const int32_t s = blockIdx.y;
  const int64_t e = slot_expert[s];
  if (e < 0 || e >= E) return;
  const uint4* from = src + e * mat_words;
  uint4* to = dst + static_cast<int64_t>(s) * mat_words;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  for (; i + 3 * stride < mat_words; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = from[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) to[i + u * stride] = v[u];
  }
  for (; i < mat_words; i += stride) to[i] = from[i];
  for (int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; j < mat_scales; j += stride)
    dst_scale[static_cast<int64_t>(s) * mat_scales + j] = src_scale[e * mat_scales + j];
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* __restrict__ dst, int64_t n, float v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) dst[i] = v;
}

}  // namespace

hipError_t launch_plan_replicas(const int32_t* counts, int32_t E, int32_t n_extra, int32_t* slot_first,
                                int32_t* slot_expert, hipStream_t s) {
  plan_replicas_kernel<<<1, kWave, 0, s>>>(counts, E, n_extra, slot_first, slot_expert);
  return hipGetLastError();
}

hipError_t launch_slot_offsets(const int32_t* offsets, int32_t E, const int32_t* slot_first,
                               const int32_t* slot_expert, int32_t S, int64_t extra_rows, int32_t* phys,
                               hipStream_t s) {
  slot_offsets_kernel<<<(S + 1 + 255) / 256, 256, 0, s>>>(offsets, E, slot_first, slot_expert, S,
                                                          extra_rows, phys);
  return hipGetLastError();
}

hipError_t launch_place_slots(const uint8_t* w, const float* w_scale, int32_t E, int64_t n, int64_t k,
                              const int32_t* slot_expert, int32_t S, uint8_t* w_slots, float* s_slots,
                              hipStream_t s) {
  if (S == 0) return hipSuccess;
  const int64_t words = n * k / 16;
  const int64_t scales = (n / kTile) * (k / kTile);
  int64_t bx = (words + 4 * 256 - 1) / (4 * 256);
  if (bx > 64) bx = 64;  // 64 blocks per slot: S * 64 blocks fill the chip for any S >= 32
  const dim3 grid(static_cast<unsigned>(bx), static_cast<unsigned>(S));
  place_slots_kernel<<<grid, 256, 0, s>>>(reinterpret_cast<const uint4*>(w), words, w_scale, scales,
                                          slot_expert, E, reinterpret_cast<uint4*>(w_slots), s_slots);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* dst, int64_t n, float v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  fill_f32_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(dst, n, v);
  return hipGetLastError();
}

}  // namespace dsmoe
