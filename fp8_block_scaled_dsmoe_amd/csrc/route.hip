// Router logits, auxiliary-loss-free group-limited top-K routing, the token
// permute and the bias update.
//
// Sources (V3 notes = xutianle.me "DeepSeek-V3 技术报告" walk-through):
//  * V3 notes §4: choose the top-K experts on s + b, weight the chosen ones by
//    the raw affinity s; after every step lower the bias of overloaded experts
//    and raise that of underloaded ones (§4.1: speed gamma = 0.001).
//  * V3 notes §4.2 / 51itzy.com infra answer (routing paragraph): a token may
//    only reach experts on a limited number of nodes (4 of 8); no dropping.
//  * V3 notes §6: the router is one of the cheap / sensitive modules kept in
//    higher precision, so its GEMM is bf16 x bf16 with FP32 accumulation.
//
// Readings taken where the page's formulas were lost: sigmoid affinity
// evaluated in float64 and rounded once to float32; key = fl32(s + b); a
// group scores by the float32 sum (largest first) of its ceil(K/Mg) largest
// keys; ties go to the lower group / expert index; gates are s normalised
// over the chosen experts (float32 sum in selection order).
#include "common.h"
#include "kernels.h"

namespace dsmoe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Router logits z[T][E] = x[T][H] . Wr[E][H]^T on bf16 MFMA (16x16x32).
// Block tile 64 tokens x 64 experts, K step 64, LDS double buffer with a
// 16-byte-segment XOR swizzle; four waves, each 32 x 32 (2 x 2 MFMA tiles).
// Small batches split H over blockIdx.z (router_splits): each split writes
// its partial sums, and a second kernel adds the splits in a fixed order, so
// the result does not depend on scheduling.
// ---------------------------------------------------------------------------
constexpr int RT = 64, RE = 64, RK = 64;  // RK bf16 = 128 bytes per row

// 16-byte segment seg of row `row` sits in slot seg ^ key(row); the key is
// distinct over any 8 consecutive rows and over the even (odd) rows of 16, so
// a 16-lane read of 16 rows spreads over all LDS banks.
__device__ __forceinline__ int swz(int row, int seg) {
  return row * 128 + ((seg ^ (row & 7) ^ ((row >> 3) & 1)) << 4);
}

__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr,
                                                            int64_t T, int64_t H, int32_t E,
                                                            int64_t k_len, float* __restrict__ z) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][RT * 128];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT;
  const int e0 = blockIdx.y * RE;
  const int64_t k_begin = static_cast<int64_t>(blockIdx.z) * k_len;   // this split's columns
  z += static_cast<int64_t>(blockIdx.z) * T * E;

  // global -> register loads: 2 x 16 bytes of x and of Wr per thread per step
  const uint16_t* xsrc[2];
  const uint16_t* wsrc[2];
  int lrow[2], lseg[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i;  // 0..511: 64 rows x 8 segments
    lrow[i] = idx >> 3;
    lseg[i] = idx & 7;
    const int64_t tr = min<int64_t>(t0 + lrow[i], T - 1);
    const int er = min(e0 + lrow[i], E - 1);
    xsrc[i] = x + tr * H + k_begin + lseg[i] * 8;
    wsrc[i] = wr + static_cast<int64_t>(er) * H + k_begin + lseg[i] * 8;
  }
  u32x4 xr[2], wrr[2];
#define DSMOE_GLOAD(k0)                                                    \
  do {                                                                     \
    _Pragma("unroll") for (int i = 0; i < 2; ++i) {                        \
      xr[i] = *reinterpret_cast<const u32x4*>(xsrc[i] + (k0));             \
      wrr[i] = *reinterpret_cast<const u32x4*>(wsrc[i] + (k0));            \
    }                                                                      \
  } while (0)
#define DSMOE_SSTORE(bb)                                                   \
  do {                                                                     \
    _Pragma("unroll") for (int i = 0; i < 2; ++i) {                        \
      *reinterpret_cast<u32x4*>(&lds[(bb)][0][swz(lrow[i], lseg[i])]) = xr[i];  \
      *reinterpret_cast<u32x4*>(&lds[(bb)][1][swz(lrow[i], lseg[i])]) = wrr[i]; \
    }                                                                      \
  } while (0)

  const int wm = wave >> 1, wn = wave & 1;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t steps = k_len / RK;
  DSMOE_GLOAD(0);
  DSMOE_SSTORE(0);
  __syncthreads();
  for (int64_t st = 0; st < steps; ++st) {
    const int buf = st & 1;
    if (st + 1 < steps) DSMOE_GLOAD((st + 1) * RK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int seg = ks * 4 + (lane >> 4);
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8*>(&lds[buf][0][swz(wm * 32 + i * 16 + (lane & 15), seg)]);
        bfr[i] = *reinterpret_cast<const bf16x8*>(&lds[buf][1][swz(wn * 32 + i * 16 + (lane & 15), seg)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (st + 1 < steps) DSMOE_SSTORE(buf ^ 1);
    __syncthreads();
  }
#undef DSMOE_GLOAD
#undef DSMOE_SSTORE

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + wn * 32 + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
        if (t < T && e < E) z[t * E + e] = acc[i][j][r];
      }
    }
}

// Wide variant for E a multiple of 256 and at least 128 tokens: block tile
// 128 tokens x 256 experts, eight waves as 2 (tokens) x 4 (experts), each
// 64 x 64 (4 x 4 MFMA tiles).  A block reads its x rows once for 256
// experts, where the 64 x 64 tiles read them once per 64, and keeps two K
// steps of loads in flight in registers: the step's data goes to LDS at the
// end of the step before, and the step after next is loaded at its start.
// (At 32768 tokens the 64 x 64 kernel, with one step of loads in flight,
// waited on them; 0.30 ms for 120 GFLOP.)  Same MFMA, same order of FP32
// accumulation over K and the same splits-and-reduce scheme as above.
constexpr int WRT = 128, WRE = 256;
constexpr int WSEGS = (WRT + WRE) * (RK * 2 / 16) / 512;   // 16-byte segments per thread and step

__global__ __launch_bounds__(512) void router_logits_wide_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ wr,
                                                                 int64_t T, int64_t H, int32_t E,
                                                                 int64_t k_len, float* __restrict__ z) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(WRT + WRE) * 128];   // x rows, then W rows
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * WRT;
  const int e0 = blockIdx.y * WRE;
  const int64_t k_begin = static_cast<int64_t>(blockIdx.z) * k_len;
  z += static_cast<int64_t>(blockIdx.z) * T * E;

  // segment i of this thread: tile row idx / 8 (x rows 0..127, W rows
  // 128..383), 16-byte segment idx % 8 of the step's 128 bytes
  const uint16_t* src[WSEGS];
  int dst[WSEGS];
#pragma unroll
  for (int i = 0; i < WSEGS; ++i) {
    const int idx = tid + 512 * i;
    const int row = idx >> 3, seg = idx & 7;
    if (row < WRT) {
      const int64_t tr = min<int64_t>(t0 + row, T - 1);
      src[i] = x + tr * H + k_begin + seg * 8;
    } else {
      src[i] = wr + static_cast<int64_t>(e0 + row - WRT) * H + k_begin + seg * 8;
    }
    dst[i] = swz(row, seg);
  }
  u32x4 ld[2][WSEGS];
#define DSMOE_WLOAD(set, k0)                                                                   \
  do {                                                                                         \
    _Pragma("unroll") for (int i = 0; i < WSEGS; ++i)                                          \
      ld[set][i] = *reinterpret_cast<const u32x4*>(src[i] + (k0));                             \
  } while (0)
#define DSMOE_WSTORE(set, bb)                                                                  \
  do {                                                                                         \
    _Pragma("unroll") for (int i = 0; i < WSEGS; ++i)                                          \
      *reinterpret_cast<u32x4*>(&lds[(bb)][dst[i]]) = ld[set][i];                              \
  } while (0)

  const int wm = wave >> 2, wn = wave & 3;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one K step on buffer bb: two MFMA K slices of 32
#define DSMOE_WCOMPUTE(bb)                                                                     \
  do {                                                                                         \
    _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                         \
      const int seg = ks * 4 + (lane >> 4);                                                    \
      bf16x8 af[4], bfr[4];                                                                    \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                          \
        af[i] = *reinterpret_cast<const bf16x8*>(&lds[(bb)][swz(wm * 64 + i * 16 + (lane & 15), seg)]); \
        bfr[i] = *reinterpret_cast<const bf16x8*>(                                             \
            &lds[(bb)][swz(WRT + wn * 64 + i * 16 + (lane & 15), seg)]);                        \
      }                                                                                        \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                                            \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                                          \
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0); \
    }                                                                                          \
  } while (0)

  const int64_t steps = k_len / RK;
  DSMOE_WLOAD(0, 0);
  if (steps > 1) DSMOE_WLOAD(1, RK);
  DSMOE_WSTORE(0, 0);
  __syncthreads();
  // step s uses buffer s & 1 and register set s & 1 (the loop is unrolled by
  // two so that the sets are indexed with constants)
  for (int64_t st = 0; st < steps; st += 2) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t s_ = st + b;
      if (s_ < steps) {
        if (s_ + 2 < steps) DSMOE_WLOAD(b, (s_ + 2) * RK);   // set b's step is in LDS already
        DSMOE_WCOMPUTE(b);
        if (s_ + 1 < steps) DSMOE_WSTORE(b ^ 1, b ^ 1);      // buffer b^1 was read in step s-1
        __syncthreads();
      }
    }
  }
#undef DSMOE_WLOAD
#undef DSMOE_WSTORE
#undef DSMOE_WCOMPUTE

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
        if (t < T) z[t * E + e] = acc[i][j][r];
      }
    }
}

// z[t][e] = sum over splits s = 0, 1, ... of part[s][t][e], in that order;
// 4 values per thread.  The splits are loaded 8 at a time before they are
// added (in the same order): one load per iteration waited for each load in
// turn, and 28 splits at 64 tokens took 9.7 us.
__global__ __launch_bounds__(256) void router_reduce_kernel(const float* __restrict__ part,
                                                            int32_t splits, int64_t n,
                                                            float* __restrict__ z) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 v = *reinterpret_cast<const f32x4*>(part + i);
  int32_t sp = 1;
  for (; sp + 8 <= splits; sp += 8) {
    f32x4 u[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      u[q] = *reinterpret_cast<const f32x4*>(part + static_cast<int64_t>(sp + q) * n + i);
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = v[r] + u[q][r];
  }
  for (; sp < splits; ++sp) {
    const f32x4 u = *reinterpret_cast<const f32x4*>(part + static_cast<int64_t>(sp) * n + i);
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = v[r] + u[r];
  }
  *reinterpret_cast<f32x4*>(z + i) = v;
}

// ---------------------------------------------------------------------------
// Top-K selection: one wave per token.  Expert e lives in lane e % 64,
// slot e / 64.  Ordering everywhere: value descending, index ascending.
// ---------------------------------------------------------------------------
struct Cand {
  float v;
  int i;      // index; -1 = no candidate
  float pay;  // payload carried with the winner (the raw affinity s)
};

__device__ __forceinline__ bool better(const Cand& a, const Cand& b) {
  if (a.i < 0) return false;
  if (b.i < 0) return true;
  return a.v > b.v || (a.v == b.v && a.i < b.i);
}

template <int CTRL>
__device__ __forceinline__ Cand cand_dpp(const Cand& c) {
  Cand d;
  d.v = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, c.v), CTRL, 0xF, 0xF, false));
  d.i = __builtin_amdgcn_update_dpp(0, c.i, CTRL, 0xF, 0xF, false);
  d.pay = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, c.pay), CTRL, 0xF, 0xF, false));
  return d;
}

// The wave's best candidate, in every lane.  `better` is a strict total order
// (value descending, index ascending; no candidate last), so any pairing of
// lanes gives the same winner: within each 16-lane row DPP exchanges with
// lane ^ 1, lane ^ 2, the mirrored lane in the 8-lane half and in the row;
// then lane ^ 16 (ds_swizzle), and the two 32-lane halves' winners meet in
// scalar registers.  (Six ds_bpermute rounds of three values made the 12
// selection rounds of a token the latency of the selection kernel.)
__device__ __forceinline__ Cand wave_best(Cand c) {
  {
    const Cand d = cand_dpp<0xB1>(c);   // quad_perm [1,0,3,2]: lane ^ 1
    if (better(d, c)) c = d;
  }
  {
    const Cand d = cand_dpp<0x4E>(c);   // quad_perm [2,3,0,1]: lane ^ 2
    if (better(d, c)) c = d;
  }
  {
    const Cand d = cand_dpp<0x141>(c);  // row_half_mirror: lane 7 - l within 8
    if (better(d, c)) c = d;
  }
  {
    const Cand d = cand_dpp<0x140>(c);  // row_mirror: lane 15 - l within 16
    if (better(d, c)) c = d;
  }
  {
    constexpr int kXor16 = (0x10 << 10) | 0x1F;   // ds_swizzle bit mode: lane ^ 16 within 32
    Cand d;
    d.v = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, c.v), kXor16));
    d.i = __builtin_amdgcn_ds_swizzle(c.i, kXor16);
    d.pay = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, c.pay), kXor16));
    if (better(d, c)) c = d;
  }
  Cand lo, hi;
  lo.v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c.v), 0));
  lo.i = __builtin_amdgcn_readlane(c.i, 0);
  lo.pay = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c.pay), 0));
  hi.v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c.v), 32));
  hi.i = __builtin_amdgcn_readlane(c.i, 32);
  hi.pay = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c.pay), 32));
  return better(hi, lo) ? hi : lo;
}

// One wave per token, WAVES tokens per block.  The block's choices are
// counted in LDS and added to counts[] with one atomic per expert it chose:
// under skew, per-choice atomics on the hot experts' counters serialised.
// LDS: (WAVES + 1) * E * 4 bytes (16 waves while that stays within 64 KB).
template <int SLOTS, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void route_select_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int64_t T, int32_t E,
    int32_t G, int32_t Mg, int32_t K, int32_t* __restrict__ topk_idx, float* __restrict__ gates,
    int32_t* __restrict__ counts) {
  extern __shared__ float key_lds[];  // [WAVES][E] keys, then [E] block counts
  int32_t* blk_cnt = reinterpret_cast<int32_t*>(key_lds + WAVES * E);
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < E; i += WAVES * 64) blk_cnt[i] = 0;
  const int64_t t_raw = static_cast<int64_t>(blockIdx.x) * WAVES + wave;
  const bool valid = t_raw < T;
  const int64_t t = valid ? t_raw : T - 1;  // tail waves recompute the last token, write nothing
  float* keys = key_lds + wave * E;

  float s[SLOTS], key[SLOTS];
  const float* zrow = logits + t * E;
#pragma unroll
  for (int j = 0; j < SLOTS; ++j) {
    const int e = j * 64 + lane;
    if (e < E) {
      const double zd = static_cast<double>(zrow[e]);
      s[j] = static_cast<float>(1.0 / (1.0 + exp(-zd)));
      key[j] = s[j] + bias[e];
      keys[e] = key[j];
    } else {
      s[j] = 0.f;
      key[j] = 0.f;
    }
  }
  __syncthreads();

  // group scores: lane g < G sums the n_top largest keys of its group, found
  // by repeated "next in order after the previous pick" scans
  const int per_group = E / G;
  const int n_top = (K + Mg - 1) / Mg;
  Cand gs;
  gs.i = -1;
  gs.v = 0.f;
  gs.pay = 0.f;
  if (lane < G) {
    float acc = 0.f;
    float pv = 0.f;
    int pi = -1;
    for (int n = 0; n < n_top; ++n) {
      float bv = 0.f;
      int bi = -1;
      // (keys read 8 at a time, then compared in index order)
      int q = 0;
      for (; q + 8 <= per_group; q += 8) {
        float kv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kv[u] = keys[lane * per_group + q + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = lane * per_group + q + u;
          const float v = kv[u];
          const bool after = (pi < 0) || (v < pv) || (v == pv && e > pi);
          if (after && (bi < 0 || v > bv)) {  // strict > keeps the lowest index on ties
            bv = v;
            bi = e;
          }
        }
      }
      for (; q < per_group; ++q) {
        const int e = lane * per_group + q;
        const float v = keys[e];
        const bool after = (pi < 0) || (v < pv) || (v == pv && e > pi);
        if (after && (bi < 0 || v > bv)) {
          bv = v;
          bi = e;
        }
      }
      acc = (n == 0) ? bv : acc + bv;
      pv = bv;
      pi = bi;
    }
    gs.v = acc;
    gs.i = lane;
  }

  // keep the Mg best groups
  uint64_t kept = 0;
  for (int m = 0; m < Mg; ++m) {
    Cand c = gs;
    if (c.i >= 0 && ((kept >> c.i) & 1ull)) c.i = -1;
    const Cand w = wave_best(c);
    kept |= 1ull << w.i;
  }

  // choose K experts among the kept groups; lane k keeps the k-th choice and
  // every lane forms the same float32 sum of s in selection order
  uint32_t taken = 0;
  int my_e = 0;
  float my_s = 0.f;
  float sum = 0.f;
  for (int k = 0; k < K; ++k) {
    Cand c;
    c.i = -1;
    c.v = 0.f;
    c.pay = 0.f;
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const int e = j * 64 + lane;
      if (e < E && !((taken >> j) & 1u) && ((kept >> (e / per_group)) & 1ull)) {
        Cand d{key[j], e, s[j]};
        if (better(d, c)) c = d;
      }
    }
    const Cand w = wave_best(c);
    if ((w.i & 63) == lane) taken |= 1u << (w.i >> 6);
    if (lane == k) {
      my_e = w.i;
      my_s = w.pay;
    }
    sum = (k == 0) ? w.pay : sum + w.pay;
  }

  if (valid && lane < K) {
    topk_idx[t * K + lane] = my_e;
    gates[t * K + lane] = my_s / sum;
    atomicAdd(&blk_cnt[my_e], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += WAVES * 64)
    if (blk_cnt[i] != 0) atomicAdd(&counts[i], blk_cnt[i]);
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// offsets = exclusive scan of counts (one block of 1024 threads, E <= 1024);
// optionally the extended table with one more group of `extra` rows.
__global__ __launch_bounds__(1024) void offsets_kernel(const int32_t* __restrict__ counts,
                                                       int32_t E, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ offsets_ext,
                                                       int64_t extra) {
  __shared__ int32_t buf[1024];
  const int tid = threadIdx.x;
  int32_t v = tid < E ? counts[tid] : 0;
  buf[tid] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t add = tid >= o ? buf[tid - o] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  if (tid < E) {
    offsets[tid + 1] = buf[tid];
    if (offsets_ext) offsets_ext[tid + 1] = buf[tid];
  }
  if (tid == 0) {
    offsets[0] = 0;
    if (offsets_ext) {
      offsets_ext[0] = 0;
      offsets_ext[E + 1] = buf[E - 1] + static_cast<int32_t>(extra);
    }
  }
}

// Block e lists the (token, k) entries that chose expert e, in token order.
// Entry i = t*K + k.  The 1024 threads take slabs of 8192 entries, 8
// consecutive entries each; a thread's matches get consecutive positions after
// an exclusive scan of the per-thread match counts (within the wave by
// shuffles, across the 16 waves through LDS).  The next slab is loaded before
// the current one is scanned.  VEC: topk_idx is 16-byte aligned (two 16-byte
// loads per thread), otherwise 4-byte loads.
constexpr int kRankThreads = 1024;
constexpr int kRankPer = 8;

template <bool VEC>
__device__ __forceinline__ void rank_load(const int32_t* __restrict__ topk_idx, int64_t first, int64_t n,
                                          int32_t (&v)[kRankPer]) {
  if (VEC && first + kRankPer <= n) {
    const int4 a = *reinterpret_cast<const int4*>(topk_idx + first);
    const int4 b = *reinterpret_cast<const int4*>(topk_idx + first + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int q = 0; q < kRankPer; ++q) v[q] = first + q < n ? topk_idx[first + q] : -1;
  }
}

template <bool VEC>
__global__ __launch_bounds__(kRankThreads) void rank_kernel(const int32_t* __restrict__ topk_idx,
                                                            const float* __restrict__ gates, int64_t T,
                                                            int32_t E, int32_t K,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ inv,
                                                            float* __restrict__ row_gate,
                                                            int32_t ext) {
  constexpr int NW = kRankThreads / 64;
  constexpr int64_t STEP = static_cast<int64_t>(kRankThreads) * kRankPer;
  __shared__ int32_t wave_cnt[2][NW];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = T * K;
  int32_t base = offsets[e];
  int32_t cur[kRankPer];
  rank_load<VEC>(topk_idx, static_cast<int64_t>(tid) * kRankPer, n, cur);
  int par = 0;
  for (int64_t i0 = 0; i0 < n; i0 += STEP) {
    const int64_t first = i0 + static_cast<int64_t>(tid) * kRankPer;
    uint32_t mask = 0;
    int m = 0;
#pragma unroll
    for (int q = 0; q < kRankPer; ++q) {
      const bool hit = cur[q] == e;
      mask |= static_cast<uint32_t>(hit) << q;
      m += hit;
    }
    if (i0 + STEP < n) rank_load<VEC>(topk_idx, first + STEP, n, cur);
    int incl = m;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    if (lane == 63) wave_cnt[par][wave] = incl;
    __syncthreads();
    int wbase = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = wave_cnt[par][w];
      wbase += w < wave ? c : 0;
      total += c;
    }
    int32_t pos = base + wbase + incl - m;
    while (mask) {
      const int q = __builtin_ctz(mask);
      mask &= mask - 1;
      const int64_t i = first + q;
      perm[pos] = static_cast<int32_t>(i / K);
      inv[i] = pos;
      if (row_gate) row_gate[pos] = gates[i];
      ++pos;
    }
    base += total;
    par ^= 1;   // the other wave_cnt buffer: no second barrier per slab
  }
  if (ext) {  // identity rows for the shared expert: perm[T*K + t] = t
    for (int64_t t = static_cast<int64_t>(e) * kRankThreads + tid; t < T;
         t += static_cast<int64_t>(E) * kRankThreads)
      perm[n + t] = static_cast<int32_t>(t);
  }
}

__global__ void update_bias_kernel(float* __restrict__ bias, const int32_t* __restrict__ counts,
                                   int32_t E, int64_t T, int32_t K, float gamma) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int64_t d = T * K - static_cast<int64_t>(E) * counts[e];
  const float step = d > 0 ? gamma : (d < 0 ? -gamma : 0.0f);
  bias[e] = bias[e] + step;
}

}  // namespace

bool router_wide(int64_t T, int32_t E) { return E % WRE == 0 && T >= WRT; }

int router_splits(int64_t T, int64_t H, int32_t E) {
  // 64 x 64 tiles: enough blocks to cover the device four times (about 1024;
  // 512 was 15% slower at 4096 tokens, 2048 no faster).  The wide tiles (one
  // block per CU: 96 KB of LDS) aim at 256 blocks.  Each split is at least
  // 256 columns long, and T * E a multiple of 4 for the reduction.
  const bool wide = router_wide(T, E);
  const int64_t base = wide ? ((T + WRT - 1) / WRT) * (E / WRE) : ((T + RT - 1) / RT) * ((E + RE - 1) / RE);
  const int64_t target = wide ? 256 : 1024;
  if (base <= 0 || base >= target || (T * E) % 4 != 0) return 1;
  int64_t want = (target + base - 1) / base;
  const int64_t steps = H / RK;
  int best = 1;
  for (int64_t sp = 2; sp <= want && sp * 4 <= steps; ++sp)
    if (steps % sp == 0) best = static_cast<int>(sp);
  return best;
}

size_t router_partial_bytes(int64_t T, int64_t H, int32_t E) {
  const int sp = router_splits(T, H, E);
  return sp > 1 ? static_cast<size_t>(sp) * T * E * sizeof(float) : 0;
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, int64_t T, int64_t H,
                                int32_t E, float* logits, float* partial, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int sp = router_splits(T, H, E);
  if (router_wide(T, E)) {
    const dim3 grid(static_cast<unsigned>((T + WRT - 1) / WRT), static_cast<unsigned>(E / WRE),
                    static_cast<unsigned>(sp));
    router_logits_wide_kernel<<<grid, 512, 0, s>>>(x, wr, T, H, E, H / sp, sp > 1 ? partial : logits);
  } else {
    const dim3 grid(static_cast<unsigned>((T + RT - 1) / RT), static_cast<unsigned>((E + RE - 1) / RE),
                    static_cast<unsigned>(sp));
    router_logits_kernel<<<grid, 256, 0, s>>>(x, wr, T, H, E, H / sp, sp > 1 ? partial : logits);
  }
  if (sp > 1) {
    const int64_t n = T * E;
    router_reduce_kernel<<<static_cast<unsigned>((n / 4 + 255) / 256), 256, 0, s>>>(partial, sp, n, logits);
  }
  return hipGetLastError();
}

hipError_t launch_route_select(const float* logits, const float* bias, int64_t T, int32_t E,
                               int32_t G, int32_t Mg, int32_t K, int32_t* topk_idx,
                               float* gates, int32_t* counts, hipStream_t s) {
  fill_i32_kernel<<<(E + 255) / 256, 256, 0, s>>>(counts, E, 0);
  if (T == 0) return hipGetLastError();
  // 16 tokens per block for large batches (fewer atomics on hot experts), 4
  // for small ones (more blocks in flight: 64 tokens in 4 blocks were slower)
  const int waves = T < 1024 ? 4 : (17 * static_cast<int64_t>(E) * 4 <= 65536) ? 16 : 8;
  const dim3 grid(static_cast<unsigned>((T + waves - 1) / waves));
  const dim3 block(waves * 64);
  const size_t lds = sizeof(float) * (waves + 1) * static_cast<size_t>(E);
  const int slots = (E + 63) / 64;
#define DSMOE_SEL(SL)                                                                              \
  do {                                                                                             \
    if (waves == 16)                                                                               \
      route_select_kernel<SL, 16><<<grid, block, lds, s>>>(logits, bias, T, E, G, Mg, K, topk_idx, \
                                                           gates, counts);                         \
    else if (waves == 8)                                                                           \
      route_select_kernel<SL, 8><<<grid, block, lds, s>>>(logits, bias, T, E, G, Mg, K, topk_idx,  \
                                                          gates, counts);                          \
    else                                                                                           \
      route_select_kernel<SL, 4><<<grid, block, lds, s>>>(logits, bias, T, E, G, Mg, K, topk_idx,  \
                                                          gates, counts);                          \
  } while (0)
  if (slots <= 1)
    DSMOE_SEL(1);
  else if (slots <= 2)
    DSMOE_SEL(2);
  else if (slots <= 4)
    DSMOE_SEL(4);
  else if (slots <= 8)
    DSMOE_SEL(8);
  else
    DSMOE_SEL(16);
#undef DSMOE_SEL
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* topk_idx, const float* gates, int64_t T, int32_t E,
                          int32_t K, const int32_t* counts, int32_t* offsets, int32_t* perm,
                          int32_t* inv, float* row_gate, int32_t* offsets_ext, hipStream_t s) {
  offsets_kernel<<<1, 1024, 0, s>>>(counts, E, offsets, offsets_ext, T);
  if (T == 0) return hipGetLastError();
  const int32_t ext = offsets_ext != nullptr ? 1 : 0;
  if ((reinterpret_cast<uintptr_t>(topk_idx) & 15) == 0)
    rank_kernel<true><<<E, kRankThreads, 0, s>>>(topk_idx, gates, T, E, K, offsets, perm, inv, row_gate, ext);
  else
    rank_kernel<false><<<E, kRankThreads, 0, s>>>(topk_idx, gates, T, E, K, offsets, perm, inv, row_gate, ext);
  return hipGetLastError();
}

hipError_t launch_update_bias(float* bias, const int32_t* counts, int32_t E, int64_t T,
                              int32_t K, float gamma, hipStream_t s) {
  update_bias_kernel<<<(E + 255) / 256, 256, 0, s>>>(bias, counts, E, T, K, gamma);
  return hipGetLastError();
}

}  // namespace dsmoe
