// Block-scaled FP8 (E4M3) grouped GEMM for gfx950 with per-128-K FP32
// promotion, and its fused epilogues.
//
// Method (V3 notes = xutianle.me "DeepSeek-V3 技术报告" walk-through):
//  * §6.1: activations carry one FP32 scale per 1x128 tile, weights one per
//    128x128 block;
//  * §6.2: the FP8 products are summed 128 at a time and each partial sum is
//    promoted to FP32, scaled, and accumulated there.
// On gfx950 one v_mfma_f32_16x16x128_f8f6f4 contracts exactly one 128-wide
// K chunk of a 16x16 output tile, so every MFMA is issued with a zero
// accumulator and its result is the chunk's partial sum; the FP32
// rescale-and-accumulate acc += P * (sa[row] * sw[block]) runs on the VALU.
//
// Tiling: block tile 128 rows x BN columns, K step 128 (one chunk), waves of
// 64 x 64 (4 x 4 MFMA tiles).  A and W chunks are staged through LDS (double
// buffered, 16-byte segments XOR-swizzled by row so MFMA operand reads are
// bank-conflict free) with the next chunk prefetched into registers.
// Rows of a group are gathered through a_rows (the token permute), so the
// permuted activation matrix is never materialised.  Group sizes stay on the
// device: every block derives its (group, row tile) from offsets[].  Logical
// tile order is remapped so that consecutive tiles land on the same XCD
// (blocks are dispatched round-robin over the 8 XCDs) and share its L2.
#include "common.h"
#include "kernels.h"

namespace dsmoe {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BK = 128;
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int row, int seg) { return row * BK + ((seg ^ (row & 7)) << 4); }

__device__ __forceinline__ f32x4 mfma_chunk(const i32x8& a, const i32x8& b) {
  // cbsz = blgp = 0 selects FP8 E4M3 for both operands; zero scale operands
  // select the unscaled instruction.
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Find the group and row range of global row-tile `mt` (tiles are numbered
// group by group, ceil(n_g / BM) per group).  Returns false past the end.
template <int THREADS>
__device__ bool decode_tile(const int32_t* __restrict__ offsets, int32_t G, int64_t mt,
                            int32_t* s_scan, int64_t* s_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = THREADS / 64;
  if (tid == 0) s_out[0] = -1;
  int64_t carry = 0;
  for (int32_t g0 = 0; g0 < G; g0 += THREADS) {
    const int32_t g = g0 + tid;
    int32_t lo = 0, hi = 0, cnt = 0;
    if (g < G) {
      lo = offsets[g];
      hi = offsets[g + 1];
      cnt = hi > lo ? (hi - lo + BM - 1) / BM : 0;
    }
    // inclusive scan of cnt over the block
    int32_t v = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t u = __shfl_up(v, o, 64);
      if (lane >= o) v += u;
    }
    if (lane == 63) s_scan[wave] = v;
    __syncthreads();
    int32_t wbase = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int32_t t = s_scan[w];
      if (w < wave) wbase += t;
      total += t;
    }
    const int64_t incl = carry + wbase + v;
    const int64_t excl = incl - cnt;
    if (cnt > 0 && mt >= excl && mt < incl) {
      const int64_t r0 = lo + (mt - excl) * BM;
      s_out[0] = g;
      s_out[1] = r0;
      s_out[2] = min<int64_t>(r0 + BM, hi);
    }
    carry += total;
    __syncthreads();
  }
  return s_out[0] >= 0;
}

template <int BN, Epilogue EPI>
struct Kcfg {
  static constexpr int WN = BN / 64;          // waves along N
  static constexpr int THREADS = 2 * WN * 64; // 2 waves along M
  static constexpr int A_LOADS = (BM * 8) / THREADS;   // 16-byte segments per thread
  static constexpr int B_LOADS = (BN * 8) / THREADS;
};

template <int BN, Epilogue EPI>
__global__ __launch_bounds__(2 * BN) void gemm_kernel(GemmProblem p, int64_t n_tiles) {
  using C = Kcfg<BN, EPI>;
  constexpr int THREADS = C::THREADS;
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][BN * BK];
  __shared__ __attribute__((aligned(16))) float s_sa[2][BM];
  __shared__ int32_t s_scan[THREADS / 64];
  __shared__ int64_t s_tile[3];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;

  // XCD-aware logical tile id: blocks bid, bid+8, ... share an XCD; give
  // each XCD a contiguous range of logical tiles.
  const int64_t nblk = gridDim.x;
  const int64_t bid = blockIdx.x;
  const int64_t per_xcd = nblk / kXcds;
  const int64_t logical = (bid % kXcds) * per_xcd + bid / kXcds;
  const int64_t mt = logical / n_tiles;
  const int64_t nt = logical - mt * n_tiles;

  if (!decode_tile<THREADS>(p.offsets, p.G, mt, s_scan, s_tile)) return;
  const int32_t g = static_cast<int32_t>(s_tile[0]);
  const int64_t row0 = s_tile[1];
  const int64_t row1 = min(s_tile[2], p.row_limit);  // guards against offsets past the buffers
  if (row0 >= row1) return;

  const int64_t K = p.K, N = p.N;
  const int64_t kchunks = K / BK;
  const bool last = (p.w_last != nullptr) && (g == p.G - 1);
  const uint8_t* wbase = last ? p.w_last : p.w + static_cast<int64_t>(g) * N * K;
  const float* wsbase = last ? p.w_scale_last : p.w_scale + static_cast<int64_t>(g) * (N / BK) * kchunks;

  // W row of local column lc (SwiGLU: 128 gate rows, then the matching 128 up rows)
  const int64_t w_row_base = (EPI == Epilogue::kSwiGLUQuant) ? nt * 128 : nt * BN;
  const int64_t w_up_shift = (EPI == Epilogue::kSwiGLUQuant) ? N / 2 - 128 : 0;
#define DSMOE_WROW(lc) (w_row_base + (lc) + ((lc) >= 128 ? w_up_shift : 0))

  // per-thread global sources
  const uint8_t* a_src[C::A_LOADS];
  int a_lds[C::A_LOADS];
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int idx = tid + THREADS * i;
    const int lr = idx >> 3, seg = idx & 7;
    const int64_t r = row0 + lr < row1 ? row0 + lr : row0;
    const int64_t src = p.a_rows ? p.a_rows[r] : r;
    a_src[i] = p.a + src * K + seg * 16;
    a_lds[i] = swz(lr, seg);
  }
  const uint8_t* b_src[C::B_LOADS];
  int b_lds[C::B_LOADS];
#pragma unroll
  for (int i = 0; i < C::B_LOADS; ++i) {
    const int idx = tid + THREADS * i;
    const int lc = idx >> 3, seg = idx & 7;
    b_src[i] = wbase + DSMOE_WROW(lc) * K + seg * 16;
    b_lds[i] = swz(lc, seg);
  }
  const float* sa_src = nullptr;
  if (tid < BM) {
    const int64_t r = row0 + tid < row1 ? row0 + tid : row0;
    const int64_t src = p.a_rows ? p.a_rows[r] : r;
    sa_src = p.a_scale + src * kchunks;
  }
  // this wave's 64 columns sit in one 128-row block of W
  const float* sw_src = wsbase + (DSMOE_WROW(wn * 64) / BK) * kchunks;
#undef DSMOE_WROW

  u32x4 ra[C::A_LOADS], rb[C::B_LOADS];
  float rsa = 0.f;
  // (plain macros rather than lambdas: a by-reference capture would make the
  // register arrays addressable and move them to LDS)
#define DSMOE_GLOAD(cc)                                                                     \
  do {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < C::A_LOADS; ++i) ra[i] =                          \
        *reinterpret_cast<const u32x4*>(a_src[i] + (cc) * BK);                              \
    _Pragma("unroll") for (int i = 0; i < C::B_LOADS; ++i) rb[i] =                          \
        *reinterpret_cast<const u32x4*>(b_src[i] + (cc) * BK);                              \
    if (tid < BM) rsa = sa_src[(cc)];                                                       \
  } while (0)
#define DSMOE_SSTORE(bb)                                                                    \
  do {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < C::A_LOADS; ++i)                                  \
        *reinterpret_cast<u32x4*>(&s_a[(bb)][a_lds[i]]) = ra[i];                            \
    _Pragma("unroll") for (int i = 0; i < C::B_LOADS; ++i)                                  \
        *reinterpret_cast<u32x4*>(&s_b[(bb)][b_lds[i]]) = rb[i];                            \
    if (tid < BM) s_sa[(bb)][tid] = rsa;                                                    \
  } while (0)

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15;       // row (A) / column (B) inside a 16x16 tile
  const int fseg = (lane >> 4) * 2; // first of the two 16-byte K segments
  DSMOE_GLOAD(0);
  DSMOE_SSTORE(0);
  __syncthreads();
  for (int64_t c = 0; c < kchunks; ++c) {
    const int buf = static_cast<int>(c & 1);
    if (c + 1 < kchunks) DSMOE_GLOAD(c + 1);
    const float sw = sw_src[c];

    i32x8 af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + i * 16 + frow;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(&s_a[buf][swz(r, fseg)]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(&s_a[buf][swz(r, fseg + 1)]);
      af[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 64 + j * 16 + frow;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(&s_b[buf][swz(r, fseg)]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(&s_b[buf][swz(r, fseg + 1)]);
      bfr[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    float scl[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 sa4 = *reinterpret_cast<const f32x4*>(&s_sa[buf][wm * 64 + i * 16 + (lane >> 4) * 4]);
#pragma unroll
      for (int r = 0; r < 4; ++r) scl[i][r] = sa4[r] * sw;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 part = mfma_chunk(af[i], bfr[j]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(part[r], scl[i][r], acc[i][j][r]);
      }
    if (c + 1 < kchunks) DSMOE_SSTORE(buf ^ 1);
    __syncthreads();
  }
#undef DSMOE_GLOAD
#undef DSMOE_SSTORE

  // ------------------------------------------------------------------ epilogues
  // lane (i, j, r) holds output row  wm*64 + 16i + 4*(lane/16) + r
  //                       and column wn*64 + 16j + lane%16
  if constexpr (EPI == Epilogue::kStore || EPI == Epilogue::kGateStore) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = row0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
        if (row >= row1) continue;
        float gsc = 1.0f;
        if constexpr (EPI == Epilogue::kGateStore) gsc = p.row_gate[row];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = nt * BN + wn * 64 + j * 16 + frow;
          float v = acc[i][j][r];
          if constexpr (EPI == Epilogue::kGateStore) v = v * gsc;
          if (p.c_f32)
            static_cast<float*>(p.c)[row * N + col] = v;
          else
            static_cast<uint16_t*>(p.c)[row * N + col] = f32_to_bf16(v);
        }
      }
  } else if constexpr (EPI == Epilogue::kCombine) {
    const int32_t K_ = p.topk;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = row0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
        if (row >= row1) continue;
        const int64_t tok = row - p.row_base;
        const int32_t* inv_t = p.inv + tok * K_;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = nt * BN + wn * 64 + j * 16 + frow;
          float v = acc[i][j][r];
          for (int k = 0; k < K_; ++k) {
            const int64_t orow = inv_t[k];
            if (p.c_f32)
              v = v + static_cast<const float*>(p.o_routed)[orow * N + col];
            else
              v = v + bf16_to_f32(static_cast<const uint16_t*>(p.o_routed)[orow * N + col]);
          }
          if (p.c_f32)
            static_cast<float*>(p.c)[tok * N + col] = v;
          else
            static_cast<uint16_t*>(p.c)[tok * N + col] = f32_to_bf16(v);
        }
      }
  } else {  // kSwiGLUQuant: waves 0,1 (per M half) hold gate columns, 2,3 up columns
    float* s_up = reinterpret_cast<float*>(&s_b[0][0]);          // [128][128] f32 = 64 KB
    float* s_rmax = reinterpret_cast<float*>(&s_a[0][0]);        // [2][128]
    uint8_t* s_code = &s_a[1][0];                                // [128][128] bytes
    if (wn >= 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int lr = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
            const int lc = (wn - 2) * 64 + j * 16 + frow;
            s_up[lr * 128 + lc] = acc[i][j][r];
          }
    }
    __syncthreads();
    float av[4][4][4];
    if (wn < 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
          float m = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int lc = wn * 64 + j * 16 + frow;
            const float gt = acc[i][j][r];
            const float up = s_up[lr * 128 + lc];
            const float a = gt / (1.0f + expf(-gt)) * up;
            av[i][j][r] = a;
            m = fmaxf(m, fabsf(a));
          }
          m = wave_max_width(m, 16);
          if (frow == 0) s_rmax[wn * 128 + lr] = m;
        }
    }
    __syncthreads();
    if (wn < 2) {
      const int64_t I = N / 2;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
          const float amax = fmaxf(s_rmax[lr], s_rmax[128 + lr]);
          const float s = amax == 0.0f ? 1.0f : amax / 448.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int lc = wn * 64 + j * 16 + frow;
            s_code[lr * 128 + lc] = static_cast<uint8_t>(e4m3_encode(av[i][j][r] / s));
          }
          const int64_t row = row0 + lr;
          if (wn == 0 && frow == 0 && row < row1) p.c_scale[row * (I / BK) + nt] = s;
        }
    }
    __syncthreads();
    // coalesced code store: 128 rows x 128 bytes, 16 bytes per thread per step
    const int64_t I = N / 2;
    for (int idx = tid; idx < BM * 8; idx += THREADS) {
      const int lr = idx >> 3, seg = idx & 7;
      const int64_t row = row0 + lr;
      if (row < row1)
        *reinterpret_cast<uint4*>(static_cast<uint8_t*>(p.c) + row * I + nt * 128 + seg * 16) =
            *reinterpret_cast<const uint4*>(&s_code[lr * 128 + seg * 16]);
    }
  }
}

template <int BN, Epilogue EPI>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t s) {
  const int64_t n_tiles = (EPI == Epilogue::kSwiGLUQuant) ? (p.N / 2) / 128 : p.N / BN;
  const int64_t m_tiles_ub = (p.M_total + BM - 1) / BM + p.G;
  int64_t blocks = m_tiles_ub * n_tiles;
  blocks = (blocks + kXcds - 1) / kXcds * kXcds;
  if (blocks == 0) return hipSuccess;
  gemm_kernel<BN, EPI><<<dim3(static_cast<unsigned>(blocks)), Kcfg<BN, EPI>::THREADS, 0, s>>>(p, n_tiles);
  return hipGetLastError();
}

// y[t][n] = sum over k of o[inv[t][k]][n] (layers without a shared expert);
// float32 sum in ascending k, 8 columns per thread.
template <bool kF32>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ o,
                                                      const int32_t* __restrict__ inv, int64_t T,
                                                      int32_t K, int64_t H, void* __restrict__ y) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per_row = H / 8;
  if (idx >= T * per_row) return;
  const int64_t t = idx / per_row;
  const int64_t c0 = (idx - t * per_row) * 8;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < K; ++k) {
    const int64_t r = inv[t * K + k];
    for (int e = 0; e < 8; ++e) {
      const float x = kF32 ? static_cast<const float*>(o)[r * H + c0 + e]
                           : bf16_to_f32(static_cast<const uint16_t*>(o)[r * H + c0 + e]);
      v[e] = (k == 0) ? x : v[e] + x;
    }
  }
  for (int e = 0; e < 8; ++e) {
    if (kF32)
      static_cast<float*>(y)[t * H + c0 + e] = v[e];
    else
      static_cast<uint16_t*>(y)[t * H + c0 + e] = f32_to_bf16(v[e]);
  }
}

}  // namespace

hipError_t launch_combine(const void* o, const int32_t* inv, int64_t T, int32_t K, int64_t H,
                          void* y, bool f32, hipStream_t s) {
  const int64_t threads = T * (H / 8);
  if (threads == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (f32)
    combine_kernel<true><<<grid, 256, 0, s>>>(o, inv, T, K, H, y);
  else
    combine_kernel<false><<<grid, 256, 0, s>>>(o, inv, T, K, H, y);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmProblem& p, hipStream_t s) {
  if (p.M_total == 0) return hipSuccess;
  switch (p.epi) {
    case Epilogue::kStore:
      return launch_cfg<128, Epilogue::kStore>(p, s);
    case Epilogue::kGateStore:
      return launch_cfg<128, Epilogue::kGateStore>(p, s);
    case Epilogue::kCombine:
      return launch_cfg<128, Epilogue::kCombine>(p, s);
    case Epilogue::kSwiGLUQuant:
      return launch_cfg<256, Epilogue::kSwiGLUQuant>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dsmoe
