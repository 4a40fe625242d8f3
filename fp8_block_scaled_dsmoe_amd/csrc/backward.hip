// The FP8 backward of the expert FFN beyond the data-gradient GEMMs (which
// run on the forward's grouped GEMM with block-transposed weights):
//
//  * quant_tokens_kernel: 1x128 tiles along each expert's tokens.  V3 notes
//    §6 puts the weight-gradient (Wgrad) GEMMs in FP8 as well; they contract
//    over the tokens of an expert, so both operands are quantised in tiles of
//    128 consecutive rows of the expert's group (per column), starting at the
//    group's first row; the codes are written transposed, [column][token], so
//    that the Wgrad GEMM reads 128-byte K chunks like every other GEMM here.
//  * wgrad_kernel: per group g, c_g = A_g B_g^T over the group's token tiles,
//    both operands with one scale per (row, tile): the per-128 promotion
//    (V3 notes §6.2) multiplies each MFMA's partial sum by sa[m] * sb[n].
//  * swiglu_bwd_kernel: the SwiGLU output recomputed from its input h (the
//    infra answer lists SwiGLU among the selectively recomputed operations)
//    and its derivative.
//  * gate_grad_kernel: the gates scale the experts' outputs outside any
//    GEMM, so dgate[t,k] = <dy[t], o_k[t]>; through the normalisation over
//    the chosen experts and the sigmoid this gives the router logits'
//    gradient (V3 notes §4: gates from the raw affinity; the bias only
//    selects and gets no gradient).
#include "common.h"
#include "kernels.h"

namespace dsmoe {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int TT = 128;   // rows per token tile = the promotion interval
constexpr int kXcds = 8;  // XCDs, over which a launch's blocks are dispatched round-robin

// ---------------------------------------------------------------------------
// Token tiles of each group: cho[g] = sum over g' < g of ceil(n_g' / 128)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void chunk_offsets_kernel(const int32_t* __restrict__ offsets,
                                                             int32_t G, int32_t* __restrict__ cho) {
  __shared__ int32_t s_wave[16];
  __shared__ int32_t s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    s_carry = 0;
    cho[0] = 0;
  }
  __syncthreads();
  for (int32_t g0 = 0; g0 < G; g0 += 1024) {
    const int32_t g = g0 + tid;
    int32_t n = 0;
    if (g < G) {
      const int32_t c = offsets[g + 1] - offsets[g];
      n = c > 0 ? (c + TT - 1) / TT : 0;
    }
    int32_t v = n;   // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t u = __shfl_up(v, o, 64);
      if (lane >= o) v += u;
    }
    if (lane == 63) s_wave[wave] = v;
    __syncthreads();
    int32_t base = s_carry;
    for (int w = 0; w < wave; ++w) base += s_wave[w];
    if (g < G) cho[g + 1] = base + v;
    __syncthreads();
    if (tid == 1023) s_carry = base + v;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// quant_tokens_kernel: block (t, column tile) quantises token tile t of its
// group over 128 columns.  Thread (ty, tx) holds rows ty + 16 i (i < 8) and
// columns 8 tx .. 8 tx + 7.  Per column: amax over the tile's rows (rows past
// the group's end count as 0), scale = amax / 448 (IEEE division; 1 for an
// all-zero column), codes of the IEEE quotients; the codes go through LDS so
// that each column's 128 row codes are written as one 128-byte line.
// ---------------------------------------------------------------------------
template <bool kF32>
__global__ __launch_bounds__(256) void quant_tokens_kernel(const void* __restrict__ src, int64_t C,
                                                           const int32_t* __restrict__ rows,
                                                           const float* __restrict__ row_scale,
                                                           const int32_t* __restrict__ offsets, int32_t G,
                                                           const int32_t* __restrict__ cho,
                                                           uint8_t* __restrict__ qt, float* __restrict__ st,
                                                           int64_t P, int64_t m_total) {
  __shared__ float s_red[16][TT];
  __shared__ float s_scale[TT];
  __shared__ __attribute__((aligned(16))) uint8_t s_code[TT][TT + 16];   // [column][row], padded
  const int64_t t = blockIdx.x;
  if (t >= cho[G]) return;
  int32_t lo = 0, hi = G;    // cho[lo] <= t < cho[hi]
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (cho[mid] <= t) lo = mid; else hi = mid;
  }
  const int64_t r0 = offsets[lo] + static_cast<int64_t>(TT) * (t - cho[lo]);
  // (rows past m_total are never read, whatever the offsets say)
  const int64_t r1 = min(min(r0 + TT, static_cast<int64_t>(offsets[lo + 1])), m_total);
  const int64_t c0 = static_cast<int64_t>(blockIdx.y) * TT;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;

  float v[8][8];
  float m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = r0 + ty + 16 * i;
    if (r < r1) {
      const int64_t sr = rows ? rows[r] : r;
      const int64_t idx = sr * C + c0 + 8 * tx;
      if constexpr (kF32) {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + idx);
        const f32x4 a = p[0], b = p[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[i][e] = a[e];
          v[i][4 + e] = b[e];
        }
      } else {
        const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + idx);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[i][2 * e] = __uint_as_float(w[e] << 16);
          v[i][2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
      }
      if (row_scale) {
        const float rs = row_scale[r];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] = rs * v[i][e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], fabsf(v[i][e]));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_red[ty][8 * tx + e] = m[e];
  __syncthreads();
  if (tid < TT) {
    float a = s_red[0][tid];
#pragma unroll
    for (int k = 1; k < 16; ++k) a = fmaxf(a, s_red[k][tid]);
    const float sc = a == 0.0f ? 1.0f : a / 448.0f;
    s_scale[tid] = sc;
    st[t * C + c0 + tid] = sc;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float sc = s_scale[8 * tx + e];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const uint32_t c2 = e4m3_encode2(v[i][e] / sc, v[i + 1][e] / sc);
      s_code[8 * tx + e][ty + 16 * i] = static_cast<uint8_t>(c2);
      s_code[8 * tx + e][ty + 16 * (i + 1)] = static_cast<uint8_t>(c2 >> 8);
    }
  }
  __syncthreads();
  // column c's 128 codes -> qt[(c0 + c) * P + 128 t ..]: 8 segments of 16 B
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = tid + 256 * q;
    const int c = idx >> 3, seg = idx & 7;
    *reinterpret_cast<u32x4*>(qt + (c0 + c) * P + t * TT + seg * 16) =
        *reinterpret_cast<const u32x4*>(&s_code[c][seg * 16]);
  }
}

// ---------------------------------------------------------------------------
// wgrad_kernel: c_g = A_g B_g^T over the group's token tiles.  A and B
// chunks (128 rows x 128 bytes each) and their per-row scales are loaded to
// registers one (column tile, token tile) pair ahead, stored to a
// double-buffered LDS stage, and multiplied there; each MFMA (zero
// accumulator) gives one token tile's partial sum, promoted as
// acc += P * (sa[m] * sb[n]).  A group without tokens gets zeros.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int seg) { return row * TT + ((seg ^ swz_key(row)) << 4); }

__device__ __forceinline__ i32x8 cat8(const u32x4& lo, const u32x4& hi) {
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ f32x4 mfma_chunk(const i32x8& a, const i32x8& b) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// A block owns one 128-row tile of group g's output and kWgTiles of its
// 128-column tiles, and runs the (column tile, token tile) pairs as one
// sequence: each step stages the pair's A and B chunks in LDS, issues the
// loads of the next pair, and runs its MFMAs; the last token tile of a column
// tile ends with that tile's stores.  The next pair's loads are thus in
// flight during a tile's MFMAs and stores.  Eight waves of 32 x 64 stay within
// 128 registers, so two blocks (16 waves) share a CU.  (One 4-wave block per
// output tile left every tile's load latency in front of its stores and ran at
// a third of the HBM peak; the stores alone, in the same pattern, reach the
// rate of a plain fill.)
//
// The MFMAs take the B fragment as their first operand, so a lane's four
// results of a 16 x 16 tile are four columns of one row, and B's rows are
// staged in the order that makes a lane's 16 values over its wave's four
// column fragments contiguous: LDS row 64 h + 16 j + 4 q + r holds tile
// column 64 h + 16 q + 4 j + r (the two 2-bit fields swapped).  Lane group q
// of the wave then holds columns 16 q .. 16 q + 15 of its rows and stores
// them straight from registers.
constexpr int kWgTiles = 4;
constexpr int kWgThreads = 512;

__device__ __forceinline__ int wg_col_swap(int r) {
  return (r & ~0x3C) | (((r >> 2) & 3) << 4) | (((r >> 4) & 3) << 2);
}

template <bool kF32Out>
__global__ __launch_bounds__(kWgThreads) __attribute__((amdgpu_waves_per_eu(4)))
void wgrad_kernel(const uint8_t* __restrict__ at, const float* __restrict__ sat,
                  const uint8_t* __restrict__ bt, const float* __restrict__ sbt,
                  const int32_t* __restrict__ cho, int64_t M, int64_t N, int64_t P, void* __restrict__ c,
                  int32_t pm, int32_t pn) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_ab[2][2 * TT * TT];   // per stage: A [TT][TT], B [TT][TT]
  __shared__ float s_sa[2][TT], s_sb[2][TT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;   // rows 32 wm .., columns 64 wn ..
  const int64_t mt = M / TT, nt = N / TT;
  const int64_t nblk = (nt + kWgTiles - 1) / kWgTiles;
  // (block indices and counts below 2^31: the grid is at most that)
  const int32_t bid = static_cast<int32_t>(blockIdx.x);
  const int32_t mt32 = static_cast<int32_t>(mt), nb32 = static_cast<int32_t>(nblk);
  int32_t g, mtile, nrun;
  if (pm > 0) {
    // Blocks are dispatched round-robin over the kXcds XCDs.  Every round of
    // kXcds blocks belongs to one group (the same work on every XCD), and XCD
    // x takes the part (x / pn, x % pn) of the group's pm x pn parts of
    // (row tile, column run) pairs: a row tile's A chunks are then read by pn
    // XCDs and a column run's B chunks by pm, instead of by every XCD.
    const int32_t mq = mt32 / pm, nq = nb32 / pn, per_x = mq * nq;
    const int32_t slot = bid / kXcds, x = bid % kXcds;
    g = slot / per_x;
    const int32_t j = slot - g * per_x;
    mtile = (x / pn) * mq + j / nq;
    nrun = (x % pn) * nq + j % nq;
  } else {
    g = bid / (mt32 * nb32);
    const int32_t rem = bid - g * mt32 * nb32;
    mtile = rem / nb32;
    nrun = rem % nb32;
  }
  g = __builtin_amdgcn_readfirstlane(g);
  mtile = __builtin_amdgcn_readfirstlane(mtile);
  nrun = __builtin_amdgcn_readfirstlane(nrun);
  const int64_t m0 = static_cast<int64_t>(mtile) * TT;
  const int64_t ntile0 = static_cast<int64_t>(nrun) * kWgTiles;
  const int64_t ntile1 = min<int64_t>(ntile0 + kWgTiles, nt);
  // (tiles past the P columns are never read, whatever chunk_off says)
  const int32_t t0 = cho[g], t1 = min(cho[g + 1], static_cast<int32_t>(P / TT));
  const int32_t ntt = t1 > t0 ? t1 - t0 : 0;

  const int frow = lane & 15;
  const int fq = lane >> 4;
  const size_t esz = kF32Out ? 4 : 2;
  uint8_t* cg = static_cast<uint8_t*>(c) + static_cast<size_t>(g) * M * N * esz;
  // a lane's 16 contiguous columns 64 wn + 16 fq .. of row slice i of column tile n
  auto store16 = [&](int i, int64_t n, const float (&v)[16]) {
    const int64_t row = m0 + wm * 32 + i * 16 + frow;
    const int64_t col = n * TT + wn * 64 + fq * 16;
    if constexpr (kF32Out) {
      f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(cg) + row * N + col);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    } else {
      u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(cg) + row * N + col);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = f32x2_to_bf16x2(v[8 * q + 2 * e], v[8 * q + 2 * e + 1]);
        dst[q] = w;
      }
    }
  };

  if (ntt == 0) {   // a group with no token: its weight gradient is zero
    float z[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = 0.0f;
    for (int64_t n = ntile0; n < ntile1; ++n)
#pragma unroll
      for (int i = 0; i < 2; ++i) store16(i, n, z);
    return;
  }

  // acc[i][j]: row slice i, column fragment j; lane element r is tile column
  // 64 wn + 16 fq + 4 j + r of row 32 wm + 16 i + frow
  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this thread's share of a pair's chunks: 2 segments of A and of B (row
  // idx >> 3, segment idx & 7 of the row's 128 bytes) and, for the first 256
  // threads, one scale
  u32x4 ra[2], rb[2];
  float rs = 0.f;
  // per-lane byte offsets of the loads within a 128-row block of A or B
  // (fixed over the steps: 127 rows of P bytes, far below 2^32); a step adds
  // the wave-uniform row-tile, column-tile and token-tile offsets
  uint32_t lane_off[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = tid + kWgThreads * q;
    lane_off[q] = static_cast<uint32_t>((idx >> 3) * P + (idx & 7) * 16);
  }
  const uint8_t* a_tile = at + m0 * P;
#define DSMOE_WG_LOAD(tt, n0)                                                             \
  do {                                                                                    \
    const int64_t koff = static_cast<int64_t>(tt) * TT;                                   \
    const uint8_t* abase = a_tile + koff;                                                 \
    const uint8_t* bbase = bt + (n0) * P + koff;                                          \
    _Pragma("unroll") for (int q = 0; q < 2; ++q) {                                       \
      ra[q] = *reinterpret_cast<const u32x4*>(abase + lane_off[q]);                       \
      rb[q] = *reinterpret_cast<const u32x4*>(bbase + lane_off[q]);                       \
    }                                                                                     \
    if (tid < TT)                                                                         \
      rs = sat[static_cast<int64_t>(tt) * M + m0 + tid];                                  \
    else if (tid < 2 * TT)                                                                \
      rs = sbt[static_cast<int64_t>(tt) * N + (n0) + (tid - TT)];                         \
  } while (0)

  const int fseg = fq * 2;
  const int64_t steps = (ntile1 - ntile0) * ntt;
  DSMOE_WG_LOAD(t0, ntile0 * TT);
  int64_t n = ntile0;
  int32_t tt = t0;
  for (int64_t st = 0; st < steps; ++st) {
    const int buf = static_cast<int>(st & 1);
    uint8_t* sa_ = &s_ab[buf][0];
    uint8_t* sb_ = &s_ab[buf][TT * TT];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = tid + kWgThreads * q;
      *reinterpret_cast<u32x4*>(&sa_[swz(idx >> 3, idx & 7)]) = ra[q];
      *reinterpret_cast<u32x4*>(&sb_[swz(wg_col_swap(idx >> 3), idx & 7)]) = rb[q];
    }
    if (tid < TT) s_sa[buf][tid] = rs;             // by tile row
    else if (tid < 2 * TT) s_sb[buf][tid - TT] = rs;   // by tile column
    __syncthreads();
    // the next pair: the next token tile, or the next column tile's first
    const bool tile_end = tt + 1 == t1;
    const int32_t tt_n = tile_end ? t0 : tt + 1;
    const int64_t n_n = tile_end ? n + 1 : n;
    if (st + 1 < steps) DSMOE_WG_LOAD(tt_n, n_n * TT);
    i32x8 fa[2];
    float sa[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 32 + i * 16 + frow;
      fa[i] = cat8(*reinterpret_cast<const u32x4*>(&sa_[swz(r, fseg)]),
                   *reinterpret_cast<const u32x4*>(&sa_[swz(r, fseg + 1)]));
      sa[i] = s_sa[buf][r];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 64 + j * 16 + frow;   // LDS row (staged order)
      const i32x8 fb = cat8(*reinterpret_cast<const u32x4*>(&sb_[swz(r, fseg)]),
                            *reinterpret_cast<const u32x4*>(&sb_[swz(r, fseg + 1)]));
      const f32x4 sb = *reinterpret_cast<const f32x4*>(&s_sb[buf][wn * 64 + fq * 16 + j * 4]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const f32x4 part = mfma_chunk(fb, fa[i]);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][j][q] = __builtin_fmaf(part[q], sa[i] * sb[q], acc[i][j][q]);
      }
    }
    if (tile_end) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) v[4 * j + q] = acc[i][j][q];
        store16(i, n, v);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    tt = tt_n;
    n = n_n;
  }
#undef DSMOE_WG_LOAD
}

// ---------------------------------------------------------------------------
// swiglu_bwd_kernel: per row, da = gate * da_raw (gate 1 without row_gate),
// sig = 1 / (1 + e^-g) evaluated as in the forward's epilogue,
// dh_gate = da * u * sig * (1 + g (1 - sig)), dh_up = da * g * sig, and the
// recomputed a = g * sig * u.  Four columns per thread and step.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ h, const float* __restrict__ da_raw,
                                                         const float* __restrict__ row_gate, int64_t I,
                                                         float* __restrict__ dh, float* __restrict__ a_out) {
  const int64_t r = blockIdx.x;
  const float gsc = row_gate ? row_gate[r] : 1.0f;
  const float* hr = h + r * 2 * I;
  const float* dr = da_raw + r * I;
  for (int64_t j = 4 * threadIdx.x; j < I; j += 4 * 256) {
    const f32x4 g4 = *reinterpret_cast<const f32x4*>(hr + j);
    const f32x4 u4 = *reinterpret_cast<const f32x4*>(hr + I + j);
    const f32x4 d4 = *reinterpret_cast<const f32x4*>(dr + j);
    f32x4 dg, du, a;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float g = g4[e], u = u4[e];
      const float da = gsc * d4[e];
      const float sig = __builtin_amdgcn_rcpf(1.0f + expf(-g));
      const float silu = g * sig;
      dg[e] = da * u * (sig * (1.0f + g * (1.0f - sig)));
      du[e] = da * silu;
      a[e] = silu * u;
    }
    *reinterpret_cast<f32x4*>(dh + r * 2 * I + j) = dg;
    *reinterpret_cast<f32x4*>(dh + r * 2 * I + I + j) = du;
    if (a_out) *reinterpret_cast<f32x4*>(a_out + r * I + j) = a;
  }
}

// ---------------------------------------------------------------------------
// gate_grad_kernel: one block per token.  dgate[t][k] = <dy[t], o[inv[t][k]]>
// (float32 products summed per thread over 8-column runs, then over the
// block in a fixed order); then, as in the forward's routing, s = fl32(1 / (1
// + e^-z)) evaluated in double, sum = float32 sum of the chosen s in
// selection order, gate_k = s_k / sum, and
// dlogits[t][e_k] = s_k (1 - s_k) (dgate_k - sum_j dgate_j gate_j) / sum; the
// other logits get 0.
// ---------------------------------------------------------------------------
template <bool kOF32>
__global__ __launch_bounds__(256) void gate_grad_kernel(const uint16_t* __restrict__ dy, const void* __restrict__ o,
                                                        const int32_t* __restrict__ inv,
                                                        const int32_t* __restrict__ topk,
                                                        const float* __restrict__ logits, int32_t E, int32_t K,
                                                        int64_t H, float* __restrict__ dgate,
                                                        float* __restrict__ dlogits) {
  __shared__ float s_part[4][32];
  __shared__ float s_dg[32];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int k = 0; k < K; ++k) {
    const int64_t orow = inv[t * K + k];
    float sum = 0.f;
    for (int64_t c = 8 * tid; c < H; c += 8 * 256) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(dy + t * H + c);
      float d[8], ov[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d[2 * e] = __uint_as_float(w[e] << 16);
        d[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
      if constexpr (kOF32) {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(o) + orow * H + c);
        const f32x4 a = p[0], b = p[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[e] = a[e];
          ov[4 + e] = b[e];
        }
      } else {
        const u32x4 q = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(o) + orow * H + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[2 * e] = __uint_as_float(q[e] << 16);
          ov[2 * e + 1] = __uint_as_float(q[e] & 0xFFFF0000u);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sum = __builtin_fmaf(d[e], ov[e], sum);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane == 0) s_part[wave][k] = sum;
  }
  __syncthreads();
  if (tid < K) s_dg[tid] = ((s_part[0][tid] + s_part[1][tid]) + s_part[2][tid]) + s_part[3][tid];
  for (int e = tid; e < E; e += 256) dlogits[t * E + e] = 0.f;
  __syncthreads();
  if (tid == 0) {
    float s[32];
    float tot = 0.f;
    for (int k = 0; k < K; ++k) {
      const double zd = static_cast<double>(logits[t * E + topk[t * K + k]]);
      s[k] = static_cast<float>(1.0 / (1.0 + exp(-zd)));
      tot = k == 0 ? s[k] : tot + s[k];
    }
    float mix = 0.f;
    for (int k = 0; k < K; ++k) mix = __builtin_fmaf(s_dg[k], s[k] / tot, mix);
    for (int k = 0; k < K; ++k) {
      dgate[t * K + k] = s_dg[k];
      const float ds = (s_dg[k] - mix) / tot;
      dlogits[t * E + topk[t * K + k]] = ds * s[k] * (1.0f - s[k]);
    }
  }
}

}  // namespace

int64_t token_tiles(int64_t m_total, int32_t G) { return (m_total + static_cast<int64_t>(TT - 1) * G) / TT; }

hipError_t launch_quant_tokens(const void* src, bool f32, int64_t C, const int32_t* rows, const float* row_scale,
                               const int32_t* offsets, int32_t G, int64_t m_total, int32_t* cho, uint8_t* qt,
                               float* st, hipStream_t s) {
  chunk_offsets_kernel<<<1, 1024, 0, s>>>(offsets, G, cho);
  const int64_t tiles = token_tiles(m_total, G);
  if (tiles == 0) return hipGetLastError();
  const dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(C / TT));
  const int64_t P = tiles * TT;
  if (f32)
    quant_tokens_kernel<true><<<grid, 256, 0, s>>>(src, C, rows, row_scale, offsets, G, cho, qt, st, P, m_total);
  else
    quant_tokens_kernel<false><<<grid, 256, 0, s>>>(src, C, rows, row_scale, offsets, G, cho, qt, st, P,
                                                    m_total);
  return hipGetLastError();
}

hipError_t launch_wgrad(const uint8_t* at, const float* sat, const uint8_t* bt, const float* sbt, const int32_t* cho,
                        int32_t G, int64_t M, int64_t N, int64_t P, void* c, bool f32, hipStream_t s) {
  const int64_t mt = M / TT, nblk = (N / TT + kWgTiles - 1) / kWgTiles;
  const int64_t blocks = static_cast<int64_t>(G) * mt * nblk;
  if (blocks == 0) return hipSuccess;
  // split of a group's (row tile, column run) pairs over the XCDs: pm row
  // parts x pn column parts, pm * pn = kXcds, the one that reads the fewest
  // operand bytes (pn copies of A's M rows, pm of B's N); 0 = none fits
  int32_t pm = 0, pn = 0;
  int64_t best = 0;
  for (int32_t q = 1; q <= kXcds; q *= 2) {
    const int32_t r = kXcds / q;   // q column parts, r row parts
    if (mt % r != 0 || nblk % q != 0) continue;
    const int64_t bytes = q * M + r * N;
    if (pm == 0 || bytes < best) {
      pm = r;
      pn = q;
      best = bytes;
    }
  }
  if (f32)
    wgrad_kernel<true><<<dim3(static_cast<unsigned>(blocks)), kWgThreads, 0, s>>>(at, sat, bt, sbt, cho, M, N, P, c, pm, pn);
  else
    wgrad_kernel<false><<<dim3(static_cast<unsigned>(blocks)), kWgThreads, 0, s>>>(at, sat, bt, sbt, cho, M, N, P, c, pm, pn);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float* h, const float* da_raw, const float* row_gate, int64_t rows, int64_t I,
                             float* dh, float* a_out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  swiglu_bwd_kernel<<<dim3(static_cast<unsigned>(rows)), 256, 0, s>>>(h, da_raw, row_gate, I, dh, a_out);
  return hipGetLastError();
}

hipError_t launch_gate_grad(const uint16_t* dy, const void* o, bool o_f32, const int32_t* inv, const int32_t* topk,
                            const float* logits, int64_t T, int32_t E, int32_t K, int64_t H, float* dgate,
                            float* dlogits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (o_f32)
    gate_grad_kernel<true><<<dim3(static_cast<unsigned>(T)), 256, 0, s>>>(dy, o, inv, topk, logits, E, K, H, dgate,
                                                                           dlogits);
  else
    gate_grad_kernel<false><<<dim3(static_cast<unsigned>(T)), 256, 0, s>>>(dy, o, inv, topk, logits, E, K, H, dgate,
                                                                            dlogits);
  return hipGetLastError();
}

}  // namespace dsmoe
