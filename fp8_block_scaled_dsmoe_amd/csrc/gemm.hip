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
// Two kernel shapes share the tile scheduling and the epilogues:
//
//  * gemm_lds_kernel -- groups of many rows (MFMA-bound).  Block tile 128
//    rows x BN columns, waves of 64 x 64; A and W chunks are copied straight
//    into a ring of LDS stages with gfx950's LDS DMA (global_load_lds), two
//    chunks in flight while one is multiplied.
//  * gemm_ws_kernel -- groups of few rows (HBM-bound on the weights, as in
//    prefill at T=4096 and decode).  Block tile BM rows x 256 columns, eight
//    waves of BM x 32; every wave streams its own W columns from HBM directly
//    into MFMA operand registers, several chunks ahead, so the bytes in
//    flight are not limited by LDS; only the small A tile goes through LDS.
//    BM is chosen so that one tile holds a whole group, which makes every
//    weight byte travel from HBM once.
//
// Rows of a group are gathered through a_rows (the token permute), so the
// permuted activation matrix is never materialised.  Group sizes stay on the
// device: every block derives its (group, row tile) from offsets[].  Logical
// tile order is remapped so that consecutive tiles land on the same XCD
// (blocks are dispatched round-robin over the 8 XCDs) and share its L2.
#include <type_traits>

#include "common.h"
#include "gemm.h"

namespace dsmoe {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 128;
constexpr int kXcds = 8;
constexpr int kMaxChunks = 256;   // K <= 32768

// LDS tiles hold 128-byte rows of 8 16-byte segments; segment seg of row
// `row` is stored in slot seg ^ swz_key(row).  MFMA operand reads have 16
// lanes read 16 rows (one segment each): the key is distinct over any 8
// consecutive rows and over the 8 even (8 odd) rows of a 16-row tile, so the
// reads spread over all banks whether a read cycle serves 8 or 16 lanes.
__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int seg) { return row * BK + ((seg ^ swz_key(row)) << 4); }

__device__ __forceinline__ f32x4 mfma_chunk(const i32x8& a, const i32x8& b) {
  // cbsz = blgp = 0 selects FP8 E4M3 for both operands; zero scale operands
  // select the unscaled instruction.
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 cat8(const u32x4& lo, const u32x4& hi) {
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Map a logical tile index to (group, column tile, row range).  Tiles are
// numbered group by group.  Inside a group the row tiles form bands of
// kRowBand; a band is numbered column tile by column tile, and inside a
// column tile row tile by row tile.  An XCD's run of 32 consecutive tiles is
// therefore (for a tall group) 4 row tiles x 8 column tiles, which share their
// A rows and weight tiles through that XCD's L2; with one tile per column
// (32 row tiles sharing a weight tile) every A row was fetched from HBM once
// per column tile.  Groups of at most kRowBand row tiles are one band: their
// row tiles that share a weight tile stay adjacent.  s_out gets {group, row0,
// row1, column tile}; returns false past the end.
constexpr int64_t kRowBand = 4;

// Inclusive prefix sum of a 64-bit value over the 64 lanes of a wave: within
// each row of 16 lanes by DPP shifts (row_shr 1, 2, 4, 8; a lane with no
// source lane adds 0), then the totals of the lower rows, read from lanes 15,
// 31 and 47.  (A shuffle per step through the LDS crossbar, two for 64 bits,
// took most of the tile decode's time.)
__device__ __forceinline__ int64_t wave_inclusive_scan64(int64_t v, int lane) {
  auto shr = [](int64_t x, auto ctrl) {
    const uint64_t u = static_cast<uint64_t>(x);
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u)), decltype(ctrl)::value, 0xF, 0xF, false));
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u >> 32)), decltype(ctrl)::value, 0xF, 0xF, false));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
  };
  v += shr(v, std::integral_constant<int, 0x111>{});   // row_shr:1
  v += shr(v, std::integral_constant<int, 0x112>{});   // row_shr:2
  v += shr(v, std::integral_constant<int, 0x114>{});   // row_shr:4
  v += shr(v, std::integral_constant<int, 0x118>{});   // row_shr:8
  auto lane64 = [&](int src) {
    const uint64_t u = static_cast<uint64_t>(v);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), src));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u >> 32)), src));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
  };
  const int64_t t0 = lane64(15), t1 = lane64(31), t2 = lane64(47);
  const int row = lane >> 4;
  return v + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}

template <int THREADS, int TILE_M>
__device__ bool decode_tile(const int32_t* __restrict__ offsets, int32_t G, int64_t logical,
                            int64_t n_tiles, int64_t* s_scan, int64_t* s_out) {
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
      cnt = hi > lo ? (hi - lo + TILE_M - 1) / TILE_M : 0;
    }
    // inclusive scan of the group's tile count (row tiles x column tiles)
    const int64_t mine = static_cast<int64_t>(cnt) * n_tiles;
    const int64_t v = wave_inclusive_scan64(mine, lane);
    if (lane == 63) s_scan[wave] = v;
    __syncthreads();
    int64_t wbase = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int64_t t = s_scan[w];
      if (w < wave) wbase += t;
      total += t;
    }
    const int64_t incl = carry + wbase + v;
    const int64_t excl = incl - mine;
    if (mine > 0 && logical >= excl && logical < incl) {
      const int64_t local = logical - excl;
      const int64_t band = local / (kRowBand * n_tiles);
      const int64_t in_band = local - band * kRowBand * n_tiles;
      const int64_t rows_in_band = min<int64_t>(kRowBand, cnt - band * kRowBand);
      const int64_t nt = in_band / rows_in_band;
      const int64_t r0 = lo + (band * kRowBand + in_band - nt * rows_in_band) * TILE_M;
      s_out[0] = g;
      s_out[1] = r0;
      s_out[2] = min<int64_t>(r0 + TILE_M, hi);
      s_out[3] = nt;
    }
    carry += total;
    __syncthreads();
  }
  return s_out[0] >= 0;
}

// Blocks are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8).  Logical tiles are handed out in rounds of 8 x kXcdRun: in every
// round each XCD gets a run of kXcdRun consecutive tiles.  Consecutive tiles
// (row tiles sharing a weight tile, column tiles sharing an A tile) thus share
// an XCD's L2, while the useful tiles -- a prefix of the logical range, since
// the grid is sized for the worst case -- are spread over all XCDs.  The grid
// is padded to whole rounds so that the mapping is a bijection.
constexpr int kXcdRun = 32;

__device__ __forceinline__ int64_t xcd_logical_block() {
  const int64_t bid = blockIdx.x;
  const int64_t slot = bid / kXcds;
  return (slot / kXcdRun) * (kXcds * kXcdRun) + (bid % kXcds) * kXcdRun + slot % kXcdRun;
}

inline int64_t pad_grid(int64_t blocks) {
  const int64_t round = kXcds * kXcdRun;
  return (blocks + round - 1) / round * round;
}

// ---------------------------------------------------------------------------
// Shared epilogues.  A wave holds NI x NJ accumulator tiles of 16 x 16; lane
// (i, j, r) holds local row row_base + 16i + 4*(lane/16) + r and column
// col0 + 16j + lane%16 of the output; row0 is the tile's first output row.
// ---------------------------------------------------------------------------
// Row-wise stores.  Each 16-row slice of the wave tile goes through the
// wave's own LDS scratch so that a lane then owns a run of 4*NJ contiguous
// columns of one row and writes it with 16-byte stores:
//   kStore      c[row][col] = acc
//   kGateStore  c[row][col] = acc * row_gate[row]
// The scratch rows are NCOL + 4 floats apart, so the 4-byte writes, whose
// 16-lane groups are 4 rows apart, land 16 banks apart and do not conflict.
// Rows NCOL floats apart made them 4-way conflicted.  The reads (4 lanes per
// row) go from 8-way to 2-way conflicts at 128 columns, from 4-way to none at
// 64, and stay 2-way at 32.  The 256 x 256 kernel's epilogue took 7.5 us per
// tile before.  Reading one row per lane of a 16-lane phase would remove the
// remaining read conflicts, but each quad of lanes then stores to four rows,
// and the weight-streaming kernel's down projection got 3% slower.
template <int NJ>
constexpr int epi_rows_stride() { return 16 * NJ + 4; }
template <int NJ>
constexpr int epi_rows_scratch_floats() { return 16 * epi_rows_stride<NJ>(); }

template <int NI, int NJ, Epilogue EPI>
__device__ __forceinline__ void epi_rows(const GemmProblem& p, const f32x4 (&acc)[NI][NJ],
                                         int64_t row0, int64_t row1, int row_base, int64_t col0,
                                         float* scratch) {
  constexpr int NCOL = 16 * NJ;
  constexpr int S = epi_rows_stride<NJ>();
  constexpr int PER = NCOL / 4;  // columns per lane
  const int lane = threadIdx.x & 63;
  const int64_t N = p.N;
  const int lr = lane >> 2;
  const int lc = (lane & 3) * PER;
  // the row gates of all slices are loaded first: a load between the slices'
  // stores would wait for those stores to complete (vmcnt counts both)
  [[maybe_unused]] float gate[NI];
  if constexpr (EPI == Epilogue::kGateStore) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int64_t row = row0 + row_base + i * 16 + lr;
      gate[i] = row < row1 ? p.row_gate[row] : 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        scratch[((lane >> 4) * 4 + r) * S + j * 16 + (lane & 15)] = acc[i][j][r];
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    const int64_t row = row0 + row_base + i * 16 + lr;
    float v[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) v[e] = scratch[lr * S + lc + e];
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    if (row < row1) {
      const int64_t col = col0 + lc;
      if constexpr (EPI == Epilogue::kGateStore) {
#pragma unroll
        for (int e = 0; e < PER; ++e) v[e] = v[e] * gate[i];
      }
      if (p.c_f32) {
        f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(p.c) + row * N + col);
#pragma unroll
        for (int q = 0; q < PER / 4; ++q) dst[q] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
      } else {
        u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.c) + row * N + col);
#pragma unroll
        for (int q = 0; q < PER / 8; ++q) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = f32x2_to_bf16x2(v[8 * q + 2 * e], v[8 * q + 2 * e + 1]);
          dst[q] = w;
        }
      }
    }
  }
}

// SwiGLU + 1x128 requantisation.  The block tile holds 128 gate columns and
// the matching 128 up columns.  Waves come in pairs: a gate wave holding gate
// columns [gcol, gcol + 16*NJ) of some rows and an up wave holding the same up
// columns of the same rows, with the same lane -> (row, column) map.  Each
// wave of a pair finishes half of those columns: the gate wave the first
// NJ/2 16-column slices, the up wave the rest; they swap the other half
// through LDS, indexed by (slice, lane) so that every access is a contiguous
// 16-byte-per-lane run.  a = silu(g) * u in float32, with silu(g) =
// g * rcp(1 + exp(-g)) (a few ulps, as any float32 evaluation); a row's amax
// over its 128 columns is reduced in registers (16 lanes, DPP) and across
// the NSLOTS waves that share the row through s_rmax by one thread per row,
// which also forms scale = amax / 448 (IEEE division), stores it and leaves
// it for the code pass: code = E4M3(a / scale) from the IEEE quotient, as in
// the standalone quantisers, by the hardware conversion.  The quotient's code
// comes from a * (1 / scale) and its bracket (e4m3_encode2_recip), with the
// division done only by a wave that has a value the bracket leaves unsure.
// The codes are stored with 16-byte writes.
//   s_ex:   [pairs][2][NI][NJ/2][64 lanes] f32x4
//   s_rmax: [NSLOTS][ROWS] f32
//   s_code: [ROWS][CS] bytes (CS >= 128; a padded stride spreads the byte writes of
//           rows 4 apart over more banks)
template <int NI, int NJ, int ROWS, int NSLOTS, int CS = 128>
__device__ __forceinline__ void epi_swiglu(const GemmProblem& p, const f32x4 (&acc)[NI][NJ],
                                           int64_t row0, int64_t row1, int row_base,
                                           bool is_gate, int pair, int slot, int gcol, int64_t nt,
                                           f32x4* s_ex, float* s_rmax, uint8_t* s_code) {
  constexpr int HJ = NJ / 2;
  static_assert(NJ % 2 == 0, "column slices split between the two waves of a pair");
  const int lane = threadIdx.x & 63;
  const int frow = lane & 15;
  f32x4* ex_gate = s_ex + ((pair * 2 + 0) * NI * HJ) * 64;   // gate values for the up wave
  f32x4* ex_up = s_ex + ((pair * 2 + 1) * NI * HJ) * 64;     // up values for the gate wave
  // is_gate is wave-uniform: each kind of wave runs its own fully unrolled
  // code, which indexes the accumulators with constants only (no selects)
  if (is_gate) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < HJ; ++j) ex_gate[(i * HJ + j) * 64 + lane] = acc[i][HJ + j];
  } else {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < HJ; ++j) ex_up[(i * HJ + j) * 64 + lane] = acc[i][j];
  }
  __syncthreads();
  float av[NI][HJ][4];
  const int jo = is_gate ? 0 : HJ;
  const f32x4* ex_other = is_gate ? ex_up : ex_gate;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (is_gate) {
#pragma unroll
      for (int j = 0; j < HJ; ++j) {
        const f32x4 up = ex_other[(i * HJ + j) * 64 + lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gt = acc[i][j][r];
          av[i][j][r] = gt * __builtin_amdgcn_rcpf(1.0f + expf(-gt)) * up[r];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < HJ; ++j) {
        const f32x4 gate = ex_other[(i * HJ + j) * 64 + lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gt = gate[r];
          av[i][j][r] = gt * __builtin_amdgcn_rcpf(1.0f + expf(-gt)) * acc[i][HJ + j][r];
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < HJ; ++j) m = fmaxf(m, fabsf(av[i][j][r]));
      m = row16_max_nonneg(m);
      if (frow == 0) s_rmax[slot * ROWS + row_base + i * 16 + (lane >> 4) * 4 + r] = m;
    }
  }
  __syncthreads();
  const int64_t I = p.N / 2;
  // one thread per row: the row's scale, stored and left in slot 0 of
  // s_rmax (each thread reads and writes only its own row)
  for (int lr = threadIdx.x; lr < ROWS; lr += blockDim.x) {
    float amax = s_rmax[lr];
#pragma unroll
    for (int w = 1; w < NSLOTS; ++w) amax = fmaxf(amax, s_rmax[w * ROWS + lr]);
    const float sc = amax == 0.0f ? 1.0f : amax / 448.0f;
    s_rmax[lr] = sc;
    const int64_t row = row0 + lr;
    if (row < row1) p.c_scale[row * (I / BK) + nt] = sc;
  }
  __syncthreads();
  const int ccol = gcol + jo * 16 + frow;
  // codes from the rows' reciprocals; a wave with any unsure code encodes
  // all of its values again from the IEEE quotients (rare)
  bool unsure = false;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int r = 0; r < 4; r += 2) {   // rows lr, lr + 1: one packed conversion
      const int lr = row_base + i * 16 + (lane >> 4) * 4 + r;
      const float rc0 = 1.0f / s_rmax[lr], rc1 = 1.0f / s_rmax[lr + 1];
#pragma unroll
      for (int j = 0; j < HJ; ++j) {
        const uint32_t c2 = e4m3_encode2_recip(av[i][j][r], av[i][j][r + 1], rc0, rc1, unsure);
        s_code[lr * CS + ccol + j * 16] = static_cast<uint8_t>(c2);
        s_code[(lr + 1) * CS + ccol + j * 16] = static_cast<uint8_t>(c2 >> 8);
      }
    }
  if (__builtin_amdgcn_ballot_w64(unsure) != 0) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const int lr = row_base + i * 16 + (lane >> 4) * 4 + r;
        const float sc0 = s_rmax[lr], sc1 = s_rmax[lr + 1];
#pragma unroll
        for (int j = 0; j < HJ; ++j) {
          const uint32_t c2 = e4m3_encode2(av[i][j][r] / sc0, av[i][j][r + 1] / sc1);
          s_code[lr * CS + ccol + j * 16] = static_cast<uint8_t>(c2);
          s_code[(lr + 1) * CS + ccol + j * 16] = static_cast<uint8_t>(c2 >> 8);
        }
      }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < ROWS * 8; idx += blockDim.x) {
    const int lr = idx >> 3, seg = idx & 7;
    const int64_t row = row0 + lr;
    if (row < row1)
      *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(p.c) + row * I + nt * 128 + seg * 16) =
          *reinterpret_cast<const u32x4*>(&s_code[lr * CS + seg * 16]);
  }
}

// ===========================================================================
// gemm_lds_kernel: 128-row tiles, LDS-DMA ring (groups of many rows)
// ===========================================================================
constexpr int LBM = 128;

template <int BN>
struct LdsCfg {
  static constexpr int WN = BN / 64;            // waves along N
  static constexpr int NW = 2 * WN;             // 2 waves along M
  static constexpr int THREADS = NW * 64;
  static constexpr int STAGES = BN == 256 ? 3 : 4;                 // LDS ring depth
  static constexpr int A_WLOADS = LBM * BK / 1024;                 // 1 KB wave-loads per chunk
  static constexpr int B_WLOADS = BN * BK / 1024;
  static constexpr int PER_WAVE = (A_WLOADS + B_WLOADS) / NW;      // tile wave-loads per wave
  static constexpr int LPS = PER_WAVE + 1;                         // + one for the row scales
  static constexpr int ROWS_PER_WAVE = LBM / NW;                   // scale rows per wave
  static_assert((A_WLOADS + B_WLOADS) % NW == 0, "uneven load split");
  static_assert(LPS * (STAGES - 2) < 64, "vmcnt range");
};

// Asynchronous global -> LDS copies (gfx950 LDS DMA).  Each lane moves its
// bytes to lds_base + lane * size; lds_base is wave-uniform (M0).  The data
// lands asynchronously and is counted by vmcnt like any vector load; these
// copies are issued from inline assembly so that the compiler neither waits
// for them conservatively nor counts them, and the kernel waits for them
// explicitly (vector memory operations of a wave complete in order).
__device__ __forceinline__ void dma_16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_4(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_base)
               : "memory", "m0");
}
// The same copy through a buffer resource (base and range in SGPRs): the
// per-lane byte offset voff is a 32-bit VGPR and the wave-uniform soff an
// SGPR, so a K loop can keep voff fixed and step soff, with no per-copy
// 64-bit address arithmetic on the VALU.
typedef int i32x4_rsrc __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_rsrc buffer_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_rsrc r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xffffu));   // stride 0
  r.z = -1;                        // range: every 32-bit offset
  r.w = 0x00020000;                // raw buffer, 32-bit data format
  return r;
}
__device__ __forceinline__ void dma_16_buf(const i32x4_rsrc& rsrc, uint32_t voff, uint32_t soff,
                                           uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(lds_base), "s"(soff)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_4_buf(const i32x4_rsrc& rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(lds_base)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

template <int BN, Epilogue EPI>
__global__ __launch_bounds__(2 * BN) void gemm_lds_kernel(GemmProblem p, int64_t n_tiles) {
  using C = LdsCfg<BN>;
  constexpr int THREADS = C::THREADS;
  constexpr int S = C::STAGES;
  __shared__ __attribute__((aligned(1024))) uint8_t s_a[S][LBM * BK];
  __shared__ __attribute__((aligned(1024))) uint8_t s_b[S][BN * BK];
  __shared__ __attribute__((aligned(256))) float s_sa[S][LBM];
  __shared__ float s_sw[2][kMaxChunks];   // weight-block scales of the two 128-column halves
  __shared__ int64_t s_scan[THREADS / 64];
  __shared__ int64_t s_tile[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int wm = wave / C::WN, wn = wave % C::WN;

  const int64_t logical = xcd_logical_block();
  if (!decode_tile<THREADS, LBM>(p.offsets, p.G, logical, n_tiles, s_scan, s_tile)) return;
  const int32_t g = static_cast<int32_t>(s_tile[0]);
  const int64_t nt = s_tile[3];
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

  // This wave's share of every chunk: PER_WAVE wave-loads of 1 KB (8 tile
  // rows each, lane -> row 8j + lane/8, physical segment lane%8 holding the
  // logical K segment (lane%8) ^ swz_key(row), which realises the swizzle)
  // plus the 1x128 scales of ROWS_PER_WAVE tile rows.
  const uint8_t* src[C::PER_WAVE];
  uint32_t dst_off[C::PER_WAVE];
  bool dst_is_a[C::PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::PER_WAVE; ++i) {
    const int j = wave * C::PER_WAVE + i;
    const bool is_a = j < C::A_WLOADS;
    const int jj = is_a ? j : j - C::A_WLOADS;
    const int row = jj * 8 + (lane >> 3);
    const int lseg = (lane & 7) ^ swz_key(row);
    if (is_a) {
      const int64_t r = row0 + row < row1 ? row0 + row : row0;
      const int64_t sr = p.a_rows ? p.a_rows[r] : r;
      src[i] = p.a + sr * K + lseg * 16;
    } else {
      src[i] = wbase + DSMOE_WROW(row) * K + lseg * 16;
    }
    dst_is_a[i] = is_a;
    dst_off[i] = jj * 1024;
  }
  const float* sa_src;
  {
    const int row = wave * C::ROWS_PER_WAVE + (lane < C::ROWS_PER_WAVE ? lane : 0);
    const int64_t r = row0 + row < row1 ? row0 + row : row0;
    const int64_t sr = p.a_rows ? p.a_rows[r] : r;
    sa_src = p.a_scale + sr * kchunks;
  }
  // weight-block scales for every chunk, staged once: half hb covers local
  // columns [128*hb, 128*hb + 128), which sit in one 128-row block of W
  constexpr int HALVES = BN / 128;
  for (int64_t i = tid; i < HALVES * kchunks; i += THREADS) {
    const int hb = static_cast<int>(i / kchunks);
    const int64_t c = i - hb * kchunks;
    s_sw[hb][c] = wsbase[(DSMOE_WROW(hb * 128) / BK) * kchunks + c];
  }
#undef DSMOE_WROW
  const int my_half = (wn * 64) / 128;
  __syncthreads();

  const uint32_t a_base = lds_addr(&s_a[0][0]);
  const uint32_t b_base = lds_addr(&s_b[0][0]);
  const uint32_t sa_base = lds_addr(&s_sa[0][0]) + 4 * wave * C::ROWS_PER_WAVE;
#define DSMOE_ISSUE(cc, st)                                                                  \
  do {                                                                                       \
    _Pragma("unroll") for (int i = 0; i < C::PER_WAVE; ++i) {                                \
      const uint32_t base = dst_is_a[i] ? a_base + (st) * (LBM * BK) : b_base + (st) * (BN * BK); \
      dma_16(src[i] + (cc) * BK, __builtin_amdgcn_readfirstlane(base + dst_off[i]));          \
    }                                                                                        \
    if (lane < C::ROWS_PER_WAVE)                                                             \
      dma_4(sa_src + (cc), __builtin_amdgcn_readfirstlane(sa_base + (st) * (LBM * 4)));       \
  } while (0)

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15;       // row (A) / column (B) inside a 16x16 tile
  const int fseg = (lane >> 4) * 2; // first of the two 16-byte K segments

  // prologue: stages 0 .. S-2 in flight
#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (st < kchunks) DSMOE_ISSUE(st, st);

  for (int64_t c = 0; c < kchunks; ++c) {
    const int buf = static_cast<int>(c % S);
    // chunk c has landed once at most (stages issued after it) * LPS of this
    // wave's copies are still outstanding
    const int64_t after = min<int64_t>(S - 2, kchunks - 1 - c);
    if (after >= 2)
      wait_vmcnt<2 * C::LPS>();
    else if (after == 1)
      wait_vmcnt<C::LPS>();
    else
      wait_vmcnt<0>();
    block_barrier();  // every wave's copies landed; every wave is done with chunk c-1
    if (c + S - 1 < kchunks) DSMOE_ISSUE(c + S - 1, static_cast<int>((c + S - 1) % S));
    const float sw = s_sw[my_half][c];

    // The chunk's 4 x 4 MFMA tiles run row by row: the W fragments and the
    // first A fragment are read first, then each row step issues its 4 MFMAs,
    // reads the next row's A fragment and scales, and promotes the previous
    // row, so LDS reads, MFMAs and promotions overlap; the scheduling-group
    // barriers fix that order.  Partial sums alternate between two register
    // sets by row parity (no copies).
    i32x8 bfr[4], fa[2];
    f32x4 sa4[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 64 + j * 16 + frow;
      bfr[j] = cat8(*reinterpret_cast<const u32x4*>(&s_b[buf][swz(r, fseg)]),
                    *reinterpret_cast<const u32x4*>(&s_b[buf][swz(r, fseg + 1)]));
    }
#define DSMOE_AFRAG(ii)                                                                       \
  do {                                                                                        \
    const int r_ = wm * 64 + (ii) * 16 + frow;                                                \
    fa[(ii) & 1] = cat8(*reinterpret_cast<const u32x4*>(&s_a[buf][swz(r_, fseg)]),            \
                        *reinterpret_cast<const u32x4*>(&s_a[buf][swz(r_, fseg + 1)]));       \
    sa4[(ii) & 1] = *reinterpret_cast<const f32x4*>(&s_sa[buf][wm * 64 + (ii) * 16 + (lane >> 4) * 4]); \
  } while (0)
    DSMOE_AFRAG(0);
    f32x4 part[2][4];
    float scl[2][4];
#pragma unroll
    for (int i = 0; i <= 4; ++i) {
      if (i < 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) part[i & 1][j] = mfma_chunk(fa[i & 1], bfr[j]);
#pragma unroll
        for (int r = 0; r < 4; ++r) scl[i & 1][r] = sa4[i & 1][r] * sw;
      }
      if (i + 1 < 4) DSMOE_AFRAG(i + 1);
      if (i > 0) {
        const int q = (i - 1) & 1;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i - 1][j][r] = __builtin_fmaf(part[q][j][r], scl[q][r], acc[i - 1][j][r]);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);    // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);    // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);   // VALU
      __builtin_amdgcn_sched_barrier(0);
    }
#undef DSMOE_AFRAG
  }
#undef DSMOE_ISSUE
  __syncthreads();  // all waves are done with the staging buffers (epilogues reuse them)

  if constexpr (EPI != Epilogue::kSwiGLUQuant) {
    static_assert(C::NW * epi_rows_scratch_floats<4>() * 4 <= sizeof(s_a), "epilogue scratch fits the stages");
    epi_rows<4, 4, EPI>(p, acc, row0, row1, wm * 64, nt * BN + wn * 64,
                        reinterpret_cast<float*>(&s_a[0][0]) + wave * epi_rows_scratch_floats<4>());
  } else {  // waves with wn 0,1 hold gate columns, 2,3 the matching up columns
    epi_swiglu<4, 4, LBM, 4>(p, acc, row0, row1, wm * 64, wn < 2, wm * 2 + (wn & 1), wn, (wn & 1) * 64,
                             nt, reinterpret_cast<f32x4*>(&s_b[0][0]),
                             reinterpret_cast<float*>(&s_a[0][0]), &s_a[1][0]);
  }
}

// ---------------------------------------------------------------------------
// Epilogues of the 256 x 256 kernel.  Its MFMAs take the weight fragment as
// the first operand, so a lane holds one row and four adjacent columns of
// each 16 x 16 tile, and its weight rows are staged in an order that makes
// the two tiles of a fragment pair adjacent: for row slice i and pair pp,
// lane l holds row row_base + 16 i + l % 16 and the 8 contiguous columns
// 32 pp + 8 (l / 16) + [0, 8) of the wave's 128, acc[i][2pp] the first four
// and acc[i][2pp + 1] the next four.  Both epilogues store straight from
// registers, 16 (or 8) contiguous bytes per lane, with no LDS staging.  (The
// SwiGLU epilogue's tile has its own column order: see epi_swiglu_pairs.)
// ---------------------------------------------------------------------------
//   kStore      c[row][col] = acc
//   kGateStore  c[row][col] = acc * row_gate[row]
template <Epilogue EPI>
__device__ __forceinline__ void epi_rows_lds2(const GemmProblem& p, const f32x4 (&acc)[4][8],
                                              int64_t row0, int64_t row1, int row_base, int64_t col0) {
  const int lane = threadIdx.x & 63;
  const int64_t N = p.N;
  const int64_t r_lane = row0 + row_base + (lane & 15);
  const int64_t c_lane = col0 + 8 * (lane >> 4);
  // the row gates of all slices are loaded before any store (a load issued
  // after stores would wait for them: vmcnt counts both)
  [[maybe_unused]] float gate[4];
  if constexpr (EPI == Epilogue::kGateStore) {
#pragma unroll
    for (int i = 0; i < 4; ++i) gate[i] = r_lane + 16 * i < row1 ? p.row_gate[r_lane + 16 * i] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = r_lane + 16 * i;
    if (row >= row1) continue;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      f32x4 lo = acc[i][2 * pp], hi = acc[i][2 * pp + 1];
      if constexpr (EPI == Epilogue::kGateStore) {
        lo = lo * gate[i];
        hi = hi * gate[i];
      }
      const int64_t off = row * N + c_lane + 32 * pp;
      if (p.c_f32) {
        f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(p.c) + off);
        dst[0] = lo;
        dst[1] = hi;
      } else {
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.c) + off) =
            u32x4{f32x2_to_bf16x2(lo[0], lo[1]), f32x2_to_bf16x2(lo[2], lo[3]),
                  f32x2_to_bf16x2(hi[0], hi[1]), f32x2_to_bf16x2(hi[2], hi[3])};
      }
    }
  }
}

// SwiGLU + 1x128 requantisation for the 256 x 256 kernel with gate and up
// columns paired inside each wave: wave (wm, wn) holds output columns
// [64 wn, 64 wn + 64) of the tile's 128, their gate values in fragments 0-3
// and the matching up values in fragments 4-7 (same lane, same positions),
// so a = silu(g) * u is formed in registers without any exchange.  A row's
// amax: the lane's own 16 values, then the 4 lanes that share the row
// (lanes 16 apart), then the two waves of the row band through s_rmax,
// where one thread per row forms scale = amax / 448 (IEEE division) and
// stores it.  Codes are those of the IEEE quotient a / scale: taken from
// a * (1 / scale) where a bracket proves them equal (e4m3_encode2_recip),
// re-encoded from the quotient by any wave with an unsure value.  A lane's 8
// codes of a fragment pair leave as one 8-byte store.
//   s_rmax: [2][256] f32
__device__ __forceinline__ void epi_swiglu_pairs(const GemmProblem& p, const f32x4 (&acc)[4][8],
                                                 int64_t row0, int64_t row1, int row_base, int wn,
                                                 int64_t nt, float* s_rmax) {
  constexpr int ROWS = 256;
  const int lane = threadIdx.x & 63;
  const int frow = lane & 15;
  float av[4][4][4];   // [slice][gate fragment][column]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gt = acc[i][j][r];
        av[i][j][r] = gt * __builtin_amdgcn_rcpf(1.0f + expf(-gt)) * acc[i][4 + j][r];
        m = fmaxf(m, fabsf(av[i][j][r]));
      }
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    if (lane < 16) s_rmax[wn * ROWS + row_base + i * 16 + frow] = m;
  }
  __syncthreads();
  const int64_t I = p.N / 2;
  // one thread per row: the row's scale, stored and left in s_rmax[row]
  for (int lr = threadIdx.x; lr < ROWS; lr += blockDim.x) {
    const float amax = fmaxf(s_rmax[lr], s_rmax[ROWS + lr]);
    const float sc = amax == 0.0f ? 1.0f : amax / 448.0f;
    s_rmax[lr] = sc;
    const int64_t row = row0 + lr;
    if (row < row1) p.c_scale[row * (I / BK) + nt] = sc;
  }
  __syncthreads();
  uint32_t code[4][2][2];   // [slice][fragment pair][word]
  bool unsure = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float rc = 1.0f / s_rmax[row_base + i * 16 + frow];
#pragma unroll
    for (int pl = 0; pl < 2; ++pl)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float* v = av[i][2 * pl + h];
        const uint32_t c01 = e4m3_encode2_recip(v[0], v[1], rc, rc, unsure);
        const uint32_t c23 = e4m3_encode2_recip(v[2], v[3], rc, rc, unsure);
        code[i][pl][h] = (c01 & 0xFFFFu) | (c23 << 16);
      }
  }
  if (__builtin_amdgcn_ballot_w64(unsure) != 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sc = s_rmax[row_base + i * 16 + frow];
#pragma unroll
      for (int pl = 0; pl < 2; ++pl)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float* v = av[i][2 * pl + h];
          const uint32_t c01 = e4m3_encode2(v[0] / sc, v[1] / sc);
          const uint32_t c23 = e4m3_encode2(v[2] / sc, v[3] / sc);
          code[i][pl][h] = (c01 & 0xFFFFu) | (c23 << 16);
        }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row0 + row_base + i * 16 + frow;
    if (row >= row1) continue;
#pragma unroll
    for (int pl = 0; pl < 2; ++pl) {
      uint8_t* dst = static_cast<uint8_t*>(p.c) + row * I + nt * 128 + 64 * wn + 32 * pl + 8 * (lane >> 4);
      *reinterpret_cast<uint2*>(dst) = uint2{code[i][pl][0], code[i][pl][1]};
    }
  }
}

// ===========================================================================
// gemm_lds2_kernel: 256 x 256 tiles for groups of many rows (MFMA-bound)
// ===========================================================================
// Eight waves as 4 (rows) x 2 (columns), each owning 64 rows x 128 columns
// (4 x 8 MFMA tiles, 128 accumulator registers; for SwiGLU, 64 gate and the
// matching 64 up columns).  The MFMAs take the weight
// fragment as their first operand, so a lane's four results of a tile lie in
// one row: one row scale per lane and slice promotes them, and the epilogues
// store a lane's adjacent columns straight from registers (the weight rows
// are staged in the order that makes them adjacent).  A and W chunks (32 KB each)
// come HBM -> LDS by DMA into two stages; per chunk a wave reads its 4 A
// fragments once and streams its 8 W fragments, 0.75 KB of LDS per MFMA
// (the 64 x 64 waves of the 128-row kernel read 1 KB).  The MFMAs of all
// chunks form one sequence in which each step issues one MFMA and promotes
// the one issued two steps earlier, so LDS reads, MFMAs and promotions
// overlap (see the main loop).  A wave whose 64 rows all lie past the tile's
// rows skips its copies of A, its reads, MFMAs and promotions (finer,
// per-slice guards cost the schedule its registers: the accumulators
// spilled).
constexpr int L2BM = 256;
#ifndef DSMOE_LDS2
#define DSMOE_LDS2 1
#endif
constexpr bool kUseLds2 = DSMOE_LDS2 != 0;
#ifndef DSMOE_LDS2_BUF
#define DSMOE_LDS2_BUF 1
#endif
constexpr bool kLds2Buf = DSMOE_LDS2_BUF != 0;

struct Lds2Cfg {
  static constexpr int THREADS = 512;
  static constexpr int NW = 8;
  static constexpr int BN = 256;
  static constexpr int A_WLOADS = L2BM * BK / 1024;   // 32 wave-loads of 1 KB per chunk
  static constexpr int B_WLOADS = BN * BK / 1024;     // 32
  static constexpr int PER_WAVE = (A_WLOADS + B_WLOADS) / NW;
  static constexpr int STAGE_BYTES = (L2BM + BN) * BK;
  // A's 1x128 scales are staged SA_BLOCK = 8 chunks at a time: lane l of a
  // copy takes row l / 8 (the row of the wave's A copy with the same index)
  // and chunk l % 8, so the lanes of one row read its contiguous run of
  // scales (the layout is [rows][chunks]).  One copy per chunk would read one
  // scale from each of 32 rows, 32 cache lines for 128 bytes, and such copies
  // took longer than the A and W copies together.
  static constexpr int SA_BLOCK = 8;
};

// kA32: every byte offset into A fits 32 bits (the host knows A's row
// count), so the A copies use buffer loads with per-lane offsets fixed for
// the whole K loop.
template <Epilogue EPI, bool kA32>
__global__ __launch_bounds__(512) void gemm_lds2_kernel(GemmProblem p, int64_t n_tiles) {
  using C = Lds2Cfg;
  constexpr int THREADS = C::THREADS;
  constexpr int BN = C::BN;
  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[2][C::STAGE_BYTES];   // [A | W] per stage
  __shared__ __attribute__((aligned(256))) float s_sa[2][L2BM * C::SA_BLOCK];   // [row][chunk % 8]
  __shared__ float s_sw[2][kMaxChunks];
  __shared__ int64_t s_scan[THREADS / 64];
  __shared__ int64_t s_tile[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int64_t logical = xcd_logical_block();
  if (!decode_tile<THREADS, L2BM>(p.offsets, p.G, logical, n_tiles, s_scan, s_tile)) return;
  const int32_t g = static_cast<int32_t>(s_tile[0]);
  const int64_t nt = s_tile[3];
  const int64_t row0 = s_tile[1];
  const int64_t row1 = min(s_tile[2], p.row_limit);
  if (row0 >= row1) return;

  const int64_t K = p.K, N = p.N;
  const int64_t kchunks = K / BK;
  const bool last = (p.w_last != nullptr) && (g == p.G - 1);
  const uint8_t* wbase = last ? p.w_last : p.w + static_cast<int64_t>(g) * N * K;
  const float* wsbase = last ? p.w_scale_last : p.w_scale + static_cast<int64_t>(g) * (N / BK) * kchunks;
  const int64_t w_row_base = (EPI == Epilogue::kSwiGLUQuant) ? nt * 128 : nt * BN;
  // SwiGLU: each wave holds 64 gate columns (fragments 0-3) and the matching
  // 64 up columns (fragments 4-7); see the W staging order below
  constexpr bool kPair = EPI == Epilogue::kSwiGLUQuant;
  const int64_t w_up_shift = (EPI == Epilogue::kSwiGLUQuant) ? N / 2 - 128 : 0;
#define DSMOE_WROW(lc) (w_row_base + (lc) + ((lc) >= 128 ? w_up_shift : 0))

  // Every wave copies 4 of the chunk's 32 A wave-loads and 4 of its 32 W
  // wave-loads (the A rows of wave w's copies, 32w .. 32w+31, lie in its own
  // 64-row slice, so a wave whose slice has no row of the tile skips them, as
  // it skips their scales, fragment reads and MFMAs): wave-load jj covers
  // tile rows 8jj .. 8jj+7 (lane -> row
  // 8jj + lane/8, physical segment lane%8 holding logical segment
  // (lane%8) ^ swz_key(row); swz_key(row) is (lane/8) ^ (jj & 1) for these
  // rows).  A copies keep the gathered row of each load (32-bit) and form the
  // address at issue time (kA32: the byte offset row * K + 16 * lseg, fixed
  // over the K loop); W copies are a wave-uniform row offset plus one of two
  // per-lane offsets (by the parity of jj), all through buffer resources.
  constexpr int CP = C::PER_WAVE / 2;   // A (and W) copies per wave
  static_assert(C::PER_WAVE == 8 && C::A_WLOADS == C::NW * CP && C::B_WLOADS == C::NW * CP,
                "a chunk's copies are spread over 5 + 3 MFMA steps");
  int32_t arow[CP];
#pragma unroll
  for (int i = 0; i < CP; ++i) {
    const int row = (wave * CP + i) * 8 + (lane >> 3);
    const int64_t r = row0 + row < row1 ? row0 + row : row0;
    arow[i] = static_cast<int32_t>(p.a_rows ? p.a_rows[r] : r);
    if constexpr (kA32) {
      const int lseg = (lane & 7) ^ (lane >> 3) ^ (i & 1);
      arow[i] = static_cast<int32_t>(static_cast<uint32_t>(static_cast<int64_t>(arow[i]) * K + lseg * 16));
    }
  }
  const i32x4_rsrc a_rsrc = buffer_rsrc(p.a);
  const i32x4_rsrc w_rsrc = buffer_rsrc(wbase);
  // W rows are staged in the order that the epilogues' layout needs: LDS
  // row 128 h + 16 j + m (h: the wave's column half, j: fragment, m = 4 q + r:
  // the fragment's row) holds tile column 128 h + 32 (j / 2) + 8 q + 4 (j % 2)
  // + r.  SwiGLU instead pairs gate and up inside the wave: fragment j < 4
  // holds gate column 64 h + 32 (j / 2) + 8 q + 4 (j % 2) + r of the output
  // tile and fragment j + 4 the up column at the same place.  For the 8 LDS
  // rows 8 jj + t of W wave-load jj either is a wave-uniform row plus
  // 8 (t / 4) + t % 4.
  uint32_t w_voff[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int t = lane >> 3;
    w_voff[par] = static_cast<uint32_t>((8 * (t >> 2) + (t & 3)) * K + (((lane & 7) ^ t ^ par) << 4));
  }
  const uint32_t st_base = lds_addr(&s_stage[0][0]);
  const uint32_t sa_base = lds_addr(&s_sa[0][0]);
  const i32x4_rsrc sa_rsrc = buffer_rsrc(p.a_scale);
  // Each wave also copies the scales of chunks [8 blk, 8 blk + 8) of the rows
  // of its A copies into s_sa[blk & 1] (chunks past the end repeat the last
  // one): copy i covers rows 8 (4w + i) + lane / 8, whose scale row starts
  // arow[i] * kchunks scales in (kA32: arow[i] / 128, since the byte offset
  // is row * K plus less than 128).
#define DSMOE_ISSUE_SA(blk)                                                                  \
  do {                                                                                       \
    const int ch_ = min(static_cast<int>(blk) * C::SA_BLOCK + lane % C::SA_BLOCK,            \
                        static_cast<int>(kchunks) - 1);                                      \
    if (nsl > 0) _Pragma("unroll") for (int i = 0; i < CP; ++i) {                            \
      const uint32_t ld_ = __builtin_amdgcn_readfirstlane(                                   \
          sa_base + ((blk) & 1) * (L2BM * C::SA_BLOCK * 4) + (wave * CP + i) * 256);         \
      if constexpr (kA32)                                                                    \
        dma_4_buf(sa_rsrc, ((static_cast<uint32_t>(arow[i]) >> 7) + ch_) * 4, ld_);          \
      else                                                                                   \
        dma_4(p.a_scale + static_cast<int64_t>(arow[i]) * kchunks + ch_, ld_);               \
    }                                                                                        \
  } while (0)
// copy i (of PER_WAVE: A copies 0-3, W copies 4-7) of this wave for chunk cc
// into stage st
#define DSMOE_ISSUE1(cc, st, i)                                                              \
  do {                                                                                       \
    if ((i) < CP) {                                                                          \
      if (nsl == 0) break;  /* no row of the wave's slice: its A rows are never read */      \
      const int jj = wave * CP + (i);                                                        \
      if constexpr (kA32) {                                                                  \
        dma_16_buf(a_rsrc, static_cast<uint32_t>(arow[i]),                                   \
                   __builtin_amdgcn_readfirstlane(static_cast<uint32_t>((cc) * BK)),          \
                   __builtin_amdgcn_readfirstlane(st_base + (st) * C::STAGE_BYTES + jj * 1024)); \
      } else {                                                                               \
        const int lseg = (lane & 7) ^ (lane >> 3) ^ ((i) & 1);                               \
        int32_t ar = arow[i];                                                                \
        asm volatile("" : "+v"(ar));  /* address formed here, not kept live across chunks */ \
        dma_16(p.a + static_cast<int64_t>(ar) * K + (cc) * BK + lseg * 16,                   \
               __builtin_amdgcn_readfirstlane(st_base + (st) * C::STAGE_BYTES + jj * 1024)); \
      }                                                                                      \
    } else {                                                                                 \
      const int jj = wave * CP + (i) - CP;                                                   \
      const int jf_ = (jj >> 1) & 7;                                                         \
      int64_t wr0;                                                                           \
      if constexpr (kPair) {                                                                 \
        const int oc_ = 64 * (jj >> 4) + 32 * ((jf_ >> 1) & 1) + 16 * (jj & 1) + 4 * (jf_ & 1); \
        wr0 = w_row_base + oc_ + (jf_ >= 4 ? N / 2 : 0);                                     \
      } else {                                                                               \
        const int wc_ = 128 * (jj >> 4) + 32 * (jf_ >> 1) + 16 * (jj & 1) + 4 * (jf_ & 1);    \
        wr0 = w_row_base + wc_;                                                              \
      }                                                                                      \
      dma_16_buf(w_rsrc, w_voff[(i) & 1],                                                    \
                 __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(wr0 * K + (cc) * BK)),  \
                 __builtin_amdgcn_readfirstlane(st_base + (st) * C::STAGE_BYTES + L2BM * BK + jj * 1024)); \
    }                                                                                        \
  } while (0)
#define DSMOE_ISSUE(cc, st)                                                                  \
  do {                                                                                       \
    _Pragma("unroll") for (int i_ = 0; i_ < C::PER_WAVE; ++i_) DSMOE_ISSUE1(cc, st, i_);     \
  } while (0)

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15;
  const int fseg = (lane >> 4) * 2;
  // whether any of this wave's 64 rows is a row of the tile (wave-uniform)
  const int nsl = __builtin_amdgcn_readfirstlane(static_cast<int>(row1 - row0 > wm * 64));

  // chunk 0's copies first: they need no staged scale, so their latency
  // overlaps the weight-block scale staging and its barrier
  DSMOE_ISSUE(0, 0);
  DSMOE_ISSUE_SA(0);
  for (int64_t i = tid; i < 2 * kchunks; i += THREADS) {
    const int hb = static_cast<int>(i / kchunks);
    const int64_t c = i - hb * kchunks;
    s_sw[hb][c] = wsbase[(DSMOE_WROW(hb * 128) / BK) * kchunks + c];
  }
#undef DSMOE_WROW
  __syncthreads();
  wait_vmcnt<0>();  // this wave's copies of chunk 0 landed
  block_barrier();  // everyone's did
  if (kchunks > 1) DSMOE_ISSUE(1, 1);

  // The MFMAs of all chunks form one stream: chunk c's 32 MFMAs run as
  // k = 4j + i (W fragment j, row slice i); step k issues MFMA k and
  // promotes MFMA k-2 (for k < 2 the last two of the previous chunk), whose
  // result the MFMA in between covers; partial sums rotate through four
  // register sets, so the ring lines up across chunks.  W fragment j+1 is
  // read at the start of column j.  The barrier sits after step 26, once the
  // wave has read its last fragment of the chunk's stage: past it the stage
  // is refilled with chunk c+2 while the last column's MFMAs run, and each of
  // them is followed by the read of the next chunk's fragment for the same
  // row slice (and that slice's row scales), so the next chunk starts with
  // its operands in registers instead of with every wave reading LDS at once.
  i32x8 fa[4], bf[2];
  f32x4 part[4];
  float scl[2][4];   // per row slice: the lane's row scale times the weight block's (SwiGLU: [gate, up])
  float s4n[4];
  float swn[2];
  const uint8_t* st0 = &s_stage[0][0];
#define DSMOE_RD_A(i_, stp)                                                                    \
  do {                                                                                         \
    const int r_ = wm * 64 + (i_) * 16 + frow;                                                 \
    fa[i_] = cat8(*reinterpret_cast<const u32x4*>((stp) + swz(r_, fseg)),                     \
                  *reinterpret_cast<const u32x4*>((stp) + swz(r_, fseg + 1)));                \
  } while (0)
#define DSMOE_RD_B(jj, stp)                                                                    \
  do {                                                                                         \
    const int r_ = wn * 128 + (jj) * 16 + frow;                                                \
    bf[(jj) & 1] = cat8(*reinterpret_cast<const u32x4*>((stp) + L2BM * BK + swz(r_, fseg)),   \
                        *reinterpret_cast<const u32x4*>((stp) + L2BM * BK + swz(r_, fseg + 1))); \
  } while (0)
  // the row scale of chunk cc for row slice i_ (one row per lane)
#define DSMOE_RD_S(i_, cc)                                                                     \
  do {                                                                                         \
    s4n[i_] = s_sa[((cc) / C::SA_BLOCK) & 1][(wm * 64 + (i_) * 16 + frow) * C::SA_BLOCK +     \
                                             (cc) % C::SA_BLOCK];                              \
  } while (0)
#define DSMOE_SCL(i_)                                                  \
  do {                                                                 \
    scl[0][i_] = s4n[i_] * swn[0];                                     \
    if constexpr (kPair) scl[1][i_] = s4n[i_] * swn[1];                \
  } while (0)
  // one step: MFMA k, then the promotion of MFMA k-2 (ring slot (k-2) & 3)
#define DSMOE_STEP(k, stp)                                                                     \
  do {                                                                                         \
    const int j_ = (k) >> 2, i_ = (k) & 3;                                                     \
    if (i_ == 0 && j_ + 1 < 8) DSMOE_RD_B(j_ + 1, stp);                                        \
    part[(k) & 3] = mfma_chunk(bf[j_ & 1], fa[i_]);                                            \
    const int kp_ = ((k) + 30) & 31, jp_ = kp_ >> 2, ip_ = kp_ & 3;                            \
    _Pragma("unroll") for (int rr = 0; rr < 4; ++rr)                                           \
      acc[ip_][jp_][rr] = __builtin_fmaf(part[kp_ & 3][rr], scl[kPair && jp_ >= 4][ip_], acc[ip_][jp_][rr]); \
  } while (0)
  // per step: the MFMA, then its LDS reads, then its VALU work (a step
  // has at most 6 reads and 8 VALU instructions)
#define DSMOE_SCHED()                                                  \
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   \
  __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);                   \
  __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);                   \
  __builtin_amdgcn_sched_barrier(0)

  // chunk 0's operands; the promotions of steps 0 and 1 (the previous
  // chunk's last MFMAs, of which there are none) add 0 * 0
  part[2] = part[3] = f32x4{0.f, 0.f, 0.f, 0.f};
  scl[0][2] = scl[0][3] = scl[1][2] = scl[1][3] = 0.f;
  if (nsl > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      DSMOE_RD_A(i, st0);
      DSMOE_RD_S(i, 0);
    }
    DSMOE_RD_B(0, st0);
    swn[0] = s_sw[kPair ? 0 : wn][0];
    swn[1] = s_sw[1][0];
    DSMOE_SCL(0);
    DSMOE_SCL(1);
  }

  for (int64_t c = 0; c < kchunks; ++c) {
    const int buf = static_cast<int>(c & 1);
    const uint8_t* stc = st0 + buf * C::STAGE_BYTES;          // chunk c
    const uint8_t* stn = st0 + (buf ^ 1) * C::STAGE_BYTES;    // chunk c + 1
    // Copies are spread over the MFMA steps, one per step: a wave that
    // issued all of a chunk's copies at once waited at issue for the address
    // unit, with its MFMAs queued behind them.  Chunk c+2's copies 0-4 go out
    // at steps 27-31 of chunk c and copies 5-7 at steps 0-2 of chunk c+1.
    // They are issued unconditionally (no branch in the MFMA stream) with the
    // chunk index clamped to the last chunk: a copy past the end (and chunk
    // 1's copies 5-7, which went out before the loop) rewrites a stage no
    // later step reads, or writes the same bytes again before the barrier.
    const int64_t c_prev = c + 1 < kchunks ? c + 1 : kchunks - 1;   // copies 5-7 of chunk c+1
    const int64_t c_next = c + 2 < kchunks ? c + 2 : kchunks - 1;   // copies 0-4 of chunk c+2
    if (nsl > 0) {
#pragma unroll
      for (int k = 0; k < 27; ++k) {
        DSMOE_STEP(k, stc);
        if (k == 0) DSMOE_SCL(2);   // after the promotion of the previous chunk's MFMA 30
        if (k == 1) DSMOE_SCL(3);
        if (k < C::PER_WAVE - 5) DSMOE_ISSUE1(c_prev, buf ^ 1, 5 + k);
        DSMOE_SCHED();
      }
    }
    // every wave has read its last fragment of chunk c's stage (W fragment 7,
    // step 24) and its copies of chunk c+1 have landed
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    block_barrier();
    if (c + 2 < kchunks) {
      if (nsl == 0) DSMOE_ISSUE(c + 2, buf);   // no MFMAs to spread them over
      if ((c + 2) % C::SA_BLOCK == 0) DSMOE_ISSUE_SA((c + 2) / C::SA_BLOCK);
    }
    if (nsl > 0) {
      const int64_t cw = c + 1 < kchunks ? c + 1 : c;
#pragma unroll
      for (int k = 27; k < 32; ++k) {
        DSMOE_STEP(k, stc);
        DSMOE_ISSUE1(c_next, buf, k - 27);
        if (k >= 28) {   // fa[k-28] had its last use in MFMA k
          DSMOE_RD_A(k - 28, stn);
          DSMOE_RD_S(k - 28, c + 1);
          if (k == 28) {
            DSMOE_RD_B(0, stn);
            swn[0] = s_sw[kPair ? 0 : wn][cw];
            swn[1] = s_sw[1][cw];
          }
        }
        if (k == 30) DSMOE_SCL(0);  // after the promotion of MFMA 28
        if (k == 31) DSMOE_SCL(1);
        DSMOE_SCHED();
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the copies past the end landed
  if (nsl > 0) {   // the last chunk's MFMAs 30 and 31
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      acc[2][7][rr] = __builtin_fmaf(part[2][rr], scl[kPair][2], acc[2][7][rr]);
      acc[3][7][rr] = __builtin_fmaf(part[3][rr], scl[kPair][3], acc[3][7][rr]);
    }
  }
#undef DSMOE_RD_A
#undef DSMOE_RD_B
#undef DSMOE_RD_S
#undef DSMOE_SCL
#undef DSMOE_STEP
#undef DSMOE_SCHED
#undef DSMOE_ISSUE
#undef DSMOE_ISSUE1
#undef DSMOE_ISSUE_SA
  if constexpr (EPI != Epilogue::kSwiGLUQuant) {
    epi_rows_lds2<EPI>(p, acc, row0, row1, wm * 64, nt * BN + wn * 128);
  } else {
    __syncthreads();  // all waves are done with the scale blocks (the row maxima reuse them)
    static_assert(2 * L2BM <= L2BM * C::SA_BLOCK, "the row maxima fit the scale blocks");
    epi_swiglu_pairs(p, acc, row0, row1, wm * 64, wn, nt, &s_sa[0][0]);
  }
}

// ===========================================================================
// gemm_ws_kernel: weight streaming for groups of few rows
// ===========================================================================
#ifndef DSMOE_WS_STORE_WAVES
#define DSMOE_WS_STORE_WAVES 8
#endif
constexpr int kWsStoreWaves = DSMOE_WS_STORE_WAVES;
#ifndef DSMOE_WS_WT
#define DSMOE_WS_WT 1
#endif
// Weight chunks are loaded a full 128-byte line per 8 lanes and reach the
// MFMA operand layout through a small per-wave LDS transpose (see the kernel).
constexpr bool kWsWt = DSMOE_WS_WT != 0;
#ifndef DSMOE_WS_WT_SLOTS
#define DSMOE_WS_WT_SLOTS 2
#endif

template <int BM, int NW_, bool SWIGLU>
struct WsCfg {
  static constexpr int NW = NW_;                 // waves (8, or 4 for two blocks per CU)
  static constexpr int THREADS = NW * 64;
  static constexpr int BN = NW * 32;             // 32 columns per wave
  static constexpr int HALVES = BN / 128;        // 128-column weight-scale blocks
  static constexpr int NI = BM / 16;             // row tiles per wave
  static constexpr int D = 3;                    // W chunks loaded ahead
  // A chunks are loaded A_SETS ahead.  Two sets keep the wait for the next A
  // chunk from draining the weight stream (see the main loop); small tiles
  // keep one set so that their register count allows four waves per SIMD
  // (two blocks per CU), which doubles their weight bytes in flight instead.
  static constexpr int A_SETS = (BM >= 64 && NW == 8) ? 2 : 1;
  // W register sets: with the LDS transpose a set is free once its chunk is
  // in LDS (the chunk before it is computed), so D sets keep D chunks in flight
  static constexpr int SLOTS = kWsWt ? DSMOE_WS_WT_SLOTS : D + 1;
  static constexpr int UNROLL = SLOTS % A_SETS == 0 ? SLOTS : SLOTS * A_SETS;
  static constexpr int A_SEGS = BM * 8;          // 16-byte segments of one A chunk
  static constexpr int A_PER = (A_SEGS + THREADS - 1) / THREADS;
  // LDS: two A stages + the row scales of each 128-column half during the K
  // loop; the SwiGLU epilogue reuses it for the gate/up exchange (f32), the
  // row maxima and the codes, the row-wise epilogues for one 16 x 32 f32
  // slice per wave
  // The tile's A row scales for every chunk follow ([SA_CHUNKS max][BM] f32)
  // when K allows (see the kernel).
  static constexpr int MAIN_BYTES = 2 * BM * BK + 2 * HALVES * BM * 4;
  static constexpr int SA_CHUNKS = 64;
  static constexpr int WT_BYTES = kWsWt ? NW * 32 * BK : 0;   // one chunk of 32 rows per wave
  static constexpr int K_BYTES = MAIN_BYTES + SA_CHUNKS * BM * 4 + WT_BYTES;
  static constexpr int EPI_BYTES = SWIGLU ? BM * 128 * 4 + 8 * BM * 4 + BM * 128 : 0;
  static constexpr int ROWS_BYTES = NW * epi_rows_scratch_floats<2>() * 4;
  static constexpr int MAX_A = K_BYTES > EPI_BYTES ? K_BYTES : EPI_BYTES;
  static constexpr int LDS_BYTES = MAX_A > ROWS_BYTES ? MAX_A : ROWS_BYTES;
};

template <int BM, int NW, Epilogue EPI>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(8 / NW)))
void gemm_ws_kernel(GemmProblem p, int64_t n_tiles) {
  using C = WsCfg<BM, NW, EPI == Epilogue::kSwiGLUQuant>;
  static_assert(EPI != Epilogue::kSwiGLUQuant || NW == 8, "SwiGLU tiles hold 128 gate + 128 up columns");
  constexpr int NI = C::NI;
  constexpr int SLOTS = C::SLOTS;
  constexpr int HV = C::HALVES;
  __shared__ __attribute__((aligned(1024))) uint8_t s_raw[C::LDS_BYTES];
  __shared__ float s_sw[HV][kMaxChunks];
  __shared__ int64_t s_scan[C::NW];
  __shared__ int64_t s_tile[4];
  uint8_t* s_a = s_raw;                                               // [2][BM*BK]
  // per stage and 128-column half: sa[row][chunk] * sw[half][chunk]
  float* s_scl = reinterpret_cast<float*>(s_raw + 2 * BM * BK);        // [2][HV][BM]
  float* s_sa = reinterpret_cast<float*>(s_raw + C::MAIN_BYTES);       // [kchunks][BM]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int64_t logical = xcd_logical_block();
  if (!decode_tile<C::THREADS, BM>(p.offsets, p.G, logical, n_tiles, s_scan, s_tile)) return;
  const int32_t g = static_cast<int32_t>(s_tile[0]);
  const int64_t nt = s_tile[3];
  const int64_t row0 = s_tile[1];
  const int64_t row1 = min(s_tile[2], p.row_limit);
  if (row0 >= row1) return;

  const int64_t K = p.K, N = p.N;
  const int64_t kchunks = K / BK;
  const bool last = (p.w_last != nullptr) && (g == p.G - 1);
  const uint8_t* wbase = last ? p.w_last : p.w + static_cast<int64_t>(g) * N * K;
  const float* wsbase = last ? p.w_scale_last : p.w_scale + static_cast<int64_t>(g) * (N / BK) * kchunks;
  const int64_t w_row_base = (EPI == Epilogue::kSwiGLUQuant) ? nt * 128 : nt * C::BN;
  const int64_t w_up_shift = (EPI == Epilogue::kSwiGLUQuant) ? N / 2 - 128 : 0;
#define DSMOE_WROW(lc) (w_row_base + (lc) + ((lc) >= 128 ? w_up_shift : 0))

  // this wave's W columns: local [32*wave, 32*wave + 32), two 16-column
  // tiles; lane reads row 16j + lane%16, bytes 16g .. 16g+15 and 64+16g ..
  // 64+16g+15 of a chunk, g = lane/16.  (The MFMA sums over its 128 K slots in
  // any order, so any split of the chunk's bytes over the four lane groups
  // works when A uses the same one.  With this split each 16-byte load
  // instruction covers one contiguous 64-byte half of each of its 16 rows'
  // 128-byte lines, so a chunk costs one request per half line; splitting
  // into 32-byte runs per group made each instruction touch both halves.)
  const uint8_t* wsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    wsrc[j] = wbase + DSMOE_WROW(wave * 32 + j * 16 + (lane & 15)) * K + (lane >> 4) * 16;
  // Transposed path: load q (0..3) of a chunk reads rows 8q .. 8q+7 of the
  // wave's 32, a whole 128-byte line per 8 lanes (lane: row 8q + lane/8, bytes
  // 16*(lane%8)); byte offsets within the group's weight matrix (< 2^32).
  // The wave writes the chunk to its LDS area, 16-byte piece s of local row
  // 8q + rb at piece slot s ^ f(rb, q), f = (rb >> 1) | ((q & 1) << 2): with
  // it both the writes (lanes 16k..16k+15: two rows x 8 pieces) and the
  // fragment reads (16 rows, one piece) hit 16 different 4-bank groups.
  // (A wave's 32 rows lie in one half of the SwiGLU column layout, so load q
  // is load 0 moved by the uniform 8q rows.  The other LDS addresses follow
  // from one per lane: q odd adds 1 KB and flips bit 2 of the piece slot,
  // i.e. address bit 6, which is 0 in the rest of the address; piece g + 4
  // likewise differs from piece g in that bit alone; q + 2 and j + 1 are 2 KB
  // further.)
  uint32_t woff0 = 0;
  int wt_w0 = 0, wt_r0 = 0;
  if constexpr (kWsWt) {
    woff0 = static_cast<uint32_t>(DSMOE_WROW(wave * 32 + (lane >> 3)) * K + (lane & 7) * 16);
    const int rbw = lane >> 3, sw_ = lane & 7;
    wt_w0 = wave * 32 * BK + rbw * 128 + ((sw_ ^ (rbw >> 1)) * 16);
    const int rbr = lane & 7, qpr = (lane & 15) >> 3, g = lane >> 4;
    wt_r0 = wave * 32 * BK + qpr * 1024 + rbr * 128 + ((g ^ ((rbr >> 1) | (qpr << 2))) * 16);
  }
  // A: BM rows x 8 segments per chunk, A_PER segments per thread
  const uint8_t* asrc[C::A_PER];
  int adst[C::A_PER];
  bool aval[C::A_PER];
#pragma unroll
  for (int i = 0; i < C::A_PER; ++i) {
    const int idx = tid + C::THREADS * i;
    aval[i] = idx < C::A_SEGS;
    const int lr = aval[i] ? idx >> 3 : 0, seg = idx & 7;
    const int64_t r = row0 + lr < row1 ? row0 + lr : row0;
    const int64_t sr = p.a_rows ? p.a_rows[r] : r;
    asrc[i] = p.a + sr * K + seg * 16;
    adst[i] = swz(lr, seg);
  }
  // (threads past the tile load a valid row too: the loads stay unconditional,
  // which keeps the rotating register sets free of merge copies)
  const float* sasrc;
  {
    const int lr = tid < BM ? tid : 0;
    const int64_t r = row0 + lr < row1 ? row0 + lr : row0;
    const int64_t sr = p.a_rows ? p.a_rows[r] : r;
    sasrc = p.a_scale + sr * kchunks;
  }
  for (int64_t i = tid; i < HV * kchunks; i += C::THREADS) {
    const int hb = static_cast<int>(i / kchunks);
    const int64_t c = i - hb * kchunks;
    s_sw[hb][c] = wsbase[(DSMOE_WROW(hb * 128) / BK) * kchunks + c];
  }
  const int my_half = (wave * 32) / 128;
#undef DSMOE_WROW

  // The tile's A row scales for all chunks, staged once into LDS (16 lanes
  // per row, 16-byte loads) instead of one scattered 4-byte load per row per
  // chunk; needs K <= 64 chunks, a multiple of 4 chunks, and a 16-byte
  // aligned scale buffer (uniform, else the per-chunk loads stay).
  const bool stage_sa = kchunks <= C::SA_CHUNKS && (kchunks & 3) == 0 &&
                        (reinterpret_cast<uintptr_t>(p.a_scale) & 15) == 0;
  // (loaded here, stored to LDS after the prologue's loads are issued, so
  // that the wait for them does not wait for the weight chunks)
  constexpr int SA_PASSES = (BM + C::THREADS / 16 - 1) / (C::THREADS / 16);
  f32x4 sv[SA_PASSES];
  if (stage_sa) {
#pragma unroll
    for (int q = 0; q < SA_PASSES; ++q) {
      const int lr = q * (C::THREADS / 16) + (tid >> 4), part = tid & 15;
      sv[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (lr < BM && part * 4 < kchunks) {
        const int64_t r = row0 + lr < row1 ? row0 + lr : row0;
        const int64_t sr = p.a_rows ? p.a_rows[r] : r;
        sv[q] = *reinterpret_cast<const f32x4*>(p.a_scale + sr * kchunks + part * 4);
      }
    }
  }

  // Register sets: W chunks rotate through SLOTS sets (D ahead), A chunks
  // through A_SETS sets.  Loads of a wave complete in order, so the wait for
  // A(c+1) before it is stored to LDS at the end of iteration c also waits for
  // every load issued before it.  With two A sets, A(c+1) was issued in
  // iteration c-1, right after W(c+1), and W(c+2), W(c+3) stay in flight
  // across the barrier; with one set it was issued in iteration c, after
  // W(c+2), and only W(c+3) does.
  constexpr int AS = C::A_SETS;
  u32x4 wr[SLOTS][2][2];   // transposed path: [slot][q >> 1][q & 1] = load q
  u32x4 ra[AS][C::A_PER];
  float rsa[AS];
  uint8_t* s_w = s_raw + C::MAIN_BYTES + C::SA_CHUNKS * BM * 4;
#define DSMOE_WLOAD(cc, slot)                                                                \
  do {                                                                                       \
    if constexpr (kWsWt) {                                                                   \
      _Pragma("unroll") for (int q = 0; q < 4; ++q)                                          \
        wr[slot][q >> 1][q & 1] =                                                            \
            *reinterpret_cast<const u32x4*>(wbase + (cc) * BK + q * 8 * K + woff0);          \
    } else {                                                                                 \
      _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                        \
        wr[slot][j][0] = *reinterpret_cast<const u32x4*>(wsrc[j] + (cc) * BK);               \
        wr[slot][j][1] = *reinterpret_cast<const u32x4*>(wsrc[j] + (cc) * BK + 64);          \
      }                                                                                      \
    }                                                                                        \
  } while (0)
  // (A_SEGS and BM are multiples of 64, so whether a thread's segment i or
  // row scale exists is the same for its whole wave: waves skip the loads
  // they do not use)
#define DSMOE_ALOAD(cc, set)                                                                 \
  do {                                                                                       \
    _Pragma("unroll") for (int i = 0; i < C::A_PER; ++i)                                     \
      if (C::THREADS * i + wave * 64 < C::A_SEGS)                                            \
        ra[set][i] = *reinterpret_cast<const u32x4*>(asrc[i] + (cc) * BK);                   \
    if (!stage_sa && wave * 64 < BM) rsa[set] = sasrc[(cc)];                                 \
  } while (0)
#define DSMOE_ASTORE(bb, set, cc)                                                            \
  do {                                                                                       \
    _Pragma("unroll") for (int i = 0; i < C::A_PER; ++i) if (aval[i])                       \
        *reinterpret_cast<u32x4*>(&s_a[(bb) * BM * BK + adst[i]]) = ra[set][i];              \
    if (tid < BM) {                                                                          \
      const float as_ = stage_sa ? s_sa[(cc) * BM + tid] : rsa[set];                         \
      _Pragma("unroll") for (int h = 0; h < HV; ++h)                                         \
        s_scl[((bb) * HV + h) * BM + tid] = as_ * s_sw[h][(cc)];                             \
    }                                                                                        \
  } while (0)

  f32x4 acc[NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15;
  const int fseg = lane >> 4;   // the A fragment takes 16-byte segments fseg and fseg + 4

  // prologue: A chunks 0 .. AS-1 and W chunks 0 .. D-1 in flight; A chunk 0
  // staged (the weight-block scales were staged above)
  DSMOE_ALOAD(0, 0);
  DSMOE_WLOAD(0, 0);
  if constexpr (AS == 2) DSMOE_ALOAD(min<int64_t>(1, kchunks - 1), 1);
#pragma unroll
  for (int d = 1; d < (kWsWt ? SLOTS : C::D); ++d) DSMOE_WLOAD(min<int64_t>(d, kchunks - 1), d);
  if (stage_sa) {
#pragma unroll
    for (int q = 0; q < SA_PASSES; ++q) {
      const int lr = q * (C::THREADS / 16) + (tid >> 4), part = tid & 15;
      if (lr < BM && part * 4 < kchunks)
#pragma unroll
        for (int e = 0; e < 4; ++e) s_sa[(part * 4 + e) * BM + lr] = sv[q][e];
    }
  }
  __syncthreads();
  DSMOE_ASTORE(0, 0, 0);
  __syncthreads();

  // 16-row slices of the tile that hold rows (wave-uniform); the MFMAs,
  // operand reads and promotions of the slices past them are skipped
  const int nti = __builtin_amdgcn_readfirstlane(static_cast<int>((row1 - row0 + 15) / 16));
  // The first kFixed slices, which the typical group of this tile height
  // (about 8/11 of BM rows) fills, run without guards: a guarded step starts
  // a basic block, at whose entry the compiler waits conservatively, and the
  // unguarded steps take about a fifth fewer cycles.  Slices past a group's
  // rows compute on clamped valid rows that the epilogue never stores.
  constexpr int kFixed = (BM * 8 / 11) / 16 > 1 ? (BM * 8 / 11) / 16 : 1;
  static_assert(C::UNROLL % AS == 0 && C::UNROLL % SLOTS == 0, "register sets follow the chunk index");
  for (int64_t c0 = 0; c0 < kchunks; c0 += C::UNROLL) {
#pragma unroll
    for (int u = 0; u < C::UNROLL; ++u) {
      const int64_t c = c0 + u;
      const int64_t cn = min<int64_t>(c + 1, kchunks - 1);
      // loads are issued unconditionally (clamped to the last chunk) so every
      // register set is written on every path; set u % AS held A(c), which
      // is in LDS already.  The A load goes first: the wait for A(c+1) at the
      // end of the iteration then leaves the later weight chunks in flight.
      DSMOE_ALOAD(min<int64_t>(c + AS, kchunks - 1), u % AS);
      i32x8 b0, b1;
      if constexpr (kWsWt) {
        // W(c) (set u % SLOTS) to this wave's LDS area, then that set takes
        // W(c + SLOTS); the fragments come back in the MFMA layout
        const int sl = u % SLOTS;
        if (c < kchunks) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<u32x4*>(s_w + ((q & 1) ? ((wt_w0 + 1024) ^ 64) : wt_w0) + (q >> 1) * 2048) =
                wr[sl][q >> 1][q & 1];
        }
        DSMOE_WLOAD(min<int64_t>(c + SLOTS, kchunks - 1), sl);
        if (c < kchunks) {
          const int wt_r1 = wt_r0 ^ 64;
          b0 = cat8(*reinterpret_cast<const u32x4*>(s_w + wt_r0),
                    *reinterpret_cast<const u32x4*>(s_w + wt_r1));
          b1 = cat8(*reinterpret_cast<const u32x4*>(s_w + wt_r0 + 2048),
                    *reinterpret_cast<const u32x4*>(s_w + wt_r1 + 2048));
        }
      } else {
        DSMOE_WLOAD(min<int64_t>(c + C::D, kchunks - 1), (u + C::D) % SLOTS);
        b0 = cat8(wr[u % SLOTS][0][0], wr[u % SLOTS][0][1]);
        b1 = cat8(wr[u % SLOTS][1][0], wr[u % SLOTS][1][1]);
      }
      if (c < kchunks) {
        const int buf = static_cast<int>(c & 1);
        const float* scl = s_scl + (buf * HV + my_half) * BM + (lane >> 4) * 4;
        // Software pipeline over the row tiles: the LDS operands of tile i+1
        // are requested before the MFMAs of tile i are issued, and tile i-1
        // is promoted after them.  Operands, partial sums and scales rotate
        // through register sets indexed by the (unrolled) tile number, so no
        // copies are needed; the scheduling barriers keep the compiler from
        // hoisting every tile's operands at once (register pressure).
        i32x8 fa[2];
        f32x4 pr[2][2], ps[3];
#define DSMOE_FRAG(ii)                                                                          \
  do {                                                                                          \
    const int r_ = (ii) * 16 + frow;                                                            \
    fa[(ii) & 1] = cat8(*reinterpret_cast<const u32x4*>(&s_a[buf * BM * BK + swz(r_, fseg)]),   \
                        *reinterpret_cast<const u32x4*>(&s_a[buf * BM * BK + swz(r_, fseg + 4)])); \
    ps[(ii) % 3] = *reinterpret_cast<const f32x4*>(scl + (ii) * 16);                           \
  } while (0)
        DSMOE_FRAG(0);
#pragma unroll
        for (int i = 0; i <= NI; ++i) {
          // slices at or past max(nti, kFixed) are skipped: step nti only
          // promotes slice nti-1, later steps do nothing (wave-uniform
          // branches)
          if (i < NI && (i < kFixed || i < nti)) {
            if (i + 1 < NI) DSMOE_FRAG(i + 1);
            pr[i & 1][0] = mfma_chunk(fa[i & 1], b0);
            pr[i & 1][1] = mfma_chunk(fa[i & 1], b1);
          }
          if (i > 0 && (i <= kFixed || i <= nti)) {
            const int q = (i - 1) & 1, qs = (i - 1) % 3;
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) {
              acc[i - 1][0][r2] = __builtin_fmaf(pr[q][0][r2], ps[qs][r2], acc[i - 1][0][r2]);
              acc[i - 1][1][r2] = __builtin_fmaf(pr[q][1][r2], ps[qs][r2], acc[i - 1][1][r2]);
            }
            // pin the promotion here (otherwise it is sunk to the loop end and
            // every tile's partial sums stay live at once)
            asm volatile("" : "+v"(acc[i - 1][0]), "+v"(acc[i - 1][1]));
          }
          // issue order inside the step: the MFMAs of tile i (operands read
          // one step earlier), the LDS reads of tile i+1, then the promotion
          // of tile i-1 (its MFMAs were issued one step earlier)
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // LDS reads
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // VALU
          __builtin_amdgcn_sched_barrier(0);
        }
#undef DSMOE_FRAG
      }
      DSMOE_ASTORE(static_cast<int>((c + 1) & 1), (u + 1) % AS, cn);
      __syncthreads();
    }
  }
#undef DSMOE_WLOAD
#undef DSMOE_ALOAD
#undef DSMOE_ASTORE

  if constexpr (EPI != Epilogue::kSwiGLUQuant) {
    epi_rows<NI, 2, EPI>(p, acc, row0, row1, 0, nt * C::BN + wave * 32,
                         reinterpret_cast<float*>(s_raw) + wave * epi_rows_scratch_floats<2>());
  } else {  // waves 0-3 hold gate columns 32w.., waves 4-7 the matching up columns (pairs w, w+4)
    epi_swiglu<NI, 2, BM, 8>(p, acc, row0, row1, 0, wave < 4, wave & 3, wave, (wave & 3) * 32, nt,
                             reinterpret_cast<f32x4*>(s_raw),
                             reinterpret_cast<float*>(s_raw + BM * 128 * 4),
                             s_raw + BM * 128 * 4 + 8 * BM * 4);
  }
}

// ---------------------------------------------------------------------------
template <int BN, Epilogue EPI>
hipError_t launch_lds(const GemmProblem& p, hipStream_t s) {
  const int64_t n_tiles = (EPI == Epilogue::kSwiGLUQuant) ? (p.N / 2) / 128 : p.N / BN;
  const int64_t blocks = pad_grid(((p.M_total + LBM - 1) / LBM + p.G) * n_tiles);
  if (blocks == 0) return hipSuccess;
  gemm_lds_kernel<BN, EPI><<<dim3(static_cast<unsigned>(blocks)), LdsCfg<BN>::THREADS, 0, s>>>(p, n_tiles);
  return hipGetLastError();
}

template <Epilogue EPI>
hipError_t launch_lds2(const GemmProblem& p, hipStream_t s) {
  const int64_t n_tiles = (EPI == Epilogue::kSwiGLUQuant) ? (p.N / 2) / 128 : p.N / Lds2Cfg::BN;
  const int64_t blocks = pad_grid(((p.M_total + L2BM - 1) / L2BM + p.G) * n_tiles);
  if (blocks == 0) return hipSuccess;
  // 32-bit A offsets when A's size is known and every row's K bytes fit
  const bool a32 = kLds2Buf && p.a_rows_total > 0 && p.a_rows_total * p.K <= 0xFFFFFFFFLL;
  if (a32)
    gemm_lds2_kernel<EPI, true><<<dim3(static_cast<unsigned>(blocks)), Lds2Cfg::THREADS, 0, s>>>(p, n_tiles);
  else
    gemm_lds2_kernel<EPI, false><<<dim3(static_cast<unsigned>(blocks)), Lds2Cfg::THREADS, 0, s>>>(p, n_tiles);
  return hipGetLastError();
}

template <int BM, Epilogue EPI>
hipError_t launch_ws(const GemmProblem& p, hipStream_t s) {
  constexpr int NW = (EPI == Epilogue::kSwiGLUQuant) ? 8 : kWsStoreWaves;
  const int64_t n_tiles = (EPI == Epilogue::kSwiGLUQuant) ? (p.N / 2) / 128 : p.N / (NW * 32);
  const int64_t blocks = pad_grid(((p.M_total + BM - 1) / BM + p.G) * n_tiles);
  if (blocks == 0) return hipSuccess;
  gemm_ws_kernel<BM, NW, EPI><<<dim3(static_cast<unsigned>(blocks)), NW * 64, 0, s>>>(p, n_tiles);
  return hipGetLastError();
}

template <Epilogue EPI>
hipError_t launch_ws_bm(const GemmProblem& p, int bm, hipStream_t s) {
  switch (bm) {
    case 16: return launch_ws<16, EPI>(p, s);
    case 32: return launch_ws<32, EPI>(p, s);
    case 64: return launch_ws<64, EPI>(p, s);
    case 96: return launch_ws<96, EPI>(p, s);
    case 128: return launch_ws<128, EPI>(p, s);
    case 160: return launch_ws<160, EPI>(p, s);
    case 176: return launch_ws<176, EPI>(p, s);
    default: return launch_ws<192, EPI>(p, s);
  }
}

// y[t][n] = o[shared0 + t][n] (when there is a shared expert) + sum over k,
// ascending, of o[inv[t][k]][n]; float32 sums, 8 columns per thread read with
// 16-byte loads (two for float32 rows).  Every row of o is read once and y is
// written once, so both go through nontemporal loads and stores (on 32768
// tokens of the V3 shapes, 4.2 GB of o, 8% faster than cached accesses).
template <bool kF32>
__device__ __forceinline__ void load_row8(const void* __restrict__ o, int64_t off, float (&v)[8]) {
  if (kF32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(o) + off);
    const f32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  } else {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(o) + off));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
}

// KT > 0: K == KT known at compile time (8, the V3 top-K); the K row indices
// and then all K rows are loaded before the sums, which keep their order.
// With a runtime K each row waited for its index and then for itself.
template <bool kF32, int KT>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ o,
                                                      const int32_t* __restrict__ inv, int64_t T,
                                                      int32_t K, int64_t H, int64_t shared0,
                                                      void* __restrict__ y) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per_row = H / 8;
  if (idx >= T * per_row) return;
  const int64_t t = idx / per_row;
  const int64_t c0 = (idx - t * per_row) * 8;
  const int32_t* inv_t = inv + t * K;
  float v[8];
  if constexpr (KT > 0) {
    int32_t r[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) r[k] = inv_t[k];
    float u[KT][8];
#pragma unroll
    for (int k = 0; k < KT; ++k) load_row8<kF32>(o, static_cast<int64_t>(r[k]) * H + c0, u[k]);
    int k0 = 0;
    if (shared0 >= 0) {
      load_row8<kF32>(o, (shared0 + t) * H + c0, v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = u[0][e];
      k0 = 1;
    }
#pragma unroll
    for (int k = 0; k < KT; ++k)
      if (k >= k0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = v[e] + u[k][e];
      }
  } else {
    int k0 = 0;
    if (shared0 >= 0) {
      load_row8<kF32>(o, (shared0 + t) * H + c0, v);
    } else {
      load_row8<kF32>(o, static_cast<int64_t>(inv_t[0]) * H + c0, v);
      k0 = 1;
    }
    for (int k = k0; k < K; ++k) {
      float u[8];
      load_row8<kF32>(o, static_cast<int64_t>(inv_t[k]) * H + c0, u);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = v[e] + u[e];
    }
  }
  if (kF32) {
    f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(y) + t * H + c0);
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, dst);
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, dst + 1);
  } else {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = f32x2_to_bf16x2(v[2 * e], v[2 * e + 1]);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + t * H + c0));
  }
}

}  // namespace

hipError_t launch_combine(const void* o, const int32_t* inv, int64_t T, int32_t K, int64_t H,
                          int64_t shared0, void* y, bool f32, hipStream_t s) {
  const int64_t threads = T * (H / 8);
  if (threads == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (K == 8) {
    if (f32)
      combine_kernel<true, 8><<<grid, 256, 0, s>>>(o, inv, T, K, H, shared0, y);
    else
      combine_kernel<false, 8><<<grid, 256, 0, s>>>(o, inv, T, K, H, shared0, y);
  } else {
    if (f32)
      combine_kernel<true, 0><<<grid, 256, 0, s>>>(o, inv, T, K, H, shared0, y);
    else
      combine_kernel<false, 0><<<grid, 256, 0, s>>>(o, inv, T, K, H, shared0, y);
  }
  return hipGetLastError();
}

// Row-tile height of the weight-streaming kernel for groups of about
// `rows_hint` rows (0: use an LDS kernel).  The height is the mean group size
// plus 3/8 (room for the spread: a group past it takes a second tile, which
// streams the group's weights again; the 16-row slices a tile does not use
// cost no MFMA work).  With 128 rows per expert this gives 176-row tiles,
// 2% faster than 160 (a quarter) and than 192.  Taller groups go to the LDS
// kernels, whose tiles reuse each staged weight chunk over more rows.
int ws_tile_rows(int64_t rows_hint) {
  const int64_t want = rows_hint * 11 / 8;
  for (int bm : {16, 32, 64, 96, 128, 160, 176, 192})
    if (want <= bm) return bm;
  return 0;
}

hipError_t launch_grouped_gemm(const GemmProblem& p, hipStream_t s) {
  if (p.M_total == 0) return hipSuccess;
  const bool wide = p.N % 256 == 0;   // 256-column tiles (8 waves) when N allows
  const int bm = (wide || p.epi == Epilogue::kSwiGLUQuant) ? ws_tile_rows(p.rows_hint) : 0;
  if (bm > 0) {
    switch (p.epi) {
      case Epilogue::kStore: return launch_ws_bm<Epilogue::kStore>(p, bm, s);
      case Epilogue::kGateStore: return launch_ws_bm<Epilogue::kGateStore>(p, bm, s);
      case Epilogue::kSwiGLUQuant: return launch_ws_bm<Epilogue::kSwiGLUQuant>(p, bm, s);
    }
  }
  // (the 256 x 256 kernel addresses a weight matrix with 32-bit offsets)
  if (kUseLds2 && wide && p.N * p.K <= 0xFFFFFFFFLL) {
    switch (p.epi) {
      case Epilogue::kStore: return launch_lds2<Epilogue::kStore>(p, s);
      case Epilogue::kGateStore: return launch_lds2<Epilogue::kGateStore>(p, s);
      case Epilogue::kSwiGLUQuant: return launch_lds2<Epilogue::kSwiGLUQuant>(p, s);
    }
  }
  switch (p.epi) {
    case Epilogue::kStore:
      return wide ? launch_lds<256, Epilogue::kStore>(p, s) : launch_lds<128, Epilogue::kStore>(p, s);
    case Epilogue::kGateStore:
      return wide ? launch_lds<256, Epilogue::kGateStore>(p, s)
                  : launch_lds<128, Epilogue::kGateStore>(p, s);
    case Epilogue::kSwiGLUQuant:
      return launch_lds<256, Epilogue::kSwiGLUQuant>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dsmoe
