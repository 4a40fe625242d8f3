// Internal launchers of the dsmoe kernels.  Called by the C ABI layer after
// it has validated every argument; each returns hipSuccess or the launch
// error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"

namespace dsmoe {

// quant.hip
hipError_t launch_quant_act(const void* x, bool x_f32, int64_t rows, int64_t cols, uint8_t* q,
                            float* scale, hipStream_t s);
hipError_t launch_quant_w(const void* w, bool w_f32, int64_t n_mats, int64_t n, int64_t k,
                          uint8_t* q, float* scale, hipStream_t s);
// unit-scale E4M3 codes of n floats; hw selects the packed hardware conversion
hipError_t launch_e4m3_codes(const float* x, int64_t n, bool hw, uint8_t* q, hipStream_t s);
// codes [n_mats][n][k] + 128x128 scales -> codes [n_mats][k][n] + scales of W^T
hipError_t launch_transpose_w(const uint8_t* q, const float* s, int64_t n_mats, int64_t n, int64_t k,
                              uint8_t* qt, float* st, hipStream_t stream);

// granularity.hip
int64_t quant_rows_max_cols();
// one scale per row over the whole row; cols % 8 == 0, cols <= quant_rows_max_cols()
hipError_t launch_quant_rows(const void* x, bool x_f32, int64_t rows, int64_t cols, uint8_t* q,
                             float* scale, hipStream_t s);
// one scale for n elements (n % 8 == 0); amax_scratch holds
// quant_tensor_scratch_floats() floats, max |x| in element 0 afterwards
int64_t quant_tensor_scratch_floats();
hipError_t launch_quant_tensor(const void* x, bool x_f32, int64_t n, uint8_t* q, float* scale,
                               float* amax_scratch, hipStream_t s);
hipError_t launch_prep_offsets(int32_t* offsets, int32_t m, hipStream_t s);
// dst[r][t] = src ? src[r * src_stride] : 1 for r < rows, t < tiles
hipError_t launch_broadcast_scale(float* dst, int64_t rows, int64_t tiles, const float* src,
                                  int64_t src_stride, hipStream_t s);
// c[m][n] *= col[n], float32 c [M][N], N % 4 == 0
hipError_t launch_scale_cols(float* c, int64_t m, int64_t n, const float* col, hipStream_t s);

// serving.hip
// replica plan: slot_first [E+1], slot_expert [E + n_extra]; E <= 1024
hipError_t launch_plan_replicas(const int32_t* counts, int32_t E, int32_t n_extra, int32_t* slot_first,
                                int32_t* slot_expert, hipStream_t s);
// group offsets of the S slots (+ the shared group when extra_rows >= 0): phys [S+2]
hipError_t launch_slot_offsets(const int32_t* offsets, int32_t E, const int32_t* slot_first,
                               const int32_t* slot_expert, int32_t S, int64_t extra_rows, int32_t* phys,
                               hipStream_t s);
// w_slots[s] = w[slot_expert[s]] ([N][K] codes and [N/128][K/128] scales)
hipError_t launch_place_slots(const uint8_t* w, const float* w_scale, int32_t E, int64_t n, int64_t k,
                              const int32_t* slot_expert, int32_t S, uint8_t* w_slots, float* s_slots,
                              hipStream_t s);
hipError_t launch_fill_f32(float* dst, int64_t n, float v, hipStream_t s);

// route.hip
// H is split over router_splits() blocks for small T; the splits' partial
// sums go to `partial` (router_partial_bytes(), NULL when that is 0)
int router_splits(int64_t T, int64_t H, int32_t E);
size_t router_partial_bytes(int64_t T, int64_t H, int32_t E);
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, int64_t T, int64_t H,
                                int32_t E, float* logits, float* partial, hipStream_t s);
// topk/gates + per-expert counts (counts are zeroed first by the launcher)
hipError_t launch_route_select(const float* logits, const float* bias, int64_t T, int32_t E,
                               int32_t G, int32_t Mg, int32_t K, int32_t* topk_idx,
                               float* gates, int32_t* counts, hipStream_t s);
// offsets from counts; perm/inv (and, when given, per-row gates and the
// identity extension of perm for `extra_rows` trailing rows)
hipError_t launch_permute(const int32_t* topk_idx, const float* gates, int64_t T, int32_t E,
                          int32_t K, const int32_t* counts, int32_t* offsets, int32_t* perm,
                          int32_t* inv, float* row_gate, int32_t* offsets_ext,
                          hipStream_t s);
hipError_t launch_update_bias(float* bias, const int32_t* counts, int32_t E, int64_t T,
                              int32_t K, float gamma, hipStream_t s);

// backward.hip
// upper bound on the 128-row token tiles of m_total rows in G groups
int64_t token_tiles(int64_t m_total, int32_t G);
// chunk offsets cho [G+1] of the groups, then codes qt [C][P] and scales st
// [P/128][C] of the 1x128 tiles along each group's rows, P = 128 * token_tiles
hipError_t launch_quant_tokens(const void* src, bool f32, int64_t C, const int32_t* rows, const float* row_scale,
                               const int32_t* offsets, int32_t G, int64_t m_total, int32_t* cho, uint8_t* qt,
                               float* st, hipStream_t s);
// c[g] [M][N] (f32 or bf16) = A_g B_g^T over group g's token tiles
hipError_t launch_wgrad(const uint8_t* at, const float* sat, const uint8_t* bt, const float* sbt, const int32_t* cho,
                        int32_t G, int64_t M, int64_t N, int64_t P, void* c, bool f32, hipStream_t s);
hipError_t launch_swiglu_bwd(const float* h, const float* da_raw, const float* row_gate, int64_t rows, int64_t I,
                             float* dh, float* a_out, hipStream_t s);
hipError_t launch_gate_grad(const uint16_t* dy, const void* o, bool o_f32, const int32_t* inv, const int32_t* topk,
                            const float* logits, int64_t T, int32_t E, int32_t K, int64_t H, float* dgate,
                            float* dlogits, hipStream_t s);

}  // namespace dsmoe
