/*
 * dsmoe.h -- C ABI of a DeepSeekMoE FFN layer forward on the fine-grained
 * FP8 recipe, for AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (cited by page and section):
 *   "V3 notes"      xutianle.me, "DeepSeek-V3 技术报告：从 671B MoE 到低成本训练系统"
 *   "infra answer"  51itzy.com DeepSeek-V3 Q&A page, the answer written from
 *                   the infrastructure point of view (FP8 and routing paragraphs)
 *   "evolution"     the "deepseek-evolution" blog post, V3 sections
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument except `stream` and the host-side descriptor
 *   structs is a DEVICE pointer.  The caller owns all memory; the library
 *   never allocates or frees, and keeps no mutable global state.
 * - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *   NULL is the default stream) and never synchronises the host.
 * - Arguments are validated on the host before anything is enqueued.  On a
 *   validation failure the call returns a non-zero status and launches
 *   nothing.  A failed launch returns DSMOE_ERR_LAUNCH.  Faults inside a
 *   kernel surface at the caller's next synchronisation.
 * - Sizes of 0 rows / tokens are valid and enqueue nothing (status OK).
 * - Alignment: FP8 code, bf16 and output matrices must be 16-byte aligned;
 *   float and int32 arrays 4-byte aligned.  Row lengths that are multiples
 *   of 128 keep every row 16-byte aligned.
 * - Values: the library computes on finite inputs; NaN/Inf inputs give
 *   unspecified (but memory-safe) results.  No flush of float32 subnormals.
 * - FP8 is OCP E4M3FN (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 *   no infinities, max 448), the format the pages prescribe for every FP8
 *   tensor (infra answer, FP8 paragraph; V3 notes §6).  Codes are stored as
 *   uint8.
 * - Calls on different streams with disjoint output buffers may overlap.
 */
#ifndef DSMOE_H
#define DSMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsmoe_status {
  DSMOE_OK = 0,
  DSMOE_ERR_NULL = 1,      /* a required pointer is NULL */
  DSMOE_ERR_SHAPE = 2,     /* a size is out of range or not a multiple of 128 */
  DSMOE_ERR_ALIGN = 3,     /* a pointer is not aligned as required */
  DSMOE_ERR_DTYPE = 4,     /* unknown dtype code */
  DSMOE_ERR_WORKSPACE = 5, /* workspace missing or smaller than required */
  DSMOE_ERR_DEVICE = 6,    /* no usable device, or it is not gfx950 */
  DSMOE_ERR_LAUNCH = 7     /* a kernel launch failed (hipGetLastError) */
} dsmoe_status;

typedef enum dsmoe_dtype {
  DSMOE_BF16 = 0,          /* bfloat16, stored as uint16 */
  DSMOE_F32 = 1            /* IEEE binary32 */
} dsmoe_dtype;

/* Static string naming a status code ("DSMOE_OK", ...); never NULL. */
const char* dsmoe_status_str(int status);

/* Version of this ABI (incremented on incompatible changes). */
int dsmoe_abi_version(void);

/* Limits checked by the calls below. */
#define DSMOE_MAX_EXPERTS 1024
#define DSMOE_MAX_GROUPS 64
#define DSMOE_MAX_TOPK 32

/*
 * dsmoe_quant_act_1x128 -- fine-grained activation quantisation.
 * Source: V3 notes §6.1 (activations scaled per 1x128 tile: one scale per
 * token per 128 channels, computed online from the current tensor); infra
 * answer, FP8 paragraph ("per-tile 1x128").
 *
 *   x      [rows][cols] row-major, dtype xt (DSMOE_BF16 or DSMOE_F32)
 *   q      [rows][cols] uint8 E4M3FN codes (output)
 *   scale  [rows][cols/128] float32 (output)
 *
 * For every row r and tile j: amax = max |x[r][128j .. 128j+127]| (exact),
 * s = fl32(amax / 448) by IEEE float32 division (s = 1 when amax = 0),
 * q = E4M3(fl32(x / s)) by IEEE float32 division, rounding to nearest with
 * ties to even, saturating at +-448, keeping the sign of zero.
 * Requires cols % 128 == 0, rows >= 0.
 */
dsmoe_status dsmoe_quant_act_1x128(const void* x, int xt, int64_t rows, int64_t cols,
                                   uint8_t* q, float* scale, void* stream);

/*
 * dsmoe_quant_w_128x128 -- fine-grained weight quantisation.
 * Source: V3 notes §6.1 (weights scaled per 128x128 block, online); infra
 * answer, FP8 paragraph ("per-group 128x128").
 *
 *   w      [n_mats][N][K] row-major (N = output channels, K = input
 *          channels), dtype wt (DSMOE_BF16 or DSMOE_F32)
 *   q      [n_mats][N][K] uint8 E4M3FN codes (output)
 *   scale  [n_mats][N/128][K/128] float32 (output)
 *
 * The same rule as dsmoe_quant_act_1x128 with amax taken over each 128x128
 * block.  Requires N % 128 == 0, K % 128 == 0, n_mats >= 0.
 */
dsmoe_status dsmoe_quant_w_128x128(const void* w, int wt, int64_t n_mats, int64_t N, int64_t K,
                                   uint8_t* q, float* scale, void* stream);

/*
 * dsmoe_e4m3_codes -- E4M3FN codes of floats taken as already scaled (scale
 * 1), with either of the two encoders the kernels use.  Source: V3 notes §6
 * and infra answer, FP8 paragraph (E4M3 for every FP8 tensor); the rounding
 * rule is that of dsmoe_quant_act_1x128.
 *
 *   x          [n] float32
 *   converter  0: the integer encoder of the quantisers; 1: gfx950's packed
 *              conversion with the inputs clamped to +-448 first (the SwiGLU
 *              epilogue's).  Both round to nearest with ties to even,
 *              saturate at +-448 and keep the sign of zero; NaN inputs have
 *              no defined code.
 *   q          [n] uint8 codes (output)
 * Requires n >= 0; a converter other than 0 or 1 gives DSMOE_ERR_DTYPE.
 */
dsmoe_status dsmoe_e4m3_codes(const float* x, int64_t n, int converter, uint8_t* q, void* stream);

/*
 * dsmoe_transpose_w_128x128 -- the weight operand of a data-gradient GEMM.
 * Source: V3 notes §6 (the activation-gradient GEMM runs in FP8 like the
 * forward) and §6.1 (128x128 weight blocks).  A block's amax does not change
 * under transposition, so W^T's codes and block scales are W's, moved:
 *
 *   q      [n_mats][N][K] codes, s [n_mats][N/128][K/128] float32 (as from
 *          dsmoe_quant_w_128x128)
 *   qt     [n_mats][K][N] codes (output), st [n_mats][K/128][N/128] (output);
 *          must not overlap the inputs
 *
 * With qt/st as the weight, dsmoe_fp8_grouped_gemm computes dA = dC . W (the
 * gradient of c = A W^T with respect to A) from the 1x128 codes of dC.
 * Requires N, K positive multiples of 128, n_mats >= 0.
 */
dsmoe_status dsmoe_transpose_w_128x128(const uint8_t* q, const float* s, int64_t n_mats, int64_t N,
                                       int64_t K, uint8_t* qt, float* st, void* stream);

/*
 * dsmoe_route -- auxiliary-loss-free, group-limited top-K routing and the
 * token permute.
 * Source: V3 notes §4 (top-K chosen on s + b, gate weights from the raw
 * affinity s), §4.2 (each token limited to experts on at most 4 nodes, no
 * token dropping), §2 (8 of 256 routed experts per token); infra answer,
 * routing paragraph (group routing to at most 4 nodes).
 *
 *   logits   [T][E] float32 router logits z
 *   bias     [E] float32 per-expert bias b (read only)
 *   topk_idx [T][K] int32 (output) chosen experts, in the order
 *            (key descending, expert index ascending)
 *   gates    [T][K] float32 (output) s_k / sum of s over the chosen experts,
 *            summed in float32 in the order of topk_idx
 *   counts   [E] int32 (output) tokens routed to each expert
 *   offsets  [E+1] int32 (output) exclusive prefix sum of counts
 *   perm     [T*K] int32 (output) row -> token; rows grouped by expert in
 *            ascending expert order, tokens ascending within an expert
 *   inv      [T][K] int32 (output) (token, k) -> row of perm
 *
 * s = fl32(sigmoid(z)) evaluated in float64; key = fl32(s + b); the E experts
 * form G contiguous groups; a group's score is the float32 sum (largest first)
 * of its ceil(K/Mg) largest keys; the Mg best groups are kept under (score
 * descending, group index ascending); the K best experts of the kept groups
 * are chosen under (key descending, index ascending).  Deterministic.
 * Requires 1 <= E <= DSMOE_MAX_EXPERTS, 1 <= G <= DSMOE_MAX_GROUPS, E % G == 0,
 * 1 <= Mg <= G, 1 <= K <= min(DSMOE_MAX_TOPK, Mg*E/G), T*K < 2^31.
 */
dsmoe_status dsmoe_route(const float* logits, const float* bias, int64_t T, int32_t E,
                         int32_t G, int32_t Mg, int32_t K, int32_t* topk_idx, float* gates,
                         int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                         void* stream);

/*
 * dsmoe_fp8_grouped_gemm -- block-scaled FP8 GEMM over groups of rows, with
 * the partial sum of every 128-wide K chunk promoted to float32.
 * Source: V3 notes §6.2 (partial sums promoted to FP32 every 128 FP8
 * products), §6 (FP8 GEMM inputs, BF16/FP32 outputs), §6.1 (scale layouts);
 * evolution, FP8 section.
 *
 *   a        [*][K] uint8 E4M3FN codes, a_scale [*][K/128] float32
 *   a_rows   [M_total] int32 or NULL: output row r reads A row a_rows[r]
 *            (NULL: A row r)
 *   offsets  [G+1] int32 on the device: group g owns output rows
 *            offsets[g] .. offsets[g+1]-1; offsets[0] = 0, non-decreasing,
 *            offsets[G] <= M_total (rows past offsets[G] are left untouched)
 *   w        [G][N][K] uint8 codes (W_g^T layout: output channel major),
 *   w_scale  [G][N/128][K/128] float32
 *   c        [M_total][N] (output), dtype ct (DSMOE_BF16 rounds to nearest
 *            even, DSMOE_F32)
 *
 * c[r][n] = sum over chunks j of a_scale[ar][j] * w_scale[g][n/128][j] *
 * (sum over k in chunk j of a[ar][k] * w[g][n][k]), ar = a_rows ? a_rows[r] : r.
 * G = 1 with offsets = {0, M} is the dense GEMM.  The group sizes are read
 * on the device; the host never synchronises.
 * Requires N % 128 == 0, K % 128 == 0, K <= 32768, 1 <= G, M_total >= 0.
 */
dsmoe_status dsmoe_fp8_grouped_gemm(const uint8_t* a, const float* a_scale,
                                    const int32_t* a_rows, const int32_t* offsets, int32_t G,
                                    int64_t M_total, const uint8_t* w, const float* w_scale,
                                    int64_t N, int64_t K, void* c, int ct, void* stream);

/*
 * Layer description.  Source: V3 notes §2 (one shared expert, 256 routed
 * experts of intermediate size 2048, 8 chosen) and §4.2 (at most 4 of 8
 * nodes).  H hidden size, I expert intermediate size (both multiples of
 * 128, at most 32768), E routed experts in G groups, Mg groups kept, K experts chosen,
 * n_shared shared experts (0 or 1; intermediate size I, gate 1).
 */
typedef struct dsmoe_moe_desc {
  int64_t H, I;
  int32_t E, G, Mg, K, n_shared;
} dsmoe_moe_desc;

/*
 * Layer weights (device pointers, read only), quantised with
 * dsmoe_quant_w_128x128:
 *   w13     [E][2I][H] codes, s13 [E][2I/128][H/128]: rows 0..I-1 of an
 *           expert are the gate projection, rows I..2I-1 the up projection
 *   w2      [E][H][I] codes,  s2  [E][H/128][I/128]: down projection
 *   w13_sh, s13_sh, w2_sh, s2_sh: the shared expert, same layouts (one
 *           matrix each); ignored when n_shared == 0
 *   router_w [E][H] bf16: the router is kept in high precision, not FP8
 *           (V3 notes §6: sensitive / cheap modules stay in higher precision)
 */
typedef struct dsmoe_moe_weights {
  const uint8_t* w13;
  const float* s13;
  const uint8_t* w2;
  const float* s2;
  const uint8_t* w13_sh;
  const float* s13_sh;
  const uint8_t* w2_sh;
  const float* s2_sh;
  const void* router_w;
} dsmoe_moe_weights;

/*
 * Optional device buffers that receive the layer's intermediates (each
 * pointer may be NULL):  qx [T][H] and sx [T][H/128] (the 1x128 codes of x),
 * logits [T][E], topk_idx and gates [T][K], offsets [E+1], perm [T*K],
 * inv [T][K], and the down projections' FP8 input: qa [T*K + n_shared*T][I]
 * codes and sa [T*K + n_shared*T][I/128] scales of the requantised SwiGLU
 * output a (V3 notes §6.1), one row per (token, routed expert) pair in the
 * order of perm (row inv[t][k] is token t's k-th expert), then, with a
 * shared expert, row T*K + t for token t.
 * stage_events (host array, may be NULL): hipEvent_t handles (passed as
 * void*) created by the caller, recorded on the stream.  dsmoe_moe_forward
 * takes DSMOE_STAGE_EVENTS of them: event 0 before the first kernel and
 * event i after stage i: 1 quantise x, 2 router logits, 3 top-K selection,
 * 4 permute, 5 gate/up GEMM + SwiGLU + requant, 6 routed down GEMM,
 * 7 shared down GEMM + combine.  dsmoe_moe_forward_serving takes
 * DSMOE_SERVING_STAGE_EVENTS (see there).  Recording them changes no result.
 */
#define DSMOE_STAGE_EVENTS 8
typedef struct dsmoe_moe_debug {
  uint8_t* qx;
  float* sx;
  float* logits;
  int32_t* topk_idx;
  float* gates;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  void* const* stage_events;
  uint8_t* qa;
  float* sa;
} dsmoe_moe_debug;

/* Bytes of device workspace dsmoe_moe_forward needs for T tokens
 * (0 if the description is invalid). */
size_t dsmoe_moe_workspace_bytes(const dsmoe_moe_desc* d, int64_t T);

/*
 * dsmoe_moe_forward -- the DeepSeekMoE FFN layer forward on FP8.
 * Source: V3 notes §2 (layer structure; the output is the shared expert's
 * output plus the gate-weighted outputs of the chosen routed experts), §4
 * and §4.2 (routing), §6 / §6.1 / §6.2 (FP8 recipe); infra answer (SwiGLU
 * as the expert activation).
 *
 *   d, w       host pointers to the description and weight table
 *   bias       [E] float32 routing bias (read only; see dsmoe_update_bias)
 *   x          [T][H] bf16 layer input
 *   y          [T][H] output, dtype yt (DSMOE_BF16 or DSMOE_F32)
 *   counts_out [E] int32 per-expert token counts of this call (required:
 *              it is what dsmoe_update_bias consumes)
 *   workspace  device buffer of at least dsmoe_moe_workspace_bytes(d, T)
 *              bytes, 256-byte aligned; contents on entry are ignored
 *   dbg        host pointer to a dsmoe_moe_debug or NULL
 *
 * Steps: x is quantised per 1x128 tile; logits = x . router_w^T (bf16
 * inputs, float32 accumulation); routing as dsmoe_route; every (token,
 * expert) pair runs h = x W13^T (block-scaled FP8 GEMM, promoted per 128),
 * a = silu(h_gate) * h_up in float32, a re-quantised per 1x128 tile,
 * o = a W2^T (block-scaled FP8 GEMM) scaled by the gate; the shared expert
 * runs the same FFN on every token with gate 1; y[t] = o_shared[t] + sum over
 * k of o[t, k], summed in float32 in a fixed order, then rounded to yt.
 * No residual add.  Deterministic: two calls with the same inputs give
 * identical bits.
 */
dsmoe_status dsmoe_moe_forward(const dsmoe_moe_desc* d, const dsmoe_moe_weights* w,
                               const float* bias, const void* x, int64_t T, void* y, int yt,
                               int32_t* counts_out, void* workspace, size_t ws_bytes,
                               const dsmoe_moe_debug* dbg, void* stream);

/*
 * dsmoe_moe_forward_noalloc -- dsmoe_moe_forward without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The forward's scratch is a device array inside the library of
 * DSMOE_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held until the process
 * ends; it covers the DeepSeek-V3 shapes (H 7168, I 2048, E 256, K 8) up to
 * T = 256 tokens (dsmoe_moe_workspace_bytes gives the need of a call).
 * Arguments and results as in dsmoe_moe_forward.  Returns
 * DSMOE_ERR_WORKSPACE, with nothing enqueued, when the call needs more than
 * that.  The call allocates nothing.  Every call on a GPU shares that GPU's
 * array (the forward reads no scratch content it did not write in the same
 * call): calls that overlap on one GPU (on different streams, or from
 * several threads) race and must be serialised by the caller.
 */
#define DSMOE_NOALLOC_SCRATCH_BYTES (80ull << 20)
dsmoe_status dsmoe_moe_forward_noalloc(const dsmoe_moe_desc* d, const dsmoe_moe_weights* w,
                                       const float* bias, const void* x, int64_t T, void* y, int yt,
                                       int32_t* counts_out, const dsmoe_moe_debug* dbg, void* stream);

/*
 * dsmoe_update_bias -- auxiliary-loss-free bias update.
 * Source: V3 notes §4 (after each step an overloaded expert's bias is
 * lowered and an underloaded expert's raised), §4.1 (speed gamma = 0.001);
 * evolution, load-balancing section.
 *
 *   bias    [E] float32, updated in place:
 *           b[e] = fl32(b[e] + fl32(gamma) * sign(T*K - E*counts[e])),
 *           sign(0) = 0 (mean load T*K/E compared with counts exactly)
 *   counts  [E] int32 loads of the step (e.g. counts_out of the forward)
 * Requires 1 <= E <= DSMOE_MAX_EXPERTS, T >= 0, K >= 1.
 */
dsmoe_status dsmoe_update_bias(float* bias, const int32_t* counts, int32_t E, int64_t T,
                               int32_t K, float gamma, void* stream);

/*
 * Decode-serving variant.  Source: V3 notes §8, the deployment section (in
 * decode the shared expert is a routed expert that every token takes, so a
 * token uses 9 experts; some GPUs hold the shared expert and redundant
 * copies of experts; the experts that run hot in live traffic are copied
 * periodically, chosen from loads observed online, and the placement is
 * adjusted); infra answer, inference paragraph (decode over 256 experts plus
 * 64 copies of hot ones).  The pages fix neither how many copies an expert
 * gets nor how a token picks a copy: the two rules below are this library's
 * readings.
 *
 * A "slot" is one physical copy of a routed expert's weights.  The slots of
 * one expert are consecutive: expert e owns slots slot_first[e] ..
 * slot_first[e+1]-1 of S = slot_first[E], and slot_expert[s] names the
 * expert of slot s.
 */

/*
 * dsmoe_plan_replicas -- slots from observed loads.
 *   counts       [E] int32 loads (e.g. counts_out of an earlier forward)
 *   n_extra      slots beyond one per expert: S = E + n_extra
 *   slot_first   [E+1] int32 (output)
 *   slot_expert  [E + n_extra] int32 (output)
 * Each extra slot goes, one at a time, to the expert with the largest load
 * per slot counts[e] / n_e (compared exactly as integers; the lowest index
 * wins ties), which minimises max_e counts[e] / n_e.  One wave on the device.
 * Requires 1 <= E <= DSMOE_MAX_EXPERTS, 0 <= n_extra <= DSMOE_MAX_EXPERTS,
 * counts >= 0.
 */
dsmoe_status dsmoe_plan_replicas(const int32_t* counts, int32_t E, int32_t n_extra,
                                 int32_t* slot_first, int32_t* slot_expert, void* stream);

/*
 * dsmoe_place_replicas -- fill slot weights: w_slots[s] = w[slot_expert[s]].
 *   w            [E][N][K] codes, w_scale [E][N/128][K/128] float32 (the
 *                layouts of dsmoe_quant_w_128x128)
 *   E            experts in w
 *   slot_expert  [n_slots] int32, each in [0, E); a slot naming anything
 *                else is left unwritten (checked on the device)
 *   w_slots      [n_slots][N][K] codes, s_slots [n_slots][N/128][K/128]
 *                (outputs; must not overlap the inputs)
 * Call it for W13 and for W2 whenever the plan changes.  Requires N, K
 * positive multiples of 128, 0 <= n_slots <= 65535.
 */
dsmoe_status dsmoe_place_replicas(const uint8_t* w, const float* w_scale, int32_t E, int64_t N,
                                  int64_t K, const int32_t* slot_expert, int32_t n_slots,
                                  uint8_t* w_slots, float* s_slots, void* stream);

/*
 * dsmoe_slot_offsets -- group offsets of the slots.
 *   offsets      [E+1] int32 group offsets of the experts (e.g. from
 *                dsmoe_route)
 *   slot_first   [E+1], slot_expert [n_slots] int32: a plan
 *   extra_rows   >= 0: rows of one more group after the routed rows (the
 *                shared expert's), else -1
 *   phys         [n_slots + 2] int32 (output): phys[s] for s < n_slots, then
 *                phys[n_slots] = offsets[E] and, when extra_rows >= 0,
 *                phys[n_slots + 1] = offsets[E] + extra_rows
 * Slot slot_first[e] + j of expert e starts at row offsets[e] +
 * floor(j * (offsets[e+1] - offsets[e]) / n_e): contiguous chunks that
 * differ by at most one row.  Requires 1 <= E <= DSMOE_MAX_EXPERTS,
 * E <= n_slots <= E + DSMOE_MAX_EXPERTS.
 */
dsmoe_status dsmoe_slot_offsets(const int32_t* offsets, int32_t E, const int32_t* slot_first,
                                const int32_t* slot_expert, int32_t n_slots, int64_t extra_rows,
                                int32_t* phys, void* stream);

#define DSMOE_SERVING_STAGE_EVENTS 5

/* Workspace of dsmoe_moe_forward_serving (0 for an invalid description). */
size_t dsmoe_moe_serving_workspace_bytes(const dsmoe_moe_desc* d, int64_t T, int32_t n_slots);

/*
 * dsmoe_moe_forward_serving -- the layer forward over slots.
 *   w            as in dsmoe_moe_forward, except that w13/s13/w2/s2 hold the
 *                n_slots slots ([S][2I][H] codes, ...), filled by
 *                dsmoe_place_replicas from the per-expert weights
 *   slot_first   [E+1], slot_expert [n_slots] int32: the plan the slots were
 *                placed with (slot_first[E] must equal n_slots)
 *   dbg          NULL, or a dsmoe_moe_debug whose buffers receive the same
 *                intermediates as in dsmoe_moe_forward (qa/sa in the same
 *                row order: the slots only refine the group offsets); its
 *                stage_events, if given, are DSMOE_SERVING_STAGE_EVENTS
 *                handles recorded at the start, after the permute, after the
 *                gate/up launch, after the down launch and after the combine
 *   everything else as in dsmoe_moe_forward
 * Routing, gates and counts_out (per expert) are those of dsmoe_moe_forward.
 * The rows of expert e (its tokens, ascending) are cut into its n_e slots in
 * contiguous chunks: slot slot_first[e] + j starts at row offsets[e] +
 * floor(j * c_e / n_e).  With n_shared = 1 the shared expert runs as one more
 * routed group, gate 1, in both GEMM launches (K + 1 experts per token).  y
 * equals dsmoe_moe_forward's up to the float32 rounding of the GEMM tiles the
 * launches pick (the same parity bar).  A plan that is not one (an expert
 * index out of range, a slot outside its expert's range) gives unspecified
 * results but no access outside the buffers.
 * Requires E <= n_slots <= E + DSMOE_MAX_EXPERTS and the limits of
 * dsmoe_moe_forward.
 */
dsmoe_status dsmoe_moe_forward_serving(const dsmoe_moe_desc* d, const dsmoe_moe_weights* w,
                                       const int32_t* slot_first, const int32_t* slot_expert,
                                       int32_t n_slots, const float* bias, const void* x, int64_t T,
                                       void* y, int yt, int32_t* counts_out, void* workspace,
                                       size_t ws_bytes, const dsmoe_moe_debug* dbg, void* stream);

/*
 * The rest of the FP8 backward of the expert FFN.  Source: V3 notes §6 (the
 * Fprop, Dgrad and Wgrad GEMMs of every Linear in FP8 E4M3, outputs BF16 or
 * FP32; 1x128 tiles for activations, 128x128 blocks for weights; partial
 * sums promoted to FP32 every 128 products, §6.1, §6.2); infra answer,
 * memory paragraph (SwiGLU is recomputed in the backward); V3 notes §4
 * (gates from the raw affinity, the bias only selects).  The pages do not
 * orient the gradient tiles: here every FP8 operand is tiled 1x128 along its
 * GEMM's contraction axis, so the weight-gradient GEMMs, which contract over
 * an expert's tokens, take both operands in tiles of 128 consecutive rows of
 * the expert's group.
 */

/* Upper bound on the 128-row token tiles of M_total rows in G groups
 * (sum over groups of ceil(n_g / 128)); sizes the buffers below. */
int64_t dsmoe_token_tiles(int64_t M_total, int32_t G);

/*
 * dsmoe_quant_tokens_128 -- 1x128 tiles along the rows of each group.
 *   src        [n_src][C] bf16 or f32 (src_type), row-major, C % 128 == 0
 *   rows       [M_total] int32 source row of each output row (NULL: row r
 *              is src row r), each in [0, n_src)
 *   row_scale  [M_total] f32 or NULL: row r is fl32(row_scale[r] * src)
 *              (e.g. the gate of the down projection's output gradient)
 *   offsets    [G+1] int32 on the device: group g holds rows offsets[g] ..
 *              offsets[g+1]-1 (nondecreasing, offsets[G] <= M_total)
 *   chunk_off  [G+1] int32 (output): first tile of each group, the
 *              exclusive scan of ceil(n_g / 128)
 *   qt         [C][P] codes (output), P = 128 * dsmoe_token_tiles(M_total, G):
 *              tile j of group g, column c is qt[c][128 (chunk_off[g] + j) ..
 *              + 127], row by row; rows past the group's end are code 0
 *   scales     [P/128][C] f32 (output): scales[chunk_off[g] + j][c]
 * Per tile and column: amax over its rows, scale = fl32(amax / 448) (1 for
 * an all-zero column), codes E4M3 of the IEEE quotients, round to nearest
 * even, saturating.  Columns of qt past the used tiles are not written.
 * Requires 1 <= G <= 65536, M_total >= 0, C > 0.
 */
dsmoe_status dsmoe_quant_tokens_128(const void* src, int src_type, int64_t n_src, int64_t C,
                                    const int32_t* rows, const float* row_scale, const int32_t* offsets,
                                    int32_t G, int64_t M_total, int32_t* chunk_off, uint8_t* qt,
                                    float* scales, void* stream);

/*
 * dsmoe_fp8_wgrad_grouped -- weight-gradient GEMM of every group.
 *   at, sa     [M][P] codes and [P/128][M] scales of the output gradient,
 *              transposed (dsmoe_quant_tokens_128 over its M columns)
 *   bt, sb     [N][P] codes and [P/128][N] scales of the GEMM input, likewise
 *   chunk_off  [G+1] the groups' tiles (from dsmoe_quant_tokens_128)
 *   c          [G][M][N] output (ct: DSMOE_BF16 or DSMOE_F32):
 *              c[g][m][n] = sum over tiles t of group g of
 *              sa[t][m] * sb[t][n] * sum_k dec(at[m][128t+k]) dec(bt[n][128t+k]),
 *              each tile's partial sum promoted to FP32; 0 for a group
 *              without rows
 * For the down projection o = a W2^T: at = quantised do^T (M = H), bt =
 * quantised a^T (N = I), c = dW2 [G][H][I].  For the gate/up projection:
 * at = quantised dh^T (M = 2I), bt = quantised x^T (N = H), c = dW13.
 * Requires M, N positive multiples of 128, 1 <= G, P a multiple of 128 and
 * 128 * P < 2^32 (DSMOE_ERR_SHAPE otherwise).
 */
dsmoe_status dsmoe_fp8_wgrad_grouped(const uint8_t* at, const float* sa, const uint8_t* bt, const float* sb,
                                     const int32_t* chunk_off, int32_t G, int64_t M, int64_t N, int64_t P,
                                     void* c, int ct, void* stream);

/*
 * dsmoe_swiglu_backward -- SwiGLU backward on the recomputed activation.
 *   h         [rows][2I] f32: the gate/up GEMM output (gate columns, then up)
 *   da        [rows][I] f32: gradient of the expert's SwiGLU output before
 *             the gate factor (the down projection's dgrad output)
 *   row_gate  [rows] f32 or NULL (1): the row's gate, multiplied in first
 *   dh        [rows][2I] f32 (output): with d = row_gate * da, sig = 1 /
 *             (1 + e^-g): dh_gate = d u sig (1 + g (1 - sig)), dh_up = d g sig
 *   a_out     [rows][I] f32 or NULL: the recomputed a = g sig u
 * Requires I % 128 == 0, rows >= 0.
 */
dsmoe_status dsmoe_swiglu_backward(const float* h, const float* da, const float* row_gate, int64_t rows,
                                   int64_t I, float* dh, float* a_out, void* stream);

/*
 * dsmoe_gate_backward -- gradients of the gates and of the router logits.
 *   dy        [T][H] bf16: gradient of the layer output y
 *   o         [T*K][H] (ot: bf16 or f32): the routed experts' ungated
 *             outputs, row inv[t][k] for token t's k-th expert
 *   inv       [T][K], topk_idx [T][K] int32, logits [T][E] f32: the forward's
 *   dgate     [T][K] f32 (output): dgate[t][k] = <dy[t], o[inv[t][k]]>
 *   dlogits   [T][E] f32 (output): with s = fl32(sigmoid(z)) (double
 *             evaluation, as the routing), S = sum of the chosen s, gate =
 *             s / S: s_k (1 - s_k) (dgate_k - sum_j dgate_j gate_j) / S at
 *             the chosen experts, 0 elsewhere (routing held fixed)
 * Requires H % 8 == 0, 1 <= K <= DSMOE_MAX_TOPK, K <= E <= DSMOE_MAX_EXPERTS.
 */
dsmoe_status dsmoe_gate_backward(const void* dy, const void* o, int ot, const int32_t* inv,
                                 const int32_t* topk_idx, const float* logits, int64_t T, int32_t E,
                                 int32_t K, int64_t H, float* dgate, float* dlogits, void* stream);

/*
 * dsmoe_combine_rows -- the forward's combine over rows of (token, expert)
 * results: y[t] = o[shared0 + t] (when shared0 >= 0) + sum over k ascending of
 * o[inv[t][k]], summed in float32 (e.g. the input gradient of the gate/up
 * projection from its per-row dgrad).  o and y share the type ot (bf16 or
 * f32), rows of H columns.  Requires H % 8 == 0.
 */
dsmoe_status dsmoe_combine_rows(const void* o, int ot, const int32_t* inv, int64_t T, int32_t K, int64_t H,
                                int64_t shared0, void* y, void* stream);

/*
 * Coarser scaling granularities, for comparison with the recipe's 1x128 /
 * 128x128 tiles.  Source: infra answer, FP8 paragraph (per-tensor E4M3
 * scaling lets a single outlier stretch the scale of a whole tensor and so
 * the quantisation error of everything else; the fine-grained tiles are the
 * recipe's answer; per-token x per-channel scaling, which needs no tiling, is
 * named there as not discussed); V3 notes §6.1 (the recipe itself).
 * Every scale below follows the rule of dsmoe_quant_act_1x128 (s =
 * fl32(amax / 448), s = 1 when amax = 0, q = E4M3(fl32(x / s))), taken over
 * a different set of values.
 */

/*
 * dsmoe_quant_rows -- one scale per row, over the whole row: per token for
 * an activation [tokens][channels], per output channel for a weight [N][K].
 *
 *   x      [rows][cols] row-major, dtype xt (DSMOE_BF16 or DSMOE_F32)
 *   q      [rows][cols] uint8 E4M3FN codes (output)
 *   scale  [rows] float32 (output)
 * Requires rows >= 0, 8 <= cols <= 32768, cols % 8 == 0.
 */
dsmoe_status dsmoe_quant_rows(const void* x, int xt, int64_t rows, int64_t cols, uint8_t* q,
                              float* scale, void* stream);

/* Floats of the scratch buffer dsmoe_quant_tensor takes (8 KB). */
#define DSMOE_QUANT_TENSOR_SCRATCH_FLOATS 2048

/*
 * dsmoe_quant_tensor -- one scale for a whole tensor of n elements.
 *
 *   x      [n] dtype xt (any shape, contiguous)
 *   q      [n] uint8 E4M3FN codes (output)
 *   scale  [1] float32 (output)
 *   amax   [DSMOE_QUANT_TENSOR_SCRATCH_FLOATS] float32 scratch: the first
 *          pass merges the blocks' maxima into 64 slots on separate 128-byte
 *          lines of it; on return amax[0] = max |x| (the rest is
 *          unspecified).  Must not alias x, q or scale.
 * Three kernels on `stream`: clear the slots, amax pass (exact, independent
 * of order), encode pass.  n = 0 writes amax[0] = 0 and scale = 1.
 * Requires n >= 0, n % 8 == 0.
 */
dsmoe_status dsmoe_quant_tensor(const void* x, int xt, int64_t n, uint8_t* q, float* scale,
                                float* amax, void* stream);

typedef enum dsmoe_granularity {
  DSMOE_SCALE_TENSOR = 0,  /* one scale for A, one for W */
  DSMOE_SCALE_CHANNEL = 1, /* one per row of A (token), one per row of W (output channel) */
  DSMOE_SCALE_BLOCK = 2    /* 1x128 tiles of A, 128x128 blocks of W (the recipe) */
} dsmoe_granularity;

/* Workspace of dsmoe_fp8_gemm_granularity (0 for invalid sizes). */
size_t dsmoe_gemm_granularity_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * dsmoe_fp8_gemm_granularity -- c = A W^T with both operands quantised to
 * E4M3 at one granularity, on the device from the high-precision inputs.
 *
 *   a          [M][K] dtype t (DSMOE_BF16 or DSMOE_F32)
 *   w          [N][K] dtype t
 *   c          [M][N] float32 (output)
 *   workspace  device buffer of at least
 *              dsmoe_gemm_granularity_workspace_bytes(M, N, K), 256-byte
 *              aligned; holds the codes and scales of both operands after
 *              the call (layout private)
 * TENSOR and CHANNEL quantise with dsmoe_quant_tensor / dsmoe_quant_rows and
 * broadcast the scales into the 1x128 / 128x128 layouts of
 * dsmoe_fp8_grouped_gemm; a per-output-channel scale of W is applied to c
 * after the GEMM (c[m][n] = fl32(sum * sw[n])).  BLOCK is the recipe
 * (dsmoe_quant_act_1x128, dsmoe_quant_w_128x128).  The GEMM promotes every
 * 128-K chunk to float32 as in dsmoe_fp8_grouped_gemm.
 * Requires M >= 0, N and K positive multiples of 128, K <= 32768.
 */
dsmoe_status dsmoe_fp8_gemm_granularity(const void* a, const void* w, int t, int64_t M, int64_t N,
                                        int64_t K, int granularity, float* c, void* workspace,
                                        size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSMOE_H */
