// The extern "C" boundary: host-side validation, workspace layout and the
// orchestration of the layer forward.  Nothing here allocates device memory;
// every call validates all arguments before it enqueues anything.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "dsmoe.h"
#include "kernels.h"

// Scratch of dsmoe_moe_forward_noalloc: one array per GPU, part of the
// library's device code, so no call allocates.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept in g_scratch_ptr.
static __device__ __align__(256) uint8_t scratch[DSMOE_NOALLOC_SCRATCH_BYTES];


namespace {

constexpr int64_t kI32Max = 2147483647LL;
constexpr int64_t kMaxK = 32768;   // contraction length limit of the FP8 GEMM (256 chunks)

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

dsmoe_status launch_status(hipError_t e) { return e == hipSuccess ? DSMOE_OK : DSMOE_ERR_LAUNCH; }

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[64];

// The current device's address of `scratch`, or nullptr on failure.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

// Device check, cached per device ordinal (idempotent).
std::atomic<int> g_dev_ok[64];

dsmoe_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DSMOE_ERR_DEVICE;
  if (dev < 64) {
    const int v = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (v == 1) return DSMOE_OK;
    if (v == 2) return DSMOE_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DSMOE_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? DSMOE_OK : DSMOE_ERR_DEVICE;
}

bool valid_dtype(int t) { return t == DSMOE_BF16 || t == DSMOE_F32; }

dsmoe_status check_routing_shape(int64_t T, int32_t E, int32_t G, int32_t Mg, int32_t K) {
  if (T < 0) return DSMOE_ERR_SHAPE;
  if (E < 1 || E > DSMOE_MAX_EXPERTS) return DSMOE_ERR_SHAPE;
  if (G < 1 || G > DSMOE_MAX_GROUPS || E % G != 0) return DSMOE_ERR_SHAPE;
  if (Mg < 1 || Mg > G) return DSMOE_ERR_SHAPE;
  if (K < 1 || K > DSMOE_MAX_TOPK || static_cast<int64_t>(K) > static_cast<int64_t>(Mg) * (E / G))
    return DSMOE_ERR_SHAPE;
  if (T * (K + 1) > kI32Max) return DSMOE_ERR_SHAPE;
  return DSMOE_OK;
}

// Workspace layout of dsmoe_moe_forward (every region 256-byte aligned).
struct Layout {
  size_t qx, sx, logits, router_part, topk, gates, offsets, offsets_ext, perm, inv, row_gate, qa, sa, o,
      total;
};

Layout layout_for(const dsmoe_moe_desc& d, int64_t T) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  const size_t TK = static_cast<size_t>(T) * d.K;
  const size_t rows1 = TK + (d.n_shared ? static_cast<size_t>(T) : 0);
  L.qx = take(static_cast<size_t>(T) * d.H);
  L.sx = take(static_cast<size_t>(T) * (d.H / 128) * 4);
  L.logits = take(static_cast<size_t>(T) * d.E * 4);
  L.router_part = take(dsmoe::router_partial_bytes(T, d.H, d.E));
  L.topk = take(TK * 4);
  L.gates = take(TK * 4);
  L.offsets = take((static_cast<size_t>(d.E) + 1) * 4);
  L.offsets_ext = take((static_cast<size_t>(d.E) + 2) * 4);
  L.perm = take(rows1 * 4);
  L.inv = take(TK * 4);
  L.row_gate = take(TK * 4);
  L.qa = take(rows1 * d.I);
  L.sa = take(rows1 * (d.I / 128) * 4);
  L.o = take(rows1 * d.H * 4);
  L.total = off;
  return L;
}

dsmoe_status check_desc(const dsmoe_moe_desc* d, int64_t T) {
  if (!d) return DSMOE_ERR_NULL;
  if (d->H <= 0 || d->I <= 0 || d->H % 128 || d->I % 128) return DSMOE_ERR_SHAPE;
  if (d->H > kMaxK || d->I > kMaxK) return DSMOE_ERR_SHAPE;
  if (d->n_shared != 0 && d->n_shared != 1) return DSMOE_ERR_SHAPE;
  const dsmoe_status s = check_routing_shape(T, d->E, d->G, d->Mg, d->K);
  if (s != DSMOE_OK) return s;
  if (T * d->H > (1LL << 40) || static_cast<int64_t>(d->E) * d->H > (1LL << 40)) return DSMOE_ERR_SHAPE;
  return DSMOE_OK;
}

// The debug buffers a caller asked for: 4-byte alignment of every pointer.
bool debug_aligned(const dsmoe_moe_debug* dbg) {
  if (!dbg) return true;
  const void* dp[] = {dbg->qx, dbg->sx, dbg->logits, dbg->topk_idx, dbg->gates,
                      dbg->offsets, dbg->perm, dbg->inv, dbg->qa, dbg->sa};
  for (const void* p : dp)
    if (p && !aligned(p, 4)) return false;
  return true;
}

// Device-to-device copies of the forward's intermediates into the debug
// buffers that are given (stream-ordered after the forward's kernels).
hipError_t copy_debug(const dsmoe_moe_debug& dbg, const dsmoe_moe_desc& d, int64_t T,
                      const Layout& L, uint8_t* ws, hipStream_t st) {
  const size_t TK = static_cast<size_t>(T) * d.K;
  const size_t rows = TK + (d.n_shared ? static_cast<size_t>(T) : 0);
  struct Cp { void* dst; size_t off; size_t n; } cps[] = {
      {dbg.qx, L.qx, static_cast<size_t>(T) * d.H},
      {dbg.sx, L.sx, static_cast<size_t>(T) * (d.H / 128) * 4},
      {dbg.logits, L.logits, static_cast<size_t>(T) * d.E * 4},
      {dbg.topk_idx, L.topk, TK * 4},
      {dbg.gates, L.gates, TK * 4},
      {dbg.offsets, L.offsets, (static_cast<size_t>(d.E) + 1) * 4},
      {dbg.perm, L.perm, TK * 4},
      {dbg.inv, L.inv, TK * 4},
      {dbg.qa, L.qa, rows * d.I},
      {dbg.sa, L.sa, rows * (d.I / 128) * 4},
  };
  for (const Cp& c : cps)
    if (c.dst) {
      const hipError_t e = hipMemcpyAsync(c.dst, ws + c.off, c.n, hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return e;
    }
  return hipSuccess;
}

// Workspace of dsmoe_moe_forward_serving: the forward's regions, then the
// per-row gates of routed and shared rows and the slots' group offsets.
struct ServingLayout {
  Layout base;
  size_t row_gate_all, phys, total;
};

ServingLayout serving_layout(const dsmoe_moe_desc& d, int64_t T, int32_t S) {
  ServingLayout L{};
  L.base = layout_for(d, T);
  size_t off = L.base.total;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  L.row_gate_all = take((static_cast<size_t>(T) * d.K + (d.n_shared ? T : 0)) * 4);
  L.phys = take((static_cast<size_t>(S) + 2) * 4);
  L.total = off;
  return L;
}

// Workspace layout of dsmoe_fp8_gemm_granularity (every region 256-byte
// aligned): codes and the 1x128 / 128x128 scale layouts of both operands,
// the per-row scales, the per-tensor scale and amax slots, the offsets {0, M}.
struct GranLayout {
  size_t qa, qw, sa, sw, row_a, row_w, scales, amax_a, amax_w, offsets, total;
};

GranLayout gran_layout(int64_t M, int64_t N, int64_t K) {
  // the header's scratch size must cover the kernels' slots
  static_assert(DSMOE_QUANT_TENSOR_SCRATCH_FLOATS >= 64 * 32, "amax scratch");
  GranLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  L.qa = take(static_cast<size_t>(M) * K);
  L.qw = take(static_cast<size_t>(N) * K);
  L.sa = take(static_cast<size_t>(M) * (K / 128) * 4);
  L.sw = take(static_cast<size_t>(N / 128) * (K / 128) * 4);
  L.row_a = take(static_cast<size_t>(M) * 4);
  L.row_w = take(static_cast<size_t>(N) * 4);
  L.scales = take(2 * 4);  // per-tensor scale of A, of W
  L.amax_a = take(DSMOE_QUANT_TENSOR_SCRATCH_FLOATS * 4);
  L.amax_w = take(DSMOE_QUANT_TENSOR_SCRATCH_FLOATS * 4);
  L.offsets = take(2 * 4);
  L.total = off;
  return L;
}

dsmoe_status check_gran_shape(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N <= 0 || K <= 0 || N % 128 || K % 128 || K > kMaxK) return DSMOE_ERR_SHAPE;
  if (M > kI32Max || N > kI32Max) return DSMOE_ERR_SHAPE;
  if (M * K > (1LL << 40) || N * K > (1LL << 40)) return DSMOE_ERR_SHAPE;
  if (((M + 15) / 16 + 1) * (N / 128) >= kI32Max) return DSMOE_ERR_SHAPE;
  return DSMOE_OK;
}

}  // namespace

extern "C" {

const char* dsmoe_status_str(int status) {
  switch (status) {
    case DSMOE_OK: return "DSMOE_OK";
    case DSMOE_ERR_NULL: return "DSMOE_ERR_NULL";
    case DSMOE_ERR_SHAPE: return "DSMOE_ERR_SHAPE";
    case DSMOE_ERR_ALIGN: return "DSMOE_ERR_ALIGN";
    case DSMOE_ERR_DTYPE: return "DSMOE_ERR_DTYPE";
    case DSMOE_ERR_WORKSPACE: return "DSMOE_ERR_WORKSPACE";
    case DSMOE_ERR_DEVICE: return "DSMOE_ERR_DEVICE";
    case DSMOE_ERR_LAUNCH: return "DSMOE_ERR_LAUNCH";
    default: return "DSMOE_ERR_UNKNOWN";
  }
}

int dsmoe_abi_version(void) { return 1; }

dsmoe_status dsmoe_quant_act_1x128(const void* x, int xt, int64_t rows, int64_t cols, uint8_t* q,
                                   float* scale, void* stream) {
  if (!valid_dtype(xt)) return DSMOE_ERR_DTYPE;
  if (rows < 0 || cols <= 0 || cols % 128) return DSMOE_ERR_SHAPE;
  if (rows * (cols / 128) * 16 / 256 >= kI32Max) return DSMOE_ERR_SHAPE;
  if (rows == 0) return DSMOE_OK;
  if (!x || !q || !scale) return DSMOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  return launch_status(dsmoe::launch_quant_act(x, xt == DSMOE_F32, rows, cols, q, scale,
                                               static_cast<hipStream_t>(stream)));
}

dsmoe_status dsmoe_quant_w_128x128(const void* w, int wt, int64_t n_mats, int64_t N, int64_t K,
                                   uint8_t* q, float* scale, void* stream) {
  if (!valid_dtype(wt)) return DSMOE_ERR_DTYPE;
  if (n_mats < 0 || N <= 0 || K <= 0 || N % 128 || K % 128) return DSMOE_ERR_SHAPE;
  if (n_mats * (N / 128) * (K / 128) >= kI32Max) return DSMOE_ERR_SHAPE;
  if (n_mats == 0) return DSMOE_OK;
  if (!w || !q || !scale) return DSMOE_ERR_NULL;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(scale, 4)) return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  return launch_status(dsmoe::launch_quant_w(w, wt == DSMOE_F32, n_mats, N, K, q, scale,
                                             static_cast<hipStream_t>(stream)));
}

dsmoe_status dsmoe_e4m3_codes(const float* x, int64_t n, int converter, uint8_t* q, void* stream) {
  if (converter != 0 && converter != 1) return DSMOE_ERR_DTYPE;
  if (n < 0 || n > (1LL << 40)) return DSMOE_ERR_SHAPE;
  if (n == 0) return DSMOE_OK;
  if (!x || !q) return DSMOE_ERR_NULL;
  if (!aligned(x, 4)) return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  return launch_status(dsmoe::launch_e4m3_codes(x, n, converter == 1, q, static_cast<hipStream_t>(stream)));
}

dsmoe_status dsmoe_transpose_w_128x128(const uint8_t* q, const float* s, int64_t n_mats, int64_t N,
                                       int64_t K, uint8_t* qt, float* st, void* stream) {
  if (n_mats < 0 || N <= 0 || K <= 0 || N % 128 || K % 128) return DSMOE_ERR_SHAPE;
  if (n_mats * (N / 128) * (K / 128) >= kI32Max || N * K > (1LL << 40)) return DSMOE_ERR_SHAPE;
  if (n_mats == 0) return DSMOE_OK;
  if (!q || !s || !qt || !st) return DSMOE_ERR_NULL;
  if (!aligned(q, 16) || !aligned(qt, 16) || !aligned(s, 4) || !aligned(st, 4)) return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  return launch_status(dsmoe::launch_transpose_w(q, s, n_mats, N, K, qt, st, static_cast<hipStream_t>(stream)));
}

dsmoe_status dsmoe_route(const float* logits, const float* bias, int64_t T, int32_t E, int32_t G,
                         int32_t Mg, int32_t K, int32_t* topk_idx, float* gates, int32_t* counts,
                         int32_t* offsets, int32_t* perm, int32_t* inv, void* stream) {
  dsmoe_status s = check_routing_shape(T, E, G, Mg, K);
  if (s != DSMOE_OK) return s;
  if (!bias || !counts || !offsets) return DSMOE_ERR_NULL;
  if (T > 0 && (!logits || !topk_idx || !gates || !perm || !inv)) return DSMOE_ERR_NULL;
  const void* ptrs[] = {logits, bias, topk_idx, gates, counts, offsets, perm, inv};
  for (const void* p : ptrs)
    if (p && !aligned(p, 4)) return DSMOE_ERR_ALIGN;
  s = check_device();
  if (s != DSMOE_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = dsmoe::launch_route_select(logits, bias, T, E, G, Mg, K, topk_idx, gates, counts, st);
  if (e != hipSuccess) return DSMOE_ERR_LAUNCH;
  e = dsmoe::launch_permute(topk_idx, gates, T, E, K, counts, offsets, perm, inv, nullptr, nullptr, st);
  return launch_status(e);
}

dsmoe_status dsmoe_fp8_grouped_gemm(const uint8_t* a, const float* a_scale,
                                    const int32_t* a_rows, const int32_t* offsets, int32_t G,
                                    int64_t M_total, const uint8_t* w, const float* w_scale,
                                    int64_t N, int64_t K, void* c, int ct, void* stream) {
  if (!valid_dtype(ct)) return DSMOE_ERR_DTYPE;
  if (G < 1 || M_total < 0 || N <= 0 || K <= 0 || N % 128 || K % 128) return DSMOE_ERR_SHAPE;
  if (K > kMaxK) return DSMOE_ERR_SHAPE;
  if (M_total > kI32Max || G > kI32Max / 2) return DSMOE_ERR_SHAPE;
  if (((M_total + 15) / 16 + G) * (N / 128) >= kI32Max) return DSMOE_ERR_SHAPE;  // grid of the smallest tiles
  if (M_total == 0) return DSMOE_OK;
  if (!a || !a_scale || !offsets || !w || !w_scale || !c) return DSMOE_ERR_NULL;
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(c, 16) || !aligned(a_scale, 4) ||
      !aligned(w_scale, 4) || !aligned(offsets, 4) || (a_rows && !aligned(a_rows, 4)))
    return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  dsmoe::GemmProblem p{};
  p.a = a;
  p.a_scale = a_scale;
  p.a_rows = a_rows;
  p.offsets = offsets;
  p.G = G;
  p.M_total = M_total;
  p.w = w;
  p.w_scale = w_scale;
  p.N = N;
  p.K = K;
  p.c = c;
  p.c_f32 = ct == DSMOE_F32;
  p.epi = dsmoe::Epilogue::kStore;
  p.row_limit = M_total;
  p.rows_hint = (M_total + G - 1) / G;
  p.a_rows_total = a_rows ? 0 : M_total;   // with a gather A's row count is not known
  return launch_status(dsmoe::launch_grouped_gemm(p, static_cast<hipStream_t>(stream)));
}

size_t dsmoe_moe_workspace_bytes(const dsmoe_moe_desc* d, int64_t T) {
  if (check_desc(d, T) != DSMOE_OK) return 0;
  return layout_for(*d, T).total;
}

dsmoe_status dsmoe_moe_forward(const dsmoe_moe_desc* d, const dsmoe_moe_weights* w,
                               const float* bias, const void* x, int64_t T, void* y, int yt,
                               int32_t* counts_out, void* workspace, size_t ws_bytes,
                               const dsmoe_moe_debug* dbg, void* stream) {
  dsmoe_status s = check_desc(d, T);
  if (s != DSMOE_OK) return s;
  if (!valid_dtype(yt)) return DSMOE_ERR_DTYPE;
  if (!w || !bias || !counts_out) return DSMOE_ERR_NULL;
  if (!w->w13 || !w->s13 || !w->w2 || !w->s2 || !w->router_w) return DSMOE_ERR_NULL;
  if (d->n_shared && (!w->w13_sh || !w->s13_sh || !w->w2_sh || !w->s2_sh)) return DSMOE_ERR_NULL;
  if (T > 0 && (!x || !y)) return DSMOE_ERR_NULL;
  const Layout L = layout_for(*d, T);
  if (T > 0 && !workspace) return DSMOE_ERR_WORKSPACE;
  if (ws_bytes < L.total) return DSMOE_ERR_WORKSPACE;
  if ((x && !aligned(x, 16)) || (y && !aligned(y, 16)) || !aligned(w->w13, 16) ||
      !aligned(w->w2, 16) || !aligned(w->router_w, 16) || !aligned(w->s13, 4) ||
      !aligned(w->s2, 4) || !aligned(bias, 4) || !aligned(counts_out, 4) ||
      (workspace && !aligned(workspace, 256)))
    return DSMOE_ERR_ALIGN;
  if (d->n_shared && (!aligned(w->w13_sh, 16) || !aligned(w->w2_sh, 16) ||
                      !aligned(w->s13_sh, 4) || !aligned(w->s2_sh, 4)))
    return DSMOE_ERR_ALIGN;
  if (!debug_aligned(dbg)) return DSMOE_ERR_ALIGN;
  s = check_device();
  if (s != DSMOE_OK) return s;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t H = d->H, I = d->I;
  const int32_t E = d->E, K = d->K;
  const bool f32out = yt == DSMOE_F32;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* qx = ws + L.qx;
  float* sx = reinterpret_cast<float*>(ws + L.sx);
  float* logits = reinterpret_cast<float*>(ws + L.logits);
  int32_t* topk = reinterpret_cast<int32_t*>(ws + L.topk);
  float* gates = reinterpret_cast<float*>(ws + L.gates);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* offsets_ext = reinterpret_cast<int32_t*>(ws + L.offsets_ext);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + L.perm);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv);
  float* row_gate = reinterpret_cast<float*>(ws + L.row_gate);
  uint8_t* qa = ws + L.qa;
  float* sa = reinterpret_cast<float*>(ws + L.sa);
  void* o = ws + L.o;

  hipError_t e;
#define DSMOE_TRY(expr)              \
  do {                               \
    e = (expr);                      \
    if (e != hipSuccess) return DSMOE_ERR_LAUNCH; \
  } while (0)

  if (T == 0) {
    DSMOE_TRY(dsmoe::launch_route_select(nullptr, bias, 0, E, d->G, d->Mg, K, nullptr, nullptr,
                                         counts_out, st));
    return DSMOE_OK;
  }
  void* const* ev = dbg ? dbg->stage_events : nullptr;
#define DSMOE_MARK(i) \
  if (ev) DSMOE_TRY(hipEventRecord(static_cast<hipEvent_t>(ev[(i)]), st))

  DSMOE_MARK(0);

  // 1x128 quantisation of x
  DSMOE_TRY(dsmoe::launch_quant_act(x, false, T, H, qx, sx, st));
  DSMOE_MARK(1);
  // router logits (bf16 MFMA, FP32 accumulation)
  DSMOE_TRY(dsmoe::launch_router_logits(static_cast<const uint16_t*>(x),
                                        static_cast<const uint16_t*>(w->router_w), T, H, E,
                                        logits, reinterpret_cast<float*>(ws + L.router_part), st));
  DSMOE_MARK(2);
  // group-limited top-K routing
  DSMOE_TRY(dsmoe::launch_route_select(logits, bias, T, E, d->G, d->Mg, K, topk, gates,
                                       counts_out, st));
  DSMOE_MARK(3);
  // counts -> offsets, permutation, inverse, per-row gates; shared rows
  DSMOE_TRY(dsmoe::launch_permute(topk, gates, T, E, K, counts_out, offsets, perm, inv, row_gate,
                                  d->n_shared ? offsets_ext : nullptr, st));
  DSMOE_MARK(4);

  // gate/up GEMM of every routed expert and the shared one, SwiGLU and 1x128 requant
  dsmoe::GemmProblem g1{};
  g1.a = qx;
  g1.a_scale = sx;
  g1.a_rows = perm;
  g1.offsets = d->n_shared ? offsets_ext : offsets;
  g1.G = E + (d->n_shared ? 1 : 0);
  g1.M_total = T * K + (d->n_shared ? T : 0);
  g1.w = w->w13;
  g1.w_scale = w->s13;
  g1.w_last = d->n_shared ? w->w13_sh : nullptr;
  g1.w_scale_last = d->n_shared ? w->s13_sh : nullptr;
  g1.N = 2 * I;
  g1.K = H;
  g1.c = qa;
  g1.c_scale = sa;
  g1.epi = dsmoe::Epilogue::kSwiGLUQuant;
  g1.row_limit = g1.M_total;
  g1.rows_hint = (T * K + E - 1) / E;
  g1.a_rows_total = T;
  DSMOE_TRY(dsmoe::launch_grouped_gemm(g1, st));
  DSMOE_MARK(5);

  // routed down projection, scaled by the gate
  dsmoe::GemmProblem g2{};
  g2.a = qa;
  g2.a_scale = sa;
  g2.a_rows = nullptr;
  g2.offsets = offsets;
  g2.G = E;
  g2.M_total = T * K;
  g2.w = w->w2;
  g2.w_scale = w->s2;
  g2.N = H;
  g2.K = I;
  g2.c = o;
  g2.c_f32 = f32out;
  g2.row_gate = row_gate;
  g2.epi = dsmoe::Epilogue::kGateStore;
  g2.row_limit = g2.M_total;
  g2.rows_hint = (T * K + E - 1) / E;
  g2.a_rows_total = g1.M_total;
  DSMOE_TRY(dsmoe::launch_grouped_gemm(g2, st));
  DSMOE_MARK(6);

  if (d->n_shared) {
    // down projection of the shared expert into rows T*K .. T*K+T-1 of o
    dsmoe::GemmProblem g3{};
    g3.a = qa;
    g3.a_scale = sa;
    g3.a_rows = nullptr;
    g3.offsets = offsets_ext + E;  // {T*K, T*K + T}
    g3.G = 1;
    g3.M_total = T;
    g3.w = w->w2_sh;
    g3.w_scale = w->s2_sh;
    g3.N = H;
    g3.K = I;
    g3.c = o;
    g3.c_f32 = f32out;
    g3.epi = dsmoe::Epilogue::kStore;
    g3.row_limit = T * K + T;
    g3.rows_hint = T;
    g3.a_rows_total = T * K + T;
    DSMOE_TRY(dsmoe::launch_grouped_gemm(g3, st));
  }
  // y[t] = shared row + routed rows in ascending k (float32 sums)
  DSMOE_TRY(dsmoe::launch_combine(o, inv, T, K, H, d->n_shared ? T * K : -1, y, f32out, st));
  DSMOE_MARK(7);
#undef DSMOE_MARK

  if (dbg) DSMOE_TRY(copy_debug(*dbg, *d, T, L, ws, st));
#undef DSMOE_TRY
  return DSMOE_OK;
}

dsmoe_status dsmoe_moe_forward_noalloc(const dsmoe_moe_desc* d, const dsmoe_moe_weights* w,
                                       const float* bias, const void* x, int64_t T, void* y, int yt,
                                       int32_t* counts_out, const dsmoe_moe_debug* dbg, void* stream) {
  const dsmoe_status s = check_desc(d, T);
  if (s != DSMOE_OK) return s;
  if (layout_for(*d, T).total > DSMOE_NOALLOC_SCRATCH_BYTES) return DSMOE_ERR_WORKSPACE;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  void* ws = scratch_for_current_device();
  if (!ws) return DSMOE_ERR_DEVICE;
  return dsmoe_moe_forward(d, w, bias, x, T, y, yt, counts_out, ws, DSMOE_NOALLOC_SCRATCH_BYTES, dbg,
                           stream);
}

dsmoe_status dsmoe_update_bias(float* bias, const int32_t* counts, int32_t E, int64_t T,
                               int32_t K, float gamma, void* stream) {
  if (E < 1 || E > DSMOE_MAX_EXPERTS || T < 0 || K < 1) return DSMOE_ERR_SHAPE;
  if (!bias || !counts) return DSMOE_ERR_NULL;
  if (!aligned(bias, 4) || !aligned(counts, 4)) return DSMOE_ERR_ALIGN;
  const dsmoe_status s = check_device();
  if (s != DSMOE_OK) return s;
  return launch_status(dsmoe::launch_update_bias(bias, counts, E, T, K, gamma,
                                                 static_cast<hipStream_t>(stream)));
}

dsmoe_status dsmoe_quant_rows(const void* x, int xt, int64_t rows, int64_t cols, uint8_t* q,
                              float* scale, void* stream) {
  if (!valid_dtype(xt)) return DSMOE_ERR_DTYPE;
  if (rows < 0 || cols < 8 || cols % 8 || cols > dsmoe::quant_rows_max_cols()) return DSMOE_ERR_SHAPE;
  if (rows > kI32Max) return DSMOE_ERR_SHAPE;
  if (rows == 0) return DSMOE_OK;
  if (!x || !q || !scale) return DSMOE_ERR_NULL;
  // rows of 8 elements keep every row start 16-byte aligned for bf16; f32 needs 32 bytes
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(scale, 4)) return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  return launch_status(dsmoe::launch_quant_rows(x, xt == DSMOE_F32, rows, cols, q, scale,
                                                static_cast<hipStream_t>(stream)));
}

dsmoe_status dsmoe_quant_tensor(const void* x, int xt, int64_t n, uint8_t* q, float* scale,
                                float* amax, void* stream) {
  if (!valid_dtype(xt)) return DSMOE_ERR_DTYPE;
  if (n < 0 || n % 8 || n > (1LL << 40)) return DSMOE_ERR_SHAPE;
  if (!scale || !amax) return DSMOE_ERR_NULL;
  if (n > 0 && (!x || !q)) return DSMOE_ERR_NULL;
  if ((x && !aligned(x, 16)) || (q && !aligned(q, 8)) || !aligned(scale, 4) || !aligned(amax, 4))
    return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  return launch_status(dsmoe::launch_quant_tensor(x, xt == DSMOE_F32, n, q, scale, amax,
                                                  static_cast<hipStream_t>(stream)));
}

size_t dsmoe_gemm_granularity_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (check_gran_shape(M, N, K) != DSMOE_OK) return 0;
  return gran_layout(M, N, K).total;
}

dsmoe_status dsmoe_fp8_gemm_granularity(const void* a, const void* w, int t, int64_t M, int64_t N,
                                        int64_t K, int granularity, float* c, void* workspace,
                                        size_t ws_bytes, void* stream) {
  if (!valid_dtype(t)) return DSMOE_ERR_DTYPE;
  if (granularity != DSMOE_SCALE_TENSOR && granularity != DSMOE_SCALE_CHANNEL &&
      granularity != DSMOE_SCALE_BLOCK)
    return DSMOE_ERR_SHAPE;
  dsmoe_status s = check_gran_shape(M, N, K);
  if (s != DSMOE_OK) return s;
  if (M == 0) return DSMOE_OK;
  if (!a || !w || !c) return DSMOE_ERR_NULL;
  const GranLayout L = gran_layout(M, N, K);
  if (!workspace || ws_bytes < L.total) return DSMOE_ERR_WORKSPACE;
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(c, 16) || !aligned(workspace, 256))
    return DSMOE_ERR_ALIGN;
  s = check_device();
  if (s != DSMOE_OK) return s;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool f32 = t == DSMOE_F32;
  char* ws = static_cast<char*>(workspace);
  uint8_t* qa = reinterpret_cast<uint8_t*>(ws + L.qa);
  uint8_t* qw = reinterpret_cast<uint8_t*>(ws + L.qw);
  float* sa = reinterpret_cast<float*>(ws + L.sa);
  float* sw = reinterpret_cast<float*>(ws + L.sw);
  float* row_a = reinterpret_cast<float*>(ws + L.row_a);
  float* row_w = reinterpret_cast<float*>(ws + L.row_w);
  float* scales = reinterpret_cast<float*>(ws + L.scales);
  float* amax_a = reinterpret_cast<float*>(ws + L.amax_a);
  float* amax_w = reinterpret_cast<float*>(ws + L.amax_w);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  const int64_t kt = K / 128, nb = N / 128;
#define DSMOE_TRY(expr)                          \
  do {                                           \
    if ((expr) != hipSuccess) return DSMOE_ERR_LAUNCH; \
  } while (0)
  switch (granularity) {
    case DSMOE_SCALE_BLOCK:
      DSMOE_TRY(dsmoe::launch_quant_act(a, f32, M, K, qa, sa, st));
      DSMOE_TRY(dsmoe::launch_quant_w(w, f32, 1, N, K, qw, sw, st));
      break;
    case DSMOE_SCALE_CHANNEL:
      DSMOE_TRY(dsmoe::launch_quant_rows(a, f32, M, K, qa, row_a, st));
      DSMOE_TRY(dsmoe::launch_quant_rows(w, f32, N, K, qw, row_w, st));
      DSMOE_TRY(dsmoe::launch_broadcast_scale(sa, M, kt, row_a, 1, st));
      DSMOE_TRY(dsmoe::launch_broadcast_scale(sw, nb, kt, nullptr, 0, st));
      break;
    default:  // DSMOE_SCALE_TENSOR
      DSMOE_TRY(dsmoe::launch_quant_tensor(a, f32, M * K, qa, scales + 0, amax_a, st));
      DSMOE_TRY(dsmoe::launch_quant_tensor(w, f32, N * K, qw, scales + 1, amax_w, st));
      DSMOE_TRY(dsmoe::launch_broadcast_scale(sa, M, kt, scales + 0, 0, st));
      DSMOE_TRY(dsmoe::launch_broadcast_scale(sw, nb, kt, scales + 1, 0, st));
      break;
  }
  DSMOE_TRY(dsmoe::launch_prep_offsets(offsets, static_cast<int32_t>(M), st));
  dsmoe::GemmProblem p{};
  p.a = qa;
  p.a_scale = sa;
  p.offsets = offsets;
  p.G = 1;
  p.M_total = M;
  p.w = qw;
  p.w_scale = sw;
  p.N = N;
  p.K = K;
  p.c = c;
  p.c_f32 = true;
  p.epi = dsmoe::Epilogue::kStore;
  p.row_limit = M;
  p.rows_hint = M;
  DSMOE_TRY(dsmoe::launch_grouped_gemm(p, st));
  if (granularity == DSMOE_SCALE_CHANNEL) DSMOE_TRY(dsmoe::launch_scale_cols(c, M, N, row_w, st));
#undef DSMOE_TRY
  return DSMOE_OK;
}

dsmoe_status dsmoe_plan_replicas(const int32_t* counts, int32_t E, int32_t n_extra,
                                 int32_t* slot_first, int32_t* slot_expert, void* stream) {
  if (E < 1 || E > DSMOE_MAX_EXPERTS || n_extra < 0 || n_extra > DSMOE_MAX_EXPERTS)
    return DSMOE_ERR_SHAPE;
  if (!counts || !slot_first || !slot_expert) return DSMOE_ERR_NULL;
  if (!aligned(counts, 4) || !aligned(slot_first, 4) || !aligned(slot_expert, 4)) return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  return launch_status(dsmoe::launch_plan_replicas(counts, E, n_extra, slot_first, slot_expert,
                                                   static_cast<hipStream_t>(stream)));
}

dsmoe_status dsmoe_place_replicas(const uint8_t* w, const float* w_scale, int32_t E, int64_t N,
                                  int64_t K, const int32_t* slot_expert, int32_t n_slots,
                                  uint8_t* w_slots, float* s_slots, void* stream) {
  if (E < 1 || N <= 0 || K <= 0 || N % 128 || K % 128 || n_slots < 0 || n_slots > 65535)
    return DSMOE_ERR_SHAPE;
  if (N * K > (1LL << 40)) return DSMOE_ERR_SHAPE;
  if (n_slots == 0) return DSMOE_OK;
  if (!w || !w_scale || !slot_expert || !w_slots || !s_slots) return DSMOE_ERR_NULL;
  if (!aligned(w, 16) || !aligned(w_slots, 16) || !aligned(w_scale, 4) || !aligned(s_slots, 4) ||
      !aligned(slot_expert, 4))
    return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  return launch_status(dsmoe::launch_place_slots(w, w_scale, E, N, K, slot_expert, n_slots, w_slots, s_slots,
                                                 static_cast<hipStream_t>(stream)));
}

dsmoe_status dsmoe_slot_offsets(const int32_t* offsets, int32_t E, const int32_t* slot_first,
                                const int32_t* slot_expert, int32_t n_slots, int64_t extra_rows,
                                int32_t* phys, void* stream) {
  if (E < 1 || E > DSMOE_MAX_EXPERTS || n_slots < E || n_slots > E + DSMOE_MAX_EXPERTS)
    return DSMOE_ERR_SHAPE;
  if (extra_rows > kI32Max) return DSMOE_ERR_SHAPE;
  if (!offsets || !slot_first || !slot_expert || !phys) return DSMOE_ERR_NULL;
  if (!aligned(offsets, 4) || !aligned(slot_first, 4) || !aligned(slot_expert, 4) || !aligned(phys, 4))
    return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  return launch_status(dsmoe::launch_slot_offsets(offsets, E, slot_first, slot_expert, n_slots,
                                                  extra_rows < 0 ? -1 : extra_rows, phys,
                                                  static_cast<hipStream_t>(stream)));
}

size_t dsmoe_moe_serving_workspace_bytes(const dsmoe_moe_desc* d, int64_t T, int32_t n_slots) {
  if (check_desc(d, T) != DSMOE_OK) return 0;
  if (n_slots < d->E || n_slots > d->E + DSMOE_MAX_EXPERTS) return 0;
  return serving_layout(*d, T, n_slots).total;
}

dsmoe_status dsmoe_moe_forward_serving(const dsmoe_moe_desc* d, const dsmoe_moe_weights* w,
                                       const int32_t* slot_first, const int32_t* slot_expert,
                                       int32_t n_slots, const float* bias, const void* x, int64_t T,
                                       void* y, int yt, int32_t* counts_out, void* workspace,
                                       size_t ws_bytes, const dsmoe_moe_debug* dbg, void* stream) {
  dsmoe_status s = check_desc(d, T);
  if (s != DSMOE_OK) return s;
  if (!valid_dtype(yt)) return DSMOE_ERR_DTYPE;
  void* const* stage_events = dbg ? dbg->stage_events : nullptr;
  if (stage_events)
    for (int i = 0; i < DSMOE_SERVING_STAGE_EVENTS; ++i)
      if (!stage_events[i]) return DSMOE_ERR_NULL;
  if (n_slots < d->E || n_slots > d->E + DSMOE_MAX_EXPERTS) return DSMOE_ERR_SHAPE;
  if (T * (d->K + 1) + n_slots > kI32Max) return DSMOE_ERR_SHAPE;
  if (!w || !bias || !counts_out || !slot_first || !slot_expert) return DSMOE_ERR_NULL;
  if (!w->w13 || !w->s13 || !w->w2 || !w->s2 || !w->router_w) return DSMOE_ERR_NULL;
  if (d->n_shared && (!w->w13_sh || !w->s13_sh || !w->w2_sh || !w->s2_sh)) return DSMOE_ERR_NULL;
  if (T > 0 && (!x || !y)) return DSMOE_ERR_NULL;
  const ServingLayout SL = serving_layout(*d, T, n_slots);
  const Layout& L = SL.base;
  if (T > 0 && !workspace) return DSMOE_ERR_WORKSPACE;
  if (ws_bytes < SL.total) return DSMOE_ERR_WORKSPACE;
  if ((x && !aligned(x, 16)) || (y && !aligned(y, 16)) || !aligned(w->w13, 16) ||
      !aligned(w->w2, 16) || !aligned(w->router_w, 16) || !aligned(w->s13, 4) ||
      !aligned(w->s2, 4) || !aligned(bias, 4) || !aligned(counts_out, 4) ||
      !aligned(slot_first, 4) || !aligned(slot_expert, 4) || (workspace && !aligned(workspace, 256)) ||
      !debug_aligned(dbg))
    return DSMOE_ERR_ALIGN;
  if (d->n_shared && (!aligned(w->w13_sh, 16) || !aligned(w->w2_sh, 16) ||
                      !aligned(w->s13_sh, 4) || !aligned(w->s2_sh, 4)))
    return DSMOE_ERR_ALIGN;
  s = check_device();
  if (s != DSMOE_OK) return s;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t H = d->H, I = d->I;
  const int32_t E = d->E, K = d->K;
  const int64_t TK = T * K;
  const int32_t sh = d->n_shared ? 1 : 0;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* qx = ws + L.qx;
  float* sx = reinterpret_cast<float*>(ws + L.sx);
  float* logits = reinterpret_cast<float*>(ws + L.logits);
  int32_t* topk = reinterpret_cast<int32_t*>(ws + L.topk);
  float* gates = reinterpret_cast<float*>(ws + L.gates);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* offsets_ext = reinterpret_cast<int32_t*>(ws + L.offsets_ext);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + L.perm);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv);
  uint8_t* qa = ws + L.qa;
  float* sa = reinterpret_cast<float*>(ws + L.sa);
  void* o = ws + L.o;
  float* row_gate = reinterpret_cast<float*>(ws + SL.row_gate_all);
  int32_t* phys = reinterpret_cast<int32_t*>(ws + SL.phys);

#define DSMOE_TRY(expr)                                \
  do {                                                 \
    if ((expr) != hipSuccess) return DSMOE_ERR_LAUNCH; \
  } while (0)
  if (T == 0) {
    DSMOE_TRY(dsmoe::launch_route_select(nullptr, bias, 0, E, d->G, d->Mg, K, nullptr, nullptr,
                                         counts_out, st));
    return DSMOE_OK;
  }
#define DSMOE_MARK(i) \
  if (stage_events) DSMOE_TRY(hipEventRecord(static_cast<hipEvent_t>(stage_events[(i)]), st))
  DSMOE_MARK(0);
  // the steps of dsmoe_moe_forward up to the permute (perm extended by the
  // shared expert's identity rows when n_shared = 1)
  DSMOE_TRY(dsmoe::launch_quant_act(x, false, T, H, qx, sx, st));
  DSMOE_TRY(dsmoe::launch_router_logits(static_cast<const uint16_t*>(x),
                                        static_cast<const uint16_t*>(w->router_w), T, H, E, logits,
                                        reinterpret_cast<float*>(ws + L.router_part), st));
  DSMOE_TRY(dsmoe::launch_route_select(logits, bias, T, E, d->G, d->Mg, K, topk, gates, counts_out, st));
  DSMOE_TRY(dsmoe::launch_permute(topk, gates, T, E, K, counts_out, offsets, perm, inv, row_gate,
                                  sh ? offsets_ext : nullptr, st));
  // the shared expert as a routed one: gate 1 on its rows
  if (sh) DSMOE_TRY(dsmoe::launch_fill_f32(row_gate + TK, T, 1.0f, st));
  // expert offsets -> slot offsets (and the shared group's end)
  DSMOE_TRY(dsmoe::launch_slot_offsets(offsets, E, slot_first, slot_expert, n_slots, sh ? T : -1, phys, st));
  DSMOE_MARK(1);

  const int64_t rows = TK + (sh ? T : 0);
  const int64_t hint = (TK + n_slots - 1) / n_slots;
  dsmoe::GemmProblem g1{};
  g1.a = qx;
  g1.a_scale = sx;
  g1.a_rows = perm;
  g1.offsets = phys;
  g1.G = n_slots + sh;
  g1.M_total = rows;
  g1.w = w->w13;
  g1.w_scale = w->s13;
  g1.w_last = sh ? w->w13_sh : nullptr;
  g1.w_scale_last = sh ? w->s13_sh : nullptr;
  g1.N = 2 * I;
  g1.K = H;
  g1.c = qa;
  g1.c_scale = sa;
  g1.epi = dsmoe::Epilogue::kSwiGLUQuant;
  g1.row_limit = rows;
  g1.rows_hint = hint;
  g1.a_rows_total = T;
  DSMOE_TRY(dsmoe::launch_grouped_gemm(g1, st));
  DSMOE_MARK(2);

  dsmoe::GemmProblem g2{};
  g2.a = qa;
  g2.a_scale = sa;
  g2.offsets = phys;
  g2.G = n_slots + sh;
  g2.M_total = rows;
  g2.w = w->w2;
  g2.w_scale = w->s2;
  g2.w_last = sh ? w->w2_sh : nullptr;
  g2.w_scale_last = sh ? w->s2_sh : nullptr;
  g2.N = H;
  g2.K = I;
  g2.c = o;
  g2.c_f32 = yt == DSMOE_F32;
  g2.row_gate = row_gate;
  g2.epi = dsmoe::Epilogue::kGateStore;
  g2.row_limit = rows;
  g2.rows_hint = hint;
  g2.a_rows_total = rows;
  DSMOE_TRY(dsmoe::launch_grouped_gemm(g2, st));
  DSMOE_MARK(3);

  DSMOE_TRY(dsmoe::launch_combine(o, inv, T, K, H, sh ? TK : -1, y, yt == DSMOE_F32, st));
  DSMOE_MARK(4);
#undef DSMOE_MARK
  if (dbg) DSMOE_TRY(copy_debug(*dbg, *d, T, L, ws, st));
#undef DSMOE_TRY
  return DSMOE_OK;
}

int64_t dsmoe_token_tiles(int64_t M_total, int32_t G) {
  if (M_total < 0 || G < 1) return 0;
  return dsmoe::token_tiles(M_total, G);
}

dsmoe_status dsmoe_quant_tokens_128(const void* src, int src_type, int64_t n_src, int64_t C,
                                    const int32_t* rows, const float* row_scale, const int32_t* offsets,
                                    int32_t G, int64_t M_total, int32_t* chunk_off, uint8_t* qt,
                                    float* scales, void* stream) {
  if (!valid_dtype(src_type)) return DSMOE_ERR_DTYPE;
  if (G < 1 || G > 65536 || M_total < 0 || n_src < 0 || C <= 0 || C % 128) return DSMOE_ERR_SHAPE;
  if (!rows && n_src < M_total) return DSMOE_ERR_SHAPE;
  const int64_t tiles = dsmoe::token_tiles(M_total, G);
  if (tiles > kI32Max || C / 128 > 65535 || C * tiles * 128 > (1LL << 40)) return DSMOE_ERR_SHAPE;
  if (!offsets || !chunk_off) return DSMOE_ERR_NULL;
  if (M_total > 0 && (!src || !qt || !scales)) return DSMOE_ERR_NULL;
  if ((src && !aligned(src, 16)) || (qt && !aligned(qt, 16)) || (scales && !aligned(scales, 4)) ||
      !aligned(offsets, 4) || !aligned(chunk_off, 4) || (rows && !aligned(rows, 4)) ||
      (row_scale && !aligned(row_scale, 4)))
    return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  return launch_status(dsmoe::launch_quant_tokens(src, src_type == DSMOE_F32, C, rows, row_scale, offsets, G,
                                                  M_total, chunk_off, qt, scales,
                                                  static_cast<hipStream_t>(stream)));
}

dsmoe_status dsmoe_fp8_wgrad_grouped(const uint8_t* at, const float* sa, const uint8_t* bt, const float* sb,
                                     const int32_t* chunk_off, int32_t G, int64_t M, int64_t N, int64_t P,
                                     void* c, int ct, void* stream) {
  if (!valid_dtype(ct)) return DSMOE_ERR_DTYPE;
  if (G < 1 || M <= 0 || N <= 0 || M % 128 || N % 128 || P < 0 || P % 128) return DSMOE_ERR_SHAPE;
  if (static_cast<int64_t>(G) * (M / 128) * (N / 128) > kI32Max) return DSMOE_ERR_SHAPE;
  if (P >= (int64_t{1} << 32) / 128) return DSMOE_ERR_SHAPE;   // the kernel's 32-bit lane offsets
  if (!at || !sa || !bt || !sb || !chunk_off || !c) return DSMOE_ERR_NULL;
  if (!aligned(at, 16) || !aligned(bt, 16) || !aligned(c, 16) || !aligned(sa, 16) || !aligned(sb, 16) ||
      !aligned(chunk_off, 4))
    return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  return launch_status(dsmoe::launch_wgrad(at, sa, bt, sb, chunk_off, G, M, N, P, c, ct == DSMOE_F32,
                                           static_cast<hipStream_t>(stream)));
}

dsmoe_status dsmoe_swiglu_backward(const float* h, const float* da, const float* row_gate, int64_t rows,
                                   int64_t I, float* dh, float* a_out, void* stream) {
  if (rows < 0 || I <= 0 || I % 128 || rows > kI32Max) return DSMOE_ERR_SHAPE;
  if (rows == 0) return DSMOE_OK;
  if (!h || !da || !dh) return DSMOE_ERR_NULL;
  if (!aligned(h, 16) || !aligned(da, 16) || !aligned(dh, 16) || (a_out && !aligned(a_out, 16)) ||
      (row_gate && !aligned(row_gate, 4)))
    return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  return launch_status(dsmoe::launch_swiglu_bwd(h, da, row_gate, rows, I, dh, a_out,
                                                static_cast<hipStream_t>(stream)));
}

dsmoe_status dsmoe_gate_backward(const void* dy, const void* o, int ot, const int32_t* inv,
                                 const int32_t* topk_idx, const float* logits, int64_t T, int32_t E,
                                 int32_t K, int64_t H, float* dgate, float* dlogits, void* stream) {
  if (!valid_dtype(ot)) return DSMOE_ERR_DTYPE;
  if (T < 0 || T > kI32Max || K < 1 || K > DSMOE_MAX_TOPK || E < K || E > DSMOE_MAX_EXPERTS || H <= 0 ||
      H % 8)
    return DSMOE_ERR_SHAPE;
  if (T == 0) return DSMOE_OK;
  if (!dy || !o || !inv || !topk_idx || !logits || !dgate || !dlogits) return DSMOE_ERR_NULL;
  if (!aligned(dy, 16) || !aligned(o, 16) || !aligned(inv, 4) || !aligned(topk_idx, 4) || !aligned(logits, 4) ||
      !aligned(dgate, 4) || !aligned(dlogits, 4))
    return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  return launch_status(dsmoe::launch_gate_grad(static_cast<const uint16_t*>(dy), o, ot == DSMOE_F32, inv,
                                               topk_idx, logits, T, E, K, H, dgate, dlogits,
                                               static_cast<hipStream_t>(stream)));
}

dsmoe_status dsmoe_combine_rows(const void* o, int ot, const int32_t* inv, int64_t T, int32_t K, int64_t H,
                                int64_t shared0, void* y, void* stream) {
  if (!valid_dtype(ot)) return DSMOE_ERR_DTYPE;
  if (T < 0 || K < 1 || H <= 0 || H % 8 || T * (K + 1) > kI32Max) return DSMOE_ERR_SHAPE;
  if (T == 0) return DSMOE_OK;
  if (!o || !inv || !y) return DSMOE_ERR_NULL;
  if (!aligned(o, 16) || !aligned(y, 16) || !aligned(inv, 4)) return DSMOE_ERR_ALIGN;
  const dsmoe_status ds = check_device();
  if (ds != DSMOE_OK) return ds;
  return launch_status(dsmoe::launch_combine(o, inv, T, K, H, shared0, y, ot == DSMOE_F32,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
