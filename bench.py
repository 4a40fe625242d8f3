"""Benchmark of the DeepSeekMoE FP8 layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload v3_skew]

The default workload is the largest configuration: the DeepSeek-V3-shaped
layer on T = 32768 tokens whose expert popularity follows Zipf(1.1) (v3_skew).
It also reports the load imbalance before and after one bias update of the
aux-loss-free balancing (and re-route), and, outside the timed region, the
imbalance along a routing-only run of many updates.  v3_prefill (T = 4096)
and v3_decode (T = 64) are the other layer workloads.

The dense workload (--workload c2_dense) times one block-scaled FP8 GEMM
instead: A [4096][7168] and B [7168][4096] (passed as W [4096][7168]) from the
seeded recipe with 1% x50 outliers in A, quantised 1x128 / 128x128 on the
GPU, then dsmoe_fp8_grouped_gemm with one group, timed with its inputs warm
in the 256 MB MALL and with a 512 MB write between launches that evicts them.

The decode-serving workload (--workload v3_decode_serving) runs the V3
decode batch (T=64) through dsmoe_moe_forward_serving: the shared expert as a
9th routed expert and --extra-slots copies of hot experts (default 64: 256 +
64 slots), planned from the loads of one plain forward on the batch and
placed once before timing.  A step is the serving forward plus the bias
update; the plain decode step is timed in the same process for comparison.

The backward workload (--workload v3_prefill_backward) times the FP8
backward of the routed experts and the shared one at V3 prefill size on the
forward's own intermediates (routing, x codes, codes of a): h and the
ungated expert outputs recomputed by the grouped GEMM, the gate and
router-logit gradients, the dgrad of the down projection on the
block-transposed W2, the SwiGLU backward (recomputing a), the dgrad of the
gate/up projection summed per token, and the weight gradients of W2 and W13
on 1x128 tiles along each expert's tokens.  dy ~ N(0, 1) stands in for the
loss gradient.  The weights' block transposes run once per weight version
and are timed apart.

The granularity workload (--workload c2_granularity) runs the same GEMM
end to end from the bf16 operands at three scaling granularities (one scale
per tensor, per token x per output channel, and the recipe's 1x128 / 128x128
tiles) with dsmoe_fp8_gemm_granularity, and times each quantiser against the
HBM roofline.  Its value is the recipe path's rate (both quantisations and
the GEMM, float32 output); the error of each granularity against the float64
product of the unquantised inputs is reported beside it, on a 256-row sample.

A step is one pass of the whole hot path over one batch: dsmoe_moe_forward
(1x128 quantisation of x, router logits, group-limited top-8 routing,
permute, gate/up FP8 GEMM with SwiGLU and requantisation, routed and shared
down FP8 GEMMs, combine) followed by dsmoe_update_bias.  Weights are
quantised once before timing (dsmoe_quant_w_128x128 over every expert; its
time is reported separately as quant_w_ms).  Inputs are seeded synthetic
tensors already resident in HBM.  Prints one JSON line on stdout; progress
goes to stderr.
"""

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + grouped-GEMM FP8 TFLOP/s (% MFMA peak / % HBM BW) @1 GPU"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
RIDGE = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="v3_skew",
                    choices=["v3_prefill", "v3_decode", "v3_skew", "tiny", "c2_dense", "c2_granularity",
                             "v3_decode_serving", "v3_prefill_backward"])
    ap.add_argument("--extra-slots", type=int, default=64,
                    help="v3_decode_serving: copies of hot experts beyond one slot per expert")
    ap.add_argument("--out-dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--wgrad-dtype", default="bf16", choices=["bf16", "f32"],
                    help="v3_prefill_backward: dtype of the weight gradients")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="tokens of the batch the CPU oracle runs (default: 128 for v3_skew, whose tokens "
                         "share few experts, else 14; about 10-15 s of oracle work either way)")
    ap.add_argument("--balance-steps", type=int, default=1000,
                    help="layer workloads: routing-only bias updates for the imbalance trajectory (0: none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (3 times): the known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


COPY_BYTES = 1 << 30
def counters_file(workload):
    return os.path.join(ROOT, "profiles", f"counters_gemm1_swiglu_{workload}.json")
GEMM_SOURCES = ["gemm.hip", "common.h", "gemm.h"]


def gemm_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "fp8_block_scaled_dsmoe_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def gemm1_counters(workload):
    """The committed rocprofv3 counter record of the gate/up launch for this
    workload, or None when it was taken on other GEMM sources."""
    try:
        with open(counters_file(workload)) as fh:
            t = json.load(fh)
    except OSError:
        return None
    if t.get("workload") != workload or t.get("gemm_sources_sha256") != gemm_sources_sha256():
        return None
    return t


def measured_traffic(workload):
    """HBM bytes per launch of the gate/up GEMM (reads from the per-size TCC
    read-request counters, writes from the write-request counters), or None."""
    t = gemm1_counters(workload)
    return None if t is None or "traffic_bytes_per_launch" not in t else int(t["traffic_bytes_per_launch"])


def measured_traffic_algorithmic(workload):
    """Algorithmic bytes of the gate/up launches the traffic counters were
    taken on (their routing can differ from this run's), or None."""
    t = gemm1_counters(workload)
    return None if t is None else t.get("algorithmic_bytes_of_profiled_launches")


def measured_mfma(workload):
    """MFMA busy fraction of the gate/up launch from the counter record, or None."""
    t = gemm1_counters(workload)
    return None if t is None or "mfma_busy_frac" not in t else t["mfma_busy_frac"]


WGRAD_SOURCES = ["backward.hip", "common.h", "kernels.h"]


def wgrad_w13_traffic(wgrad_dtype):
    """HBM bytes of the W13 weight-gradient launch from its committed counter
    record (bf16 gradients), or None when the record was taken on other
    sources of that kernel."""
    import hashlib
    if wgrad_dtype != "bf16":
        return None
    try:
        with open(os.path.join(ROOT, "profiles", "counters_wgrad_w13_v3_prefill_backward.json")) as fh:
            t = json.load(fh)
    except OSError:
        return None
    h = hashlib.sha256()
    for f in WGRAD_SOURCES:
        with open(os.path.join(ROOT, "fp8_block_scaled_dsmoe_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return int(t["traffic_bytes_per_launch"]) if t.get("sources_sha256") == h.hexdigest() else None


def host_info():
    """CPU model and the BLAS NumPy uses (name, version, threads)."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                break
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas}


def copy_calibration(torch):
    src = torch.empty((COPY_BYTES,), dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}), flush=True)


def build_layer(cfg, d, torch, dsi):
    """Device inputs and FP8 weights; returns (x, bias, weights, quant_w_ms)."""
    E, H, I = cfg.E, cfg.H, cfg.I
    x, wr, bias = dsi.layer_activations_device(cfg, "cuda")
    if cfg.name == "tiny":
        inp = dsi.layer_inputs_host(cfg, 0)
        w13_all = torch.from_numpy(inp["w13"]).to(torch.bfloat16).cuda()
        w2_all = torch.from_numpy(inp["w2"]).to(torch.bfloat16).cuda()
    else:
        w13_all = torch.empty((E + 1, 2 * I, H), dtype=torch.bfloat16, device="cuda")
        w2_all = torch.empty((E + 1, H, I), dtype=torch.bfloat16, device="cuda")
        for e in range(E + 1):
            a, b = dsi.expert_weights_device(cfg, e, "cuda")
            w13_all[e].copy_(a)
            w2_all[e].copy_(b)
            del a, b
    q13 = torch.empty((E + 1, 2 * I, H), dtype=torch.uint8, device="cuda")
    s13 = torch.empty((E + 1, 2 * I // 128, H // 128), dtype=torch.float32, device="cuda")
    q2 = torch.empty((E + 1, H, I), dtype=torch.uint8, device="cuda")
    s2 = torch.empty((E + 1, H // 128, I // 128), dtype=torch.float32, device="cuda")
    times = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        d.quant_w_128x128(w13_all, q13, s13)
        d.quant_w_128x128(w2_all, q2, s2)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del w13_all, w2_all
    torch.cuda.empty_cache()
    weights = d.MoEWeights(q13[:E], s13[:E], q2[:E], s2[:E], q13[E], s13[E], q2[E], s2[E], wr)
    weights.stacked = (q13, s13, q2, s2)      # routed experts, then the shared one
    return x, bias, weights, statistics.median(times)


def imbalance(counts):
    """Load-balance figures of one routing: max/mean and coefficient of
    variation of the per-expert loads, experts with no load."""
    import numpy as np
    c = np.asarray(counts, np.float64)
    return {"max_over_mean": round(float(c.max() / c.mean()), 3),
            "cv": round(float(c.std() / c.mean()), 3),
            "zero_load_experts": int((c == 0).sum())}


def row_tile_fill(counts, T):
    """Rows of the gate/up GEMM's groups (the routed experts' counts, then the
    shared expert's T rows) over the rows of the row tiles covering them, for
    the 256-row tiles of the MFMA-bound kernel: the share of its MFMA row
    slots that hold a row."""
    import numpy as np
    rows = np.append(np.asarray(counts, np.int64), T)
    return round(float(rows.sum() / (np.ceil(rows / 256) * 256).sum()), 4)


def routing_trajectory(d, torch, logits, bias_init, cfg, n_steps):
    """Imbalance along n_steps aux-loss-free bias updates with routing only
    (dsmoe_route + dsmoe_update_bias on the batch's fixed logits), at a few
    step counts; untimed."""
    bias = bias_init.clone()
    marks = sorted({m for m in (0, 1, 10, 100, 300, 1000, 3000, n_steps) if m <= n_steps})
    out = {}
    for i in range(n_steps + 1):
        r = d.route(logits, bias, cfg.G, cfg.Mg, cfg.K)
        if i in marks:
            out[str(i)] = imbalance(r["counts"].cpu().numpy())
        d.update_bias(bias, r["counts"], cfg.T, cfg.K, 0.001)
    return out


def cpu_baseline(cfg, n_tokens, torch, dsi):
    """The oracle, as it stands, on a bounded sample: n_tokens tokens of the
    same batch through the whole layer (weight quantisation excluded, as on
    the GPU side)."""
    import numpy as np
    from oracle import layer as ol
    from oracle import quant as oq
    from oracle import route as orr
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    inp = dsi.layer_inputs_host(cfg, 0, with_weights=False)
    xs = inp["x"][:n_tokens]
    z, _ = ol.router_logits(xs, inp["router_w"])
    r = orr.route(z.astype(np.float32), inp["bias"], cfg.G, cfg.Mg, cfg.K)
    needed = sorted(set(r["topk_idx"].reshape(-1).tolist()) | {cfg.E})
    full = dsi.layer_inputs_host(cfg, 0) if cfg.name == "tiny" else None
    host_w = {}
    for e in needed:
        if full is not None:
            host_w[e] = (full["w13"][e], full["w2"][e])
        else:
            at, bt = dsi.expert_weights_device(cfg, e, "cuda")
            host_w[e] = (at.float().cpu().numpy(), bt.float().cpu().numpy())

    def quant(e):
        a, b = host_w.pop(e)
        return e, oq.quant_w_128x128(a) + oq.quant_w_128x128(b)

    from concurrent.futures import ThreadPoolExecutor
    log(f"cpu baseline: quantising {len(needed)} experts on the host (untimed)")
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as pool:
        cache = dict(pool.map(quant, needed))
    log(f"cpu baseline: oracle on {n_tokens} tokens, {len(needed)} experts")
    t0 = time.perf_counter()
    ol.moe_layer(xs, inp["router_w"], inp["bias"], lambda e: cache[e], cache[cfg.E], cfg.G, cfg.Mg, cfg.K)
    dt = time.perf_counter() - t0
    return {
        "value": n_tokens / dt, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle", **host_info(),
        "sample": f"{n_tokens} tokens of the {cfg.name} batch through the whole layer "
                  f"({len(needed)} experts incl. shared; float64 NumPy; weight quantisation excluded), "
                  f"{dt:.1f} s",
    }


def dense_cpu_baseline(a, w, n_rows):
    """The oracle GEMM, as it stands, on the first n_rows rows of A (float64,
    codes and scales from the oracle's own quantisers, untimed)."""
    from oracle import gemm as og
    from oracle import quant as oq
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    qa, sa = oq.quant_act_1x128(a[:n_rows])
    qw, sw = oq.quant_w_128x128(w)
    t0 = time.perf_counter()
    og.block_scaled_gemm(qa, sa, qw, sw)
    dt = time.perf_counter() - t0
    flops = 2.0 * n_rows * w.shape[0] * w.shape[1]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle", **host_info(),
            "sample": f"the first {n_rows} rows of A through the oracle GEMM (float64 NumPy, "
                      f"quantisation excluded), {dt:.1f} s"}


def run_dense(args, torch):
    import numpy as np
    import fp8_block_scaled_dsmoe_amd as d
    import dsmoe_inputs as dsi
    M, N, K = 4096, 4096, 7168
    out_dtype = torch.bfloat16 if args.out_dtype == "bf16" else torch.float32
    log(f"workload c2_dense: M={M} N={N} K={K}, 1% x50 outliers in A, y {args.out_dtype}")
    a, w = dsi.dense_gemm_inputs_host(M, N, K, seed=0)
    a_dev = torch.from_numpy(a).to("cuda").to(torch.bfloat16)
    w_dev = torch.from_numpy(w).to("cuda").to(torch.bfloat16)
    qa, sa = d.quant_act_1x128(a_dev)
    qw, sw = d.quant_w_128x128(w_dev)
    offsets = torch.tensor([0, M], dtype=torch.int32, device="cuda")
    c = torch.empty((M, N), dtype=out_dtype, device="cuda")
    flush = torch.empty((512 << 20,), dtype=torch.uint8, device="cuda")

    def gemm():
        d.fp8_grouped_gemm(qa, sa, offsets, qw.unsqueeze(0), sw.unsqueeze(0), c=c)

    def quant():
        d.quant_act_1x128(a_dev, qa, sa)

    for _ in range(args.warmup):
        quant()
        gemm()
    torch.cuda.synchronize()

    def timed(fn, flush_between):
        ts = []
        for _ in range(args.steps):
            if flush_between:
                flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)

    warm_ms = timed(gemm, False)
    cold_ms = timed(gemm, True)
    quant_ms = timed(quant, False)
    flops = 2.0 * M * N * K
    tf = flops / (warm_ms * 1e-3) / 1e12
    tf_cold = flops / (cold_ms * 1e-3) / 1e12
    log(f"GEMM {warm_ms * 1e3:.1f} us warm ({tf:.0f} TFLOP/s), {cold_ms * 1e3:.1f} us after a MALL flush "
        f"({tf_cold:.0f} TFLOP/s); quantising A {quant_ms * 1e3:.1f} us")
    result = {
        "metric": METRIC,
        "value": round(tf, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(warm_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"c2_dense: one block-scaled FP8 GEMM, M={M} N={N} K={K}, "
                               f"A with 1% x50 outliers, 1x128 / 128x128 scales, y {args.out_dtype}",
                   "M": M, "N": N, "K": K},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_FP8_TFLOPS, 4), "traffic": None,
                     "kernel": "dense block-scaled FP8 GEMM (256 x 256 tiles)",
                     "algorithmic_flops": flops, "avg_ms": round(warm_ms, 4)},
        "mall_flushed": {"ms": round(cold_ms, 4), "tflops": round(tf_cold, 2),
                         "frac": round(tf_cold / PEAK_FP8_TFLOPS, 4)},
        "quant_a_ms": round(quant_ms, 4),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = dense_cpu_baseline(a, w, 64)
    print(json.dumps(result), flush=True)


def granularity_cpu_baseline(a, w, n_rows):
    """The oracle's recipe path, as it stands: quantise the first n_rows rows
    of A (1x128) and all of W (128x128), then the float64 product."""
    from oracle import granularity as ogr
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    t0 = time.perf_counter()
    ah, wh = ogr.dequantised(a[:n_rows], w, "block")
    ah @ wh.T
    dt = time.perf_counter() - t0
    flops = 2.0 * n_rows * w.shape[0] * w.shape[1]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle", **host_info(),
            "sample": f"the first {n_rows} rows of A through the oracle's block-granularity path "
                      f"(quantisation of the A rows and all of W included; float64 NumPy), {dt:.1f} s"}


def run_granularity(args, torch):
    import numpy as np
    import fp8_block_scaled_dsmoe_amd as d
    import dsmoe_inputs as dsi
    M, N, K = 4096, 4096, 7168
    log(f"workload c2_granularity: M={M} N={N} K={K}, 1% x50 outliers in A, c float32")
    a, w = dsi.dense_gemm_inputs_host(M, N, K, seed=0)
    a_dev = torch.from_numpy(a).to("cuda").to(torch.bfloat16)
    w_dev = torch.from_numpy(w).to("cuda").to(torch.bfloat16)
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty((d.gemm_granularity_workspace_bytes(M, N, K),), dtype=torch.uint8, device="cuda")
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa_t = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    sa_r = torch.empty((M,), dtype=torch.float32, device="cuda")
    s1 = torch.empty((1,), dtype=torch.float32, device="cuda")
    am = torch.empty((d.QUANT_TENSOR_SCRATCH_FLOATS,), dtype=torch.float32, device="cuda")

    def timed(fn, reps=1):
        """Median over the steps of (event time around `reps` back-to-back calls) / reps."""
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / reps)
        return statistics.median(ts)

    flops = 2.0 * M * N * K
    rows = np.arange(256)
    exact = a[rows].astype(np.float64) @ w.astype(np.float64).T
    d_norm = np.abs(a[rows]).astype(np.float64) @ np.abs(w).astype(np.float64).T
    grans = {}
    for g in ("tensor", "channel", "block"):
        ms = timed(lambda: d.fp8_gemm_granularity(a_dev, w_dev, g, c=c, workspace=ws))
        d.fp8_gemm_granularity(a_dev, w_dev, g, c=c, workspace=ws)
        cs = c[:256].cpu().numpy().astype(np.float64)
        grans[g] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                    "rel_frobenius": float(np.linalg.norm(cs - exact) / np.linalg.norm(exact)),
                    "max_norm_err": float((np.abs(cs - exact) / d_norm).max())}
        log(f"{g:8s} {ms * 1e3:8.1f} us end to end ({grans[g]['tflops']:.0f} TFLOP/s), "
            f"rel. Frobenius error {grans[g]['rel_frobenius']:.4f}, max normalised {grans[g]['max_norm_err']:.4f}")

    # the quantisers on A alone, 10 launches per timed interval (a single ~20 us
    # launch would carry the launch latency): algorithmic bytes = 2 (bf16 read)
    # + 1 (code) per element + scales
    elems = M * K
    quants = {
        "quant_act_1x128": (lambda: d.quant_act_1x128(a_dev, qa, sa_t), 3 * elems + 4 * elems // 128),
        "quant_rows": (lambda: d.quant_rows(a_dev, qa, sa_r), 3 * elems + 4 * M),
        "quant_tensor": (lambda: d.quant_tensor(a_dev, qa, s1, am), 3 * elems + 8),
    }
    qres = {}
    for name, (fn, nbytes) in quants.items():
        ms = timed(fn, reps=10)
        gbps = nbytes / (ms * 1e-3) / 1e9
        qres[name] = {"ms": round(ms, 4), "algorithmic_bytes": nbytes, "gbps": round(gbps, 1),
                      "frac": round(gbps / PEAK_HBM_GBPS, 4)}
        log(f"{name:16s} {ms * 1e3:7.1f} us, {gbps:.0f} GB/s of algorithmic bytes "
            f"({gbps / PEAK_HBM_GBPS:.0%} of HBM peak)")
    qres["quant_tensor"]["note"] = "two passes over x (amax, then codes): 5 B per element moved, 3 counted"

    # the dominant kernel: the GEMM of the recipe path (float32 output), alone
    d.fp8_gemm_granularity(a_dev, w_dev, "block", c=c, workspace=ws)
    qa_b, sa_b = d.quant_act_1x128(a_dev)
    qw_b, sw_b = d.quant_w_128x128(w_dev)
    offsets = torch.tensor([0, M], dtype=torch.int32, device="cuda")
    gemm_ms = timed(lambda: d.fp8_grouped_gemm(qa_b, sa_b, offsets, qw_b.unsqueeze(0), sw_b.unsqueeze(0), c=c))
    tf_gemm = flops / (gemm_ms * 1e-3) / 1e12
    log(f"GEMM alone {gemm_ms * 1e3:.1f} us ({tf_gemm:.0f} TFLOP/s)")
    val = grans["block"]["tflops"]
    result = {
        "metric": METRIC,
        "value": val,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": grans["block"]["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"c2_granularity: quantise A [{M}][{K}] and W [{N}][{K}] from bf16 and run "
                               f"the FP8 GEMM, at per-tensor, per-token x per-channel and 1x128 / 128x128 "
                               f"scaling, c float32",
                   "M": M, "N": N, "K": K},
        "roofline": {"bound": "mfma", "achieved": round(tf_gemm, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf_gemm / PEAK_FP8_TFLOPS, 4), "traffic": None,
                     "kernel": "dense block-scaled FP8 GEMM (256 x 256 tiles), float32 output",
                     "algorithmic_flops": flops, "avg_ms": round(gemm_ms, 4)},
        "granularities": grans,
        "quantisers_on_A": qres,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = granularity_cpu_baseline(a, w, M)
    print(json.dumps(result), flush=True)


def run_serving(args, torch):
    import numpy as np
    import fp8_block_scaled_dsmoe_amd as d
    import dsmoe_inputs as dsi
    cfg = dsi.LAYER_CONFIGS["v3_decode"]
    out_dtype = torch.bfloat16 if args.out_dtype == "bf16" else torch.float32
    T, H, I, E, K = cfg.T, cfg.H, cfg.I, cfg.E, cfg.K
    R = args.extra_slots
    S = E + R
    log(f"workload v3_decode_serving: T={T} H={H} E={E} G={cfg.G} Mg={cfg.Mg} K={K} I={I}, "
        f"{R} extra slots, shared expert as a routed group")
    x, bias, weights, quant_w_ms = build_layer(cfg, d, torch, dsi)
    desc = d.MoEDesc(H, I, E, cfg.G, cfg.Mg, K, 1)
    y = torch.empty((T, H), dtype=out_dtype, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    ws_plain = torch.empty((d.moe_workspace_bytes(desc, T),), dtype=torch.uint8, device="cuda")
    ws_srv = torch.empty((d.moe_serving_workspace_bytes(desc, T, S),), dtype=torch.uint8, device="cuda")
    bias0 = bias.clone()

    # observed loads: one plain forward on the batch (the bias is not updated)
    d.moe_forward(desc, weights, bias, x, y=y, counts=counts, workspace=ws_plain)
    observed = counts.clone()

    def once(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        out = fn()
        e1.record()
        torch.cuda.synchronize()
        return out, e0.elapsed_time(e1)

    (slot_first, slot_expert), _ = once(lambda: d.plan_replicas(observed, R))      # warm
    (slot_first, slot_expert), plan_ms = once(lambda: d.plan_replicas(observed, R))
    slot_w, place_ms = once(lambda: d.place_layer_replicas(weights, slot_expert))
    place_bytes = 2 * S * (3 * H * I + ((2 * I // 128) * (H // 128) + (H // 128) * (I // 128)) * 4)

    def timed_steps(step, n_ev):
        for _ in range(args.warmup):
            step(None)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
        for row in ev:
            for e in row:
                e.record()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for i in range(args.steps):
            step(ev[i])
        t1.record()
        torch.cuda.synchronize()
        stages = [statistics.mean(r[j].elapsed_time(r[j + 1]) for r in ev) for j in range(n_ev - 1)]
        return t0.elapsed_time(t1) / args.steps, stages

    def plain(ev):
        d.moe_forward(desc, weights, bias, x, y=y, counts=counts, workspace=ws_plain,
                      stage_events=None if ev is None else [e.cuda_event for e in ev])
        d.update_bias(bias, counts, T, K, 0.001)

    def serving(ev):
        d.moe_forward_serving(desc, slot_w, slot_first, slot_expert, bias, x, y=y, counts=counts,
                              workspace=ws_srv, stage_events=None if ev is None else [e.cuda_event for e in ev])
        d.update_bias(bias, counts, T, K, 0.001)

    # no extra slots: only the shared expert joins the routed launches
    sf0, se0 = d.plan_replicas(observed, 0)
    slot_w0 = d.place_layer_replicas(weights, se0)
    ws0 = torch.empty((d.moe_serving_workspace_bytes(desc, T, E),), dtype=torch.uint8, device="cuda")

    def serving0(ev):
        d.moe_forward_serving(desc, slot_w0, sf0, se0, bias, x, y=y, counts=counts, workspace=ws0,
                              stage_events=None if ev is None else [e.cuda_event for e in ev])
        d.update_bias(bias, counts, T, K, 0.001)

    plain_ms, plain_st = timed_steps(plain, d.STAGE_EVENTS)
    bias.copy_(bias0)
    srv0_ms, srv0_st = timed_steps(serving0, d.SERVING_STAGE_EVENTS)
    del slot_w0
    torch.cuda.empty_cache()
    bias.copy_(bias0)
    srv_ms, srv_st = timed_steps(serving, d.SERVING_STAGE_EVENTS)
    srv_stage = dict(zip(d.SERVING_STAGES, srv_st))
    plain_stage = dict(zip(d.STAGES, plain_st))
    log(f"plain decode {plain_ms:.3f} ms/step; serving without copies {srv0_ms:.3f}; "
        f"serving {srv_ms:.3f} ms/step; serving stages " +
        ", ".join(f"{k} {v:.3f}" for k, v in srv_stage.items()))

    # loads of the last step over the plan's slots
    c_last = counts.cpu().numpy()
    off = torch.tensor(np.concatenate([[0], np.cumsum(c_last)]), dtype=torch.int32, device="cuda")
    phys = d.slot_offsets(off, slot_first, slot_expert, T).cpu().numpy()
    rows_slot = np.diff(phys[:S + 1])
    active = int(np.count_nonzero(rows_slot))
    obs = observed.cpu().numpy()
    n_rep = np.diff(slot_first.cpu().numpy())
    rows1 = T * K + T
    g1_bytes = ((active + 1) * 2 * I * H + (active + 1) * (2 * I // 128) * (H // 128) * 4 +
                T * H + T * (H // 128) * 4 + rows1 * I + rows1 * (I // 128) * 4)
    g1_ms = srv_stage["gemm1_swiglu_requant"]
    g1_gbps = g1_bytes / (g1_ms * 1e-3) / 1e9
    w_bytes = (active + 1) * 3 * H * I
    layer_gbps = (w_bytes + T * H * 4 + E * H * 2) / (srv_ms * 1e-3) / 1e9
    log(f"slots holding rows: {active} of {S}; max rows per slot {rows_slot.max()} (per expert "
        f"{c_last.max()}); plan {plan_ms * 1e3:.1f} us, placement {place_ms:.2f} ms "
        f"({place_bytes / (place_ms * 1e-3) / 1e9:.0f} GB/s)")
    result = {
        "metric": METRIC,
        "value": round(T / (srv_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(srv_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"v3_decode_serving: DeepSeekMoE layer forward over {S} expert slots "
                               f"({R} copies of hot experts planned from observed loads) with the shared "
                               f"expert as a 9th routed expert, + bias update, T={T}, H={H}, E={E}, "
                               f"top-{K} within {cfg.Mg} of {cfg.G} groups, I={I}, y {args.out_dtype}",
                   "T": T, "H": H, "E": E, "G": cfg.G, "Mg": cfg.Mg, "K": K, "I": I, "slots": S},
        "roofline": {"bound": "hbm", "achieved": round(g1_gbps, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(g1_gbps / PEAK_HBM_GBPS, 4), "traffic": measured_traffic("v3_decode_serving"),
                     "kernel": "gate/up grouped FP8 GEMM + SwiGLU + 1x128 requant over the slots (one launch)",
                     "algorithmic_bytes": int(g1_bytes), "avg_ms": round(g1_ms, 4)},
        "layer_hbm_gbps": round(layer_gbps, 1),
        "layer_frac_hbm_peak": round(layer_gbps / PEAK_HBM_GBPS, 4),
        "stage_ms": {k: round(v, 4) for k, v in srv_stage.items()},
        "plain_decode": {"ms_per_step": round(plain_ms, 4), "tokens_per_s": round(T / (plain_ms * 1e-3), 1),
                         "stage_ms": {k: round(v, 4) for k, v in plain_stage.items()}},
        "serving_without_copies": {"ms_per_step": round(srv0_ms, 4),
                                   "tokens_per_s": round(T / (srv0_ms * 1e-3), 1),
                                   "stage_ms": {k: round(v, 4) for k, v in
                                                zip(d.SERVING_STAGES, srv0_st)}},
        "slots": {"total": S, "holding_rows_last_step": active,
                  "max_rows_per_slot_last_step": int(rows_slot.max()),
                  "max_rows_per_expert_last_step": int(c_last.max()),
                  "planned_from_max_load": int(obs.max()),
                  "planned_max_load_per_slot": round(float((obs / n_rep).max()), 3),
                  "max_copies_of_one_expert": int(n_rep.max())},
        "plan_us": round(plan_ms * 1e3, 2),
        "placement_ms": round(place_ms, 3),
        "placement_gbps": round(place_bytes / (place_ms * 1e-3) / 1e9, 1),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_tokens or 14, torch, dsi)
        result["cpu_baseline"]["sample"] += " (the serving forward computes the same layer)"
    print(json.dumps(result), flush=True)


def run_backward(args, torch):
    import fp8_block_scaled_dsmoe_amd as d
    import dsmoe_inputs as dsi
    cfg = dsi.LAYER_CONFIGS["v3_prefill"]
    T, H, I, E, K = cfg.T, cfg.H, cfg.I, cfg.E, cfg.K
    rows = T * K + T
    wdt = torch.bfloat16 if args.wgrad_dtype == "bf16" else torch.float32
    log(f"workload v3_prefill_backward: T={T} H={H} E={E} K={K} I={I}, routed experts + shared, "
        f"weight gradients {args.wgrad_dtype}")
    x, bias, weights, _ = build_layer(cfg, d, torch, dsi)
    desc = d.MoEDesc(H, I, E, cfg.G, cfg.Mg, K, 1)
    _, counts, dbg = d.moe_forward(desc, weights, bias, x, debug=True)
    w = weights.stacked
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    dy = torch.randn((T, H), device="cuda", generator=g).to(torch.bfloat16)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)

    # the weights' block transposes: once per weight version, outside the step
    t_tr = timed(lambda: (d.transpose_w_128x128(w[0], w[1]), d.transpose_w_128x128(w[2], w[3])))
    wt = d.transpose_w_128x128(w[0], w[1]) + d.transpose_w_128x128(w[2], w[3])
    for _ in range(args.warmup):
        d.moe_backward_experts(dbg, x, dy, w, wt, T, K, wgrad_dtype=wdt)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(9)] for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        out = d.moe_backward_experts(dbg, x, dy, w, wt, T, K, wgrad_dtype=wdt, stage_events=ev[i])
        del out
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    stage = {n: statistics.mean(r[j].elapsed_time(r[j + 1]) for r in ev) for j, n in enumerate(d.BACKWARD_STAGES)}
    touched = int((counts > 0).sum().item()) + 1
    gb = lambda b, t: b / (t * 1e-3) / 1e9
    tf = lambda f, t: f / (t * 1e-3) / 1e12
    # FP8 GEMM flops of the step: recomputed h (2I x H) and o (H x I), the two
    # dgrads and the two weight gradients
    gemm_flops = 2.0 * rows * H * I * (2 + 1 + 1 + 2 + 1 + 2)
    esz = 2 if wdt == torch.bfloat16 else 4
    w13_out = (E + 1) * 2 * I * H * esz
    # the weight gradient of W13: every expert's [2I][H] written once, plus the
    # token-tile codes and scales of dh and x it reads (x read once per expert)
    wg13_bytes = w13_out + rows * (2 * I + H) + rows // 128 * (2 * I + H) * 4
    wg13_ms = stage["wgrad_w13"]
    log(f"{args.steps} steps: {ms:.3f} ms/step; stages " + ", ".join(f"{k} {v:.3f}" for k, v in stage.items()) +
        f"; transposes {t_tr:.3f} ms per weight version")
    result = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic (dy ~ N(0,1) stands in for the loss gradient; every other input is the forward's)",
        "config": {"workload": f"v3_prefill_backward: FP8 backward of the routed and shared experts on the "
                               f"forward's intermediates (recomputed h and o, gate and router-logit gradients, "
                               f"both dgrads, SwiGLU backward, both weight gradients in {args.wgrad_dtype}), "
                               f"T={T}, H={H}, E={E}, top-{K}, I={I}",
                   "T": T, "H": H, "E": E, "K": K, "I": I},
        "roofline": {"bound": "hbm", "achieved": round(gb(wg13_bytes, wg13_ms), 2), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(gb(wg13_bytes, wg13_ms) / PEAK_HBM_GBPS, 4),
                     "traffic": wgrad_w13_traffic(args.wgrad_dtype),
                     "kernel": "weight gradient of W13 (grouped FP8 Wgrad GEMM over each expert's tokens)",
                     "algorithmic_bytes": int(wg13_bytes), "avg_ms": round(wg13_ms, 4)},
        "grouped_gemm_tflops": round(tf(gemm_flops, ms), 2),
        "grouped_gemm_frac_mfma_peak": round(tf(gemm_flops, ms) / PEAK_FP8_TFLOPS, 4),
        "stage_ms": {k: round(v, 4) for k, v in stage.items()},
        "transpose_ms_per_weight_version": round(t_tr, 4),
        "experts_touched": touched,
    }
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.workload == "c2_dense":
        run_dense(args, torch)
        return
    if args.workload == "c2_granularity":
        run_granularity(args, torch)
        return
    if args.workload == "v3_decode_serving":
        run_serving(args, torch)
        return
    if args.workload == "v3_prefill_backward":
        run_backward(args, torch)
        return
    import fp8_block_scaled_dsmoe_amd as d
    import dsmoe_inputs as dsi

    cfg = dsi.LAYER_CONFIGS[args.workload]
    out_dtype = torch.bfloat16 if args.out_dtype == "bf16" else torch.float32
    T, H, I, E, K = cfg.T, cfg.H, cfg.I, cfg.E, cfg.K
    log(f"workload {cfg.name}: T={T} H={H} E={E} G={cfg.G} Mg={cfg.Mg} K={K} I={I}")
    x, bias, weights, quant_w_ms = build_layer(cfg, d, torch, dsi)
    log(f"weights quantised: {quant_w_ms:.2f} ms for {E + 1} experts")
    desc = d.MoEDesc(H, I, E, cfg.G, cfg.Mg, K, 1)
    ws = torch.empty((d.moe_workspace_bytes(desc, T),), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, H), dtype=out_dtype, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")

    def step(ev=None):
        d.moe_forward(desc, weights, bias, x, y=y, counts=counts, workspace=ws,
                      stage_events=None if ev is None else [e.cuda_event for e in ev])
        d.update_bias(bias, counts, T, K, 0.001)

    # Load balance: the routing of the batch with the initial bias, then one
    # bias update (the step's own) and the re-route.
    import numpy as np
    bias_init = bias.clone()
    _, _, dbg0 = d.moe_forward(desc, weights, bias, x, y=y, counts=counts, workspace=ws, debug=True)
    counts_before = counts.cpu().numpy()
    d.update_bias(bias, counts, T, K, 0.001)
    d.moe_forward(desc, weights, bias, x, y=y, counts=counts, workspace=ws)
    counts_after1 = counts.cpu().numpy()
    bias.copy_(bias_init)
    balance = {"before": imbalance(counts_before), "after_one_update": imbalance(counts_after1)}
    if args.balance_steps > 0:
        balance["routing_only_trajectory"] = routing_trajectory(d, torch, dbg0["logits"], bias_init, cfg,
                                                                args.balance_steps)
    del dbg0
    log("load imbalance (max/mean): before " + f"{balance['before']['max_over_mean']:.3f}, after one update "
        f"{balance['after_one_update']['max_over_mean']:.3f}")
    # (with no warm-up and two timed steps, the run's gate/up launches route
    # exactly so: initial, updated, initial, updated -- the bias is reset
    # above -- which sets a profiled run's traffic against those launches'
    # own algorithmic bytes)
    log(f"experts touched: {int(np.count_nonzero(counts_before))} with the initial bias, "
        f"{int(np.count_nonzero(counts_after1))} after one update")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(d.STAGE_EVENTS)] for _ in range(args.steps)]
    for row in ev:
        for e in row:
            e.record()          # creates the underlying event
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step(ev[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    stage_ms = {}
    for s_i, name in enumerate(d.STAGES):
        stage_ms[name] = statistics.mean(r[s_i].elapsed_time(r[s_i + 1]) for r in ev)
    log(f"{args.steps} steps: {ms_step:.3f} ms/step (wall {1e3 * wall / args.steps:.3f}); stages " +
        ", ".join(f"{k} {v:.3f}" for k, v in stage_ms.items()))

    counts_last = counts.cpu().numpy()
    touched = int(np.count_nonzero(counts_last))
    rows1 = T * K + T
    # algorithmic work
    gemm_flops = 6.0 * rows1 * H * I                      # gate/up + down, routed + shared
    w_bytes = (touched + 1) * 3 * H * I                   # FP8 weights of the experts touched
    s_bytes = (touched + 1) * ((2 * I // 128) * (H // 128) + (H // 128) * (I // 128)) * 4
    io_bytes = T * H * 2 + T * H * (2 if out_dtype == torch.bfloat16 else 4) + E * H * 2
    layer_bytes = w_bytes + s_bytes + io_bytes
    tok_s = T / (ms_step * 1e-3)
    # dominant kernel: gate/up GEMM + SwiGLU + requant
    g1_flops = 2.0 * rows1 * H * 2 * I
    g1_bytes = ((touched + 1) * 2 * I * H + (touched + 1) * (2 * I // 128) * (H // 128) * 4 +
                T * H + T * (H // 128) * 4 + rows1 * I + rows1 * (I // 128) * 4)
    g1_ms = stage_ms["gemm1_swiglu_requant"]
    g1_bound = "hbm" if g1_flops / g1_bytes < RIDGE else "mfma"
    if g1_bound == "hbm":
        achieved, peak, unit = g1_bytes / (g1_ms * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"
    else:
        achieved, peak, unit = g1_flops / (g1_ms * 1e-3) / 1e12, PEAK_FP8_TFLOPS, "TFLOP/s"
    gemm_ms = g1_ms + stage_ms["gemm2_routed"] + stage_ms["gemm2_shared_combine"]

    result = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: DeepSeekMoE layer forward + bias update, T={T}, H={H}, "
                               f"E={E} in G={cfg.G} groups, top-{K} within {cfg.Mg} groups, "
                               f"1 shared expert, I={I}, y {args.out_dtype}" +
                               (f", expert popularity Zipf({cfg.zipf_s}) through the router logits"
                                if cfg.zipf_s else ""),
                   "T": T, "H": H, "E": E, "G": cfg.G, "Mg": cfg.Mg, "K": K, "I": I},
        "roofline": {"bound": g1_bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(cfg.name),
                     "traffic_algorithmic_bytes": measured_traffic_algorithmic(cfg.name),
                     "mfma_busy_frac": measured_mfma(cfg.name),
                     "kernel": "gate/up grouped FP8 GEMM + SwiGLU + 1x128 requant (one launch)",
                     "algorithmic_bytes": int(g1_bytes), "algorithmic_flops": g1_flops,
                     "avg_ms": round(g1_ms, 4)},
        "grouped_gemm_tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 2),
        "grouped_gemm_frac_mfma_peak": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
        "layer_tflops": round(gemm_flops / (ms_step * 1e-3) / 1e12, 2),
        "layer_frac_mfma_peak": round(gemm_flops / (ms_step * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
        "layer_hbm_gbps": round(layer_bytes / (ms_step * 1e-3) / 1e9, 1),
        "layer_frac_hbm_peak": round(layer_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "layer_algorithmic_bytes": int(layer_bytes),
        "experts_touched": touched,
        "row_tile_fill": row_tile_fill(counts_last, T),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "quant_w_ms": round(quant_w_ms, 3),
        "load_balance": dict(balance, last_timed_step=imbalance(counts_last)),
    }
    if not args.no_cpu_baseline:
        n_cpu = args.cpu_tokens if args.cpu_tokens is not None else (128 if cfg.zipf_s else 14)
        result["cpu_baseline"] = cpu_baseline(cfg, n_cpu, torch, dsi)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
