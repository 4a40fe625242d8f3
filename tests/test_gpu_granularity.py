"""GPU parity of the coarser scaling granularities (dsmoe_quant_rows,
dsmoe_quant_tensor, dsmoe_fp8_gemm_granularity) against oracle.granularity.

Codes and scales must match bit for bit.  The GEMM meets the block-scaled
GEMM's bar: max |gpu - oracle| / (|A_hat| |W_hat|^T) <= 2e-3 for its float32
output, where A_hat, W_hat are the oracle's dequantised operands."""

import numpy as np
import pytest
import torch

from dsmoe_inputs import dense_gemm_inputs_host, normal_bf16
from gpu_util import assert_normalised_close, banner, dev, host
from oracle import granularity as og

pytestmark = pytest.mark.gpu

TOL = 2e-3
OUT = np.float32(448.0 * 448.0 * 1024.0)


def _d():
    import fp8_block_scaled_dsmoe_amd as d
    return d


def _same_bits(got, want, what):
    got = np.asarray(got, np.float32).reshape(-1)
    want = np.asarray(want, np.float32).reshape(-1)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{what}: scales differ"


def _same_codes(got, want, what):
    bad = np.argwhere(np.asarray(got) != np.asarray(want))
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first {bad[:5].tolist()}"


def _input(rows, cols, f32, seed):
    """Dense-workload activations (N(0,1), 1% x50 outliers); the float32
    variant is scaled by 1.37 so that it is no longer bf16-representable."""
    a, _ = dense_gemm_inputs_host(rows, 8, cols, seed=seed)
    if f32:
        a = (a * np.float32(1.37)).astype(np.float32)
    return a


# ---------------------------------------------------------------------------
# per-row quantiser

@pytest.mark.parametrize("rows,cols", [(1, 8), (3, 136), (257, 1000), (64, 7168), (5, 32768)])
@pytest.mark.parametrize("f32", [False, True])
def test_quant_rows_matches_oracle(rows, cols, f32):
    banner(f"quant_rows {rows}x{cols} f32={f32}")
    x = _input(rows, cols, f32, seed=cols)
    q, s = _d().quant_rows(dev(x, torch.float32 if f32 else torch.bfloat16))
    qo, so = og.quant_rows(x)
    _same_bits(host(s), so, "quant_rows")
    _same_codes(host(q), qo, "quant_rows")


def test_quant_rows_special_rows():
    """An all-zero row (scale 1), the closed-form outlier rows, a row of
    negative values, and one whose amax sits in its last element."""
    banner("quant_rows special rows")
    x = np.full((5, 256), 448.0, np.float32)
    x[0, 0] = OUT
    x[2] = 0.0
    x[3] = -x[1]
    x[4] = np.linspace(-1.0, 1.0, 256, dtype=np.float32)
    x[4, -1] = 3.0
    q, s = _d().quant_rows(dev(x, torch.float32))
    qo, so = og.quant_rows(x)
    _same_bits(host(s), so, "special rows")
    _same_codes(host(q), qo, "special rows")
    assert host(s)[2] == 1.0 and np.all(host(q)[2] == 0)
    assert host(s)[0] == np.float32(458752.0) and np.all(host(q)[0, 1:] == 0)


# ---------------------------------------------------------------------------
# per-tensor quantiser

@pytest.mark.parametrize("shape", [(1, 8), (37, 136), (300, 7168), (2048 * 2 + 3, 1024), (8200, 1024),
                                   (5000, 8192)])
@pytest.mark.parametrize("f32", [False, True])
def test_quant_tensor_matches_oracle(shape, f32):
    """Sizes from one partial block to a full grid whose threads hold from
    one to eight loads in flight (8200 x 1024: 1,049,600 vectors over a grid
    of 524,288 threads, so 2 or 3 each), 5000 x 8192 (5,120,000 vectors: the
    outer loop runs twice), and the 4096 x 7168 case below (7 each)."""
    banner(f"quant_tensor {shape} f32={f32}")
    x = _input(shape[0], shape[1], f32, seed=shape[0])
    q, s, amax = _d().quant_tensor(dev(x, torch.float32 if f32 else torch.bfloat16))
    qo, so = og.quant_tensor(x)
    assert host(amax)[0] == np.max(np.abs(x))
    _same_bits(host(s), so, "quant_tensor")
    _same_codes(host(q), qo, "quant_tensor")


def test_quant_tensor_closed_form_and_empty():
    d = _d()
    banner("quant_tensor closed form")
    a = np.full((2, 256), 448.0, np.float32)
    a[0, 0] = OUT
    for dt in (torch.bfloat16, torch.float32):
        q, s, amax = d.quant_tensor(dev(a, dt))
        assert host(s)[0] == np.float32(458752.0) and host(amax)[0] == OUT
        qg = host(q).reshape(-1)
        assert qg[0] == 0x7E and np.all(qg[1:] == 0)   # 448 / s = 2^-10, the tie, goes to 0
    banner("quant_tensor empty")
    e = torch.empty((0,), dtype=torch.bfloat16, device="cuda")
    q, s, amax = d.quant_tensor(e)
    assert host(amax)[0] == 0.0 and host(s)[0] == 1.0


def test_quant_tensor_reused_amax_slot():
    """A second call on a smaller-magnitude tensor with the same amax slot
    starts from 0, not from the first call's maximum."""
    d = _d()
    banner("quant_tensor reused slot")
    big = normal_bf16("gran_big", (64, 256), 10.0, seed=1)
    small = normal_bf16("gran_small", (64, 256), 0.01, seed=1)
    scratch = torch.empty((d.QUANT_TENSOR_SCRATCH_FLOATS,), dtype=torch.float32, device="cuda")
    scale = torch.empty((1,), dtype=torch.float32, device="cuda")
    d.quant_tensor(dev(big, torch.bfloat16), scale=scale, scratch=scratch)
    q, s, a2 = d.quant_tensor(dev(small, torch.bfloat16), scale=scale, scratch=scratch)
    qo, so = og.quant_tensor(small)
    assert host(a2)[0] == np.max(np.abs(small))
    _same_bits(host(s), so, "second call")
    _same_codes(host(q), qo, "second call")


def test_quant_tensor_full_size():
    """The dense workload's A (4096 x 7168) as the GEMM path quantises it."""
    banner("quant_tensor 4096x7168")
    a, _ = dense_gemm_inputs_host(4096, 8, 7168, seed=0)
    q, s, _ = _d().quant_tensor(dev(a, torch.bfloat16))
    qo, so = og.quant_tensor(a)
    _same_bits(host(s), so, "full size")
    _same_codes(host(q), qo, "full size")


# ---------------------------------------------------------------------------
# GEMM at each granularity

def _check_gemm(a, w, g, dt, what, rows=None):
    c = _d().fp8_gemm_granularity(dev(a, dt), dev(w, dt), g)
    ah, wh = og.dequantised(a, w, g)
    if rows is not None:
        ah = ah[rows]
    want = ah @ wh.T
    norm = np.abs(ah) @ np.abs(wh).T
    got = host(c) if rows is None else host(c)[rows]
    return assert_normalised_close(got, want, norm, TOL, f"{what} {g}")


@pytest.mark.parametrize("g", og.GRANULARITIES)
@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (77, 256, 384), (300, 384, 1024), (129, 512, 7168)])
def test_gemm_granularity_matches_oracle(g, M, N, K):
    banner(f"gemm_granularity {g} M={M} N={N} K={K}")
    a, w = dense_gemm_inputs_host(M, N, K, seed=M + K)
    _check_gemm(a, w, g, torch.bfloat16, f"{M}x{N}x{K}")


@pytest.mark.parametrize("g", og.GRANULARITIES)
def test_gemm_granularity_f32_inputs(g):
    banner(f"gemm_granularity f32 {g}")
    a, w = dense_gemm_inputs_host(200, 256, 640, seed=5)
    a = (a * np.float32(1.37)).astype(np.float32)
    w = (w * np.float32(0.71)).astype(np.float32)
    _check_gemm(a, w, g, torch.float32, "f32 200x256x640")


@pytest.mark.parametrize("g", og.GRANULARITIES)
def test_gemm_granularity_closed_forms(g):
    """The oracle pins' closed forms, through the GPU: exact products."""
    banner(f"gemm_granularity closed forms {g}")
    a = np.full((2, 256), 448.0, np.float32)
    a[0, 0] = OUT
    w = np.full((128, 256), 448.0, np.float32)
    c = host(_d().fp8_gemm_granularity(dev(a, torch.float32), dev(w, torch.float32), g))
    ah, wh = og.dequantised(a, w, g)
    assert np.array_equal(c, (ah @ wh.T).astype(np.float32)), g
    a2 = np.full((3, 128), 448.0, np.float32)
    w2 = np.full((128, 128), 448.0, np.float32)
    w2[0] *= np.float32(2.0 ** 20)
    c2 = host(_d().fp8_gemm_granularity(dev(a2, torch.float32), dev(w2, torch.float32), g))
    ah, wh = og.dequantised(a2, w2, g)
    assert np.array_equal(c2, (ah @ wh.T).astype(np.float32)), g


def test_gemm_granularity_study_on_gpu():
    """The study itself on the GPU's outputs: error of each granularity against
    the float64 product of the unquantised inputs, equal to the oracle's to
    1e-3 relative, and ordered block < channel < tensor."""
    banner("granularity study 256x512x7168")
    a, w = dense_gemm_inputs_host(256, 512, 7168, seed=0)
    exact = a.astype(np.float64) @ w.astype(np.float64).T
    errs = {}
    for g in og.GRANULARITIES:
        c = host(_d().fp8_gemm_granularity(dev(a, torch.bfloat16), dev(w, torch.bfloat16), g))
        got = float(np.linalg.norm(c - exact) / np.linalg.norm(exact))
        want = og.gemm_errors(a, w, g)["rel_frobenius"]
        print(f"[study] {g}: rel_frobenius gpu {got:.5f} oracle {want:.5f}", flush=True)
        assert abs(got - want) <= 1e-3 * want, (g, got, want)
        errs[g] = got
    assert errs["block"] < errs["channel"] < errs["tensor"], errs


@pytest.mark.parametrize("g", og.GRANULARITIES)
def test_gemm_granularity_full_size_sampled_rows(g):
    """The dense workload (M = N = 4096, K = 7168) as bench.py runs it,
    checked on 24 sampled rows (first, last, random)."""
    banner(f"gemm_granularity full size {g}")
    a, w = dense_gemm_inputs_host(4096, 4096, 7168, seed=0)
    rows = np.unique(np.concatenate([[0, 4095], np.random.default_rng(9).choice(4096, 22, replace=False)]))
    _check_gemm(a, w, g, torch.bfloat16, "4096x4096x7168", rows=rows)


def test_gemm_granularity_rejects_bad_arguments():
    d = _d()
    a = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((128, 256), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((4, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty((16,), dtype=torch.uint8, device="cuda")
    with pytest.raises(d.DsmoeError, match="WORKSPACE"):
        d.fp8_gemm_granularity(a, w, "block", c=c, workspace=ws)
    with pytest.raises(d.DsmoeError, match="SHAPE"):
        d.fp8_gemm_granularity(a[:, :200].contiguous(), w[:, :200].contiguous(), "tensor")
