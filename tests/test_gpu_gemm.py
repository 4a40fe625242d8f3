"""GPU parity of dsmoe_fp8_grouped_gemm against the oracle's block-scaled
GEMM.  Bar: max |gpu - oracle| / D <= 2e-3 for float32 output and 1e-2 for
bf16 output, D = |a_hat| . |w_hat|^T element-wise (the oracle's normaliser).
Quantised operands come from the oracle's own quantisers (the GPU quantisers
are checked bit-exact against them separately)."""

import numpy as np
import pytest
import torch

from dsmoe_inputs import dense_gemm_inputs_host, normal_bf16
from gpu_util import assert_normalised_close, banner, dev, host
from oracle import gemm as og
from oracle import quant as oq

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 2e-3, torch.bfloat16: 1e-2}


def _dsmoe():
    import fp8_block_scaled_dsmoe_amd as d
    return d


def _codes(r, shape):
    c = r.integers(0, 256, size=shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c & 0xF0, c).astype(np.uint8)


def test_golden_two_chunk(golden):
    d = _dsmoe()
    g = golden("gemm_two_chunk.json")
    a = np.zeros((1, 256), np.float32)
    a[0, :128] = g["a_row"]["cols_0_127"]
    a[0, 128:] = g["a_row"]["cols_128_255"]
    w = np.zeros((128, 256), np.float32)
    w[0, :128] = g["w_row0"]["cols_0_127"]
    w[0, 128:] = g["w_row0"]["cols_128_255"]
    qa, sa = oq.quant_act_1x128(a)
    qw, sw = oq.quant_w_128x128(w)
    banner("gemm golden two-chunk")
    for dt in (torch.float32, torch.bfloat16):
        c = d.fp8_grouped_gemm(dev(qa), dev(sa), dev(np.array([0, 1], np.int32)), dev(qw[None]),
                               dev(sw[None]), out_dtype=dt)
        ch = host(c)
        assert ch[0, 0] == g["expected_c00"]
        assert np.all(ch[0, 1:] == 0)


# float32 bit patterns (positive) whose bf16 rounding is a corner case:
# ties to even either way, one ulp off a tie, subnormals (ties, the smallest,
# the largest, rounding up to the smallest normal), and the top of the range
# (a tie that rounds to infinity, values just below and above it)
_BF16_CORNERS = [0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001, 0x3F800000, 0x3FFFFFFF,
                 0x00008000, 0x00018000, 0x00000001, 0x0000C000, 0x007FFFFF, 0x00808000,
                 0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0x7F7E8000, 0x0B7F8000, 0x34818000]


# (M, N): the weight-streaming kernel, the 128-column LDS kernel, the 256 x 256 kernel
@pytest.mark.parametrize("M,N", [(40, 256), (300, 128), (600, 256)])
def test_bf16_output_rounding(M, N):
    """bf16 outputs are the float32 results rounded to nearest, ties to even,
    subnormals kept.  Every output is exact in float32: row r holds one
    non-zero product, (+-1) x 1 at column 0, so c[r][n] = +-sa[r][0]; the row
    scales are the corner patterns above and random positive floats.  The
    float32 output must equal +-sa exactly and the bf16 output torch's CPU
    rounding of it, bit for bit."""
    d = _dsmoe()
    r = np.random.default_rng(M + N)
    K = 256
    bits = r.integers(0x00000001, 0x7F800000, size=M, dtype=np.int64).astype(np.uint32)
    bits[:len(_BF16_CORNERS)] = _BF16_CORNERS
    vals = bits.view(np.float32)
    neg = r.random(M) < 0.5
    qa = np.zeros((M, K), np.uint8)
    qa[:, 0] = np.where(neg, 0xB8, 0x38)            # -1.0 / +1.0
    sa = np.ones((M, K // 128), np.float32)
    sa[:, 0] = vals
    qw = np.zeros((N, K), np.uint8)
    qw[:, 0] = 0x38
    sw = np.ones((N // 128, K // 128), np.float32)
    want32 = np.where(neg, -vals, vals).astype(np.float32)
    want16 = torch.from_numpy(want32).to(torch.bfloat16).view(torch.int16).numpy()
    offs = dev(np.array([0, M], np.int32))
    banner(f"gemm bf16 output rounding M={M} N={N}")
    c32 = d.fp8_grouped_gemm(dev(qa), dev(sa), offs, dev(qw[None]), dev(sw[None]), out_dtype=torch.float32)
    c16 = d.fp8_grouped_gemm(dev(qa), dev(sa), offs, dev(qw[None]), dev(sw[None]), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    g32 = c32.cpu().numpy()
    g16 = c16.view(torch.int16).cpu().numpy()
    assert np.array_equal(g32.view(np.uint32), np.repeat(want32.view(np.uint32)[:, None], N, axis=1)), \
        "float32 output differs from the exact value"
    bad = g16 != want16[:, None]
    assert not bad.any(), f"{int(bad.sum())} bf16 outputs differ from round-to-nearest-even, e.g. " + \
        ", ".join(f"{int(want32.view(np.uint32)[i]):#010x} -> {int(g16[i, j]) & 0xFFFF:#06x} "
                  f"(want {int(want16[i]) & 0xFFFF:#06x})" for i, j in zip(*np.nonzero(bad)) if True)[:400]


# (700, 256, 128) and (513, 768, 384): the 256 x 256 kernel with one and
# three K chunks (its stage ring and cross-chunk pipeline at their shortest)
@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (300, 384, 640), (129, 256, 1024), (1000, 512, 256),
                                   (700, 256, 128), (513, 768, 384)])
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_dense_random_codes(M, N, K, dt):
    d = _dsmoe()
    r = np.random.default_rng(M * 7 + N + K)
    qa, qw = _codes(r, (M, K)), _codes(r, (N, K))
    sa = np.ldexp(1.0, r.integers(-8, -2, size=(M, K // 128))).astype(np.float32)
    sw = np.ldexp(1.0, r.integers(-12, -6, size=(N // 128, K // 128))).astype(np.float32)
    sa *= r.uniform(1, 2, size=sa.shape).astype(np.float32)     # non-power-of-two scales too
    banner(f"gemm dense codes M={M} N={N} K={K} {dt}")
    c = d.fp8_grouped_gemm(dev(qa), dev(sa), dev(np.array([0, M], np.int32)), dev(qw[None]),
                           dev(sw[None]), out_dtype=dt)
    want = og.block_scaled_gemm(qa, sa, qw, sw)
    dn = og.gemm_normaliser(qa, sa, qw, sw)
    assert_normalised_close(host(c), want, dn, TOL[dt], f"dense {M}x{N}x{K} {dt}")


# Long contractions: 65 chunks (the weight-streaming kernel's row scales are
# then loaded per chunk instead of staged once per tile) and the 256-chunk
# maximum, on the weight-streaming kernel (few rows) and the 256 x 256 kernel.
@pytest.mark.parametrize("M,N,K", [(40, 256, 8320), (600, 512, 8320), (40, 256, 32768), (300, 256, 32768)])
def test_dense_long_k(M, N, K):
    d = _dsmoe()
    r = np.random.default_rng(M + N + K)
    qa, qw = _codes(r, (M, K)), _codes(r, (N, K))
    sa = (np.ldexp(1.0, r.integers(-8, -2, size=(M, K // 128))) *
          r.uniform(1, 2, size=(M, K // 128))).astype(np.float32)
    sw = np.ldexp(1.0, r.integers(-12, -6, size=(N // 128, K // 128))).astype(np.float32)
    banner(f"gemm dense long K M={M} N={N} K={K}")
    c = d.fp8_grouped_gemm(dev(qa), dev(sa), dev(np.array([0, M], np.int32)), dev(qw[None]),
                           dev(sw[None]), out_dtype=torch.float32)
    want = og.block_scaled_gemm(qa, sa, qw, sw)
    dn = og.gemm_normaliser(qa, sa, qw, sw)
    assert_normalised_close(host(c), want, dn, TOL[torch.float32], f"dense {M}x{N}x{K}")


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_dense_outlier_inputs(dt):
    d = _dsmoe()
    a, w = dense_gemm_inputs_host(512, 384, 1024, seed=5)
    qa, sa = oq.quant_act_1x128(a)
    qw, sw = oq.quant_w_128x128(w)
    banner(f"gemm dense outliers {dt}")
    c = d.fp8_grouped_gemm(dev(qa), dev(sa), dev(np.array([0, 512], np.int32)), dev(qw[None]),
                           dev(sw[None]), out_dtype=dt)
    want = og.block_scaled_gemm(qa, sa, qw, sw)
    dn = og.gemm_normaliser(qa, sa, qw, sw)
    assert_normalised_close(host(c), want, dn, TOL[dt], f"dense outliers {dt}")


def test_grouped_with_gather_and_ragged_groups():
    d = _dsmoe()
    r = np.random.default_rng(11)
    sizes = [0, 1, 127, 128, 129, 300, 0, 5]
    G, N, K, rows_a = len(sizes), 256, 384, 200
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    m_total = int(offsets[-1])
    qa = _codes(r, (rows_a, K))
    sa = (np.ldexp(1.0, r.integers(-8, -2, size=(rows_a, K // 128))) *
          r.uniform(1, 2, size=(rows_a, K // 128))).astype(np.float32)
    qw = _codes(r, (G, N, K))
    sw = np.ldexp(1.0, r.integers(-12, -6, size=(G, N // 128, K // 128))).astype(np.float32)
    a_rows = r.integers(0, rows_a, size=m_total).astype(np.int32)
    banner("gemm grouped gather ragged")
    # sentinel rows past offsets[G] stay untouched
    c = torch.full((m_total + 3, N), -7.0, dtype=torch.float32, device="cuda")
    d.fp8_grouped_gemm(dev(qa), dev(sa), dev(offsets), dev(qw), dev(sw), a_rows=dev(a_rows),
                       m_total=m_total + 3, c=c)
    want, dn = og.grouped_gemm(qa, sa, a_rows, offsets, qw, sw)
    ch = host(c)
    assert np.all(ch[m_total:] == -7.0)
    assert_normalised_close(ch[:m_total], want, dn, TOL[torch.float32], "grouped gather")


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_dense_full_size_sampled_rows(dt):
    """M=N=4096, K=7168 with 1% x50 outliers, the launch the benchmark times;
    checked on 48 sampled rows (every column) against the oracle."""
    d = _dsmoe()
    M, N, K = 4096, 4096, 7168
    a, w = dense_gemm_inputs_host(M, N, K, seed=0)
    banner(f"gemm dense full size {dt}")
    qa_t, sa_t = d.quant_act_1x128(dev(a, torch.bfloat16))
    qw_t, sw_t = d.quant_w_128x128(dev(w, torch.bfloat16))
    c = d.fp8_grouped_gemm(qa_t, sa_t, dev(np.array([0, M], np.int32)), qw_t.unsqueeze(0),
                           sw_t.unsqueeze(0), out_dtype=dt)
    rows = np.random.default_rng(1).choice(M, size=48, replace=False)
    rows[:2] = [0, M - 1]
    qa, sa = oq.quant_act_1x128(a[rows])
    qw, sw = oq.quant_w_128x128(w)
    assert np.array_equal(host(qa_t)[rows], qa)
    assert np.array_equal(host(qw_t), qw)
    want = og.block_scaled_gemm(qa, sa, qw, sw)
    dn = og.gemm_normaliser(qa, sa, qw, sw)
    assert_normalised_close(host(c)[rows], want, dn, TOL[dt], f"dense full size {dt}")


@pytest.mark.parametrize("mean_rows", [3, 12, 20, 42, 62, 82, 105, 114, 400])
def test_grouped_tile_shapes(mean_rows):
    """Group sizes around each row-tile height the library picks (weight
    streaming with 16/32/64/96/128/160/176/192-row tiles, and the 256-row LDS
    kernel), including empty groups and groups longer than one tile."""
    d = _dsmoe()
    r = np.random.default_rng(mean_rows)
    G, N, K = 7, 512, 384
    sizes = r.poisson(mean_rows, size=G)
    sizes[1] = 0
    sizes[3] = 3 * mean_rows + 17
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    m_total = int(offsets[-1])
    rows_a = max(m_total, 1)
    qa = _codes(r, (rows_a, K))
    sa = (np.ldexp(1.0, r.integers(-8, -2, size=(rows_a, K // 128))) *
          r.uniform(1, 2, size=(rows_a, K // 128))).astype(np.float32)
    qw = _codes(r, (G, N, K))
    sw = np.ldexp(1.0, r.integers(-12, -6, size=(G, N // 128, K // 128))).astype(np.float32)
    a_rows = r.permutation(rows_a)[:m_total].astype(np.int32)
    banner(f"gemm grouped tile shapes mean_rows={mean_rows} sizes={sizes.tolist()}")
    for dt in (torch.float32, torch.bfloat16):
        c = d.fp8_grouped_gemm(dev(qa), dev(sa), dev(offsets), dev(qw), dev(sw), a_rows=dev(a_rows),
                               out_dtype=dt)
        want, dn = og.grouped_gemm(qa, sa, a_rows, offsets, qw, sw)
        assert_normalised_close(host(c), want, dn, TOL[dt], f"grouped mean {mean_rows} {dt}")


@pytest.mark.parametrize("K", [640, 2048])
def test_grouped_blocks_run_several_tiles(K):
    """More tiles than blocks that fit on the GPU at once, so the launch runs
    in several rounds of blocks.  K = 640 gives 5 chunks, which does not
    divide the register ring; groups of ~100 rows, some empty, some longer
    than one tile; gathered A rows."""
    d = _dsmoe()
    r = np.random.default_rng(K)
    G, N = 72, 2048
    sizes = r.poisson(100, size=G)
    sizes[::9] = 0
    sizes[5] = 400
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    m_total = int(offsets[-1])
    rows_a = m_total + 7
    qa = _codes(r, (rows_a, K))
    sa = (np.ldexp(1.0, r.integers(-8, -2, size=(rows_a, K // 128))) *
          r.uniform(1, 2, size=(rows_a, K // 128))).astype(np.float32)
    qw = _codes(r, (G, N, K))
    sw = np.ldexp(1.0, r.integers(-12, -6, size=(G, N // 128, K // 128))).astype(np.float32)
    a_rows = r.permutation(rows_a)[:m_total].astype(np.int32)
    banner(f"gemm grouped several tiles per block G={G} N={N} K={K} rows={m_total}")
    want, dn = og.grouped_gemm(qa, sa, a_rows, offsets, qw, sw)
    for dt in (torch.float32, torch.bfloat16):
        c = d.fp8_grouped_gemm(dev(qa), dev(sa), dev(offsets), dev(qw), dev(sw), a_rows=dev(a_rows),
                               out_dtype=dt)
        assert_normalised_close(host(c), want, dn, TOL[dt], f"grouped several tiles K={K} {dt}")


@pytest.mark.parametrize("G,mean_rows", [(1100, 3), (600, 260)])
def test_grouped_many_groups(G, mean_rows):
    """More groups than a block has threads, so the tile decoder's scan over
    the group table takes several passes: 1100 groups of a few rows
    (weight-streaming tiles) and 600 groups of ~260 rows (256 x 256 tiles),
    with empty groups among them."""
    d = _dsmoe()
    r = np.random.default_rng(G)
    N, K = 256, 256
    sizes = r.poisson(mean_rows, size=G)
    sizes[r.choice(G, size=G // 10, replace=False)] = 0
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    m_total = int(offsets[-1])
    qa = _codes(r, (m_total, K))
    sa = (np.ldexp(1.0, r.integers(-8, -2, size=(m_total, K // 128))) *
          r.uniform(1, 2, size=(m_total, K // 128))).astype(np.float32)
    qw = _codes(r, (G, N, K))
    sw = np.ldexp(1.0, r.integers(-12, -6, size=(G, N // 128, K // 128))).astype(np.float32)
    a_rows = np.arange(m_total, dtype=np.int32)
    banner(f"gemm many groups G={G} rows={m_total}")
    c = d.fp8_grouped_gemm(dev(qa), dev(sa), dev(offsets), dev(qw), dev(sw), out_dtype=torch.float32)
    want, dn = og.grouped_gemm(qa, sa, a_rows, offsets, qw, sw)
    assert_normalised_close(host(c), want, dn, TOL[torch.float32], f"grouped G={G}")
