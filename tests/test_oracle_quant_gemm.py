"""Pins of the oracle's quantisers and block-scaled GEMM.

* hand-worked tiles and the two-chunk GEMM (tests/golden);
* quantisation error bounds that follow from the E4M3 format alone;
* weight blocking is transpose-invariant and scales land on the right block;
* with power-of-two scales the block-scaled GEMM is an integer matmul, checked
  exactly with int64 arithmetic (catches a dropped chunk scale, a swapped
  block index or a transposed operand).
"""

import numpy as np
import pytest

from oracle import e4m3, gemm, quant
from dsmoe_inputs import dense_gemm_inputs_host, normal_bf16


def test_golden_activation_tiles(golden):
    g = golden("quant_tiles.json")
    row = np.zeros((1, 256), np.float32)
    for k, v in g["tile0_nonzero"].items():
        row[0, int(k)] = float(v)
    for k, v in g["tile1_nonzero"].items():
        row[0, 128 + int(k)] = float(v)
    q, s = quant.quant_act_1x128(row)
    assert s.dtype == np.float32
    assert list(s[0]) == g["expected_scales"]
    want = np.zeros(256, np.uint8)
    for k, v in g["expected_codes_tile0_nonzero"].items():
        want[int(k)] = int(v, 16)
    for k, v in g["expected_codes_tile1_nonzero"].items():
        want[128 + int(k)] = int(v, 16)
    assert np.array_equal(q[0], want)
    assert gemm.dequant_act(q, s)[0, 2] == 0.1015625


def test_zero_tile_scale_one_and_signed_zero():
    x = np.zeros((2, 128), np.float32)
    x[1, 5] = -0.0
    q, s = quant.quant_act_1x128(x)
    assert np.all(s == 1.0)
    assert q[1, 5] == 0x80 and q[0, 5] == 0x00


def _check_act_quant_bounds(x, q, s):
    rows, cols = x.shape
    xt = x.reshape(rows, cols // 128, 128).astype(np.float64)
    deq = gemm.dequant_act(q, s).reshape(rows, cols // 128, 128)
    s64 = s.astype(np.float64)[:, :, None]
    # half a quantisation step: 2^-4 relative for normals, 2^-10 * s absolute
    # for the subnormal range; plus the float32 rounding of x / s (2^-24 rel)
    bound = np.abs(xt) * (2.0 ** -4 + 2.0 ** -23) + (2.0 ** -10) * s64
    assert np.all(np.abs(deq - xt) <= bound)
    # the largest element of every non-zero tile maps to +-448
    amax = np.max(np.abs(xt), axis=2)
    codes = q.reshape(rows, cols // 128, 128)
    am_pos = np.argmax(np.abs(xt), axis=2)
    top = np.take_along_axis(codes, am_pos[:, :, None], axis=2)[:, :, 0] & 0x7F
    assert np.all(top[amax > 0] == 0x7E)
    assert np.max(codes & 0x7F) <= 0x7E


def test_activation_quant_bounds_with_outliers():
    a, _ = dense_gemm_inputs_host(64, 128, 1024, seed=3)
    q, s = quant.quant_act_1x128(a)
    _check_act_quant_bounds(a, q, s)
    # scale is amax / 448 rounded once to float32
    amax = np.max(np.abs(a.reshape(64, 8, 128)), axis=2)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))


def test_weight_blocking_transpose_invariant():
    w = normal_bf16("wt", (384, 256), 0.02, seed=1)
    q1, s1 = quant.quant_w_128x128(w)
    q2, s2 = quant.quant_w_128x128(np.ascontiguousarray(w.T))
    assert np.array_equal(q1.T, q2)
    assert np.array_equal(s1.T, s2)


def test_weight_scales_land_on_their_block():
    # block (i, j) holds one element of magnitude 448 * 2^(i - 2j); scale is 2^(i-2j)
    n_b, k_b = 3, 4
    w = np.full((n_b * 128, k_b * 128), 2.0 ** -20, np.float32)
    r = np.random.default_rng(0)
    for i in range(n_b):
        for j in range(k_b):
            w[i * 128 + r.integers(128), j * 128 + r.integers(128)] = -448.0 * 2.0 ** (i - 2 * j)
    q, s = quant.quant_w_128x128(w[None])
    want = np.array([[2.0 ** (i - 2 * j) for j in range(k_b)] for i in range(n_b)], np.float32)
    assert np.array_equal(s[0], want)
    assert np.sum(q[0] == 0xFE) == n_b * k_b


def test_golden_two_chunk_gemm(golden):
    g = golden("gemm_two_chunk.json")
    a = np.zeros((1, 256), np.float32)
    a[0, :128] = g["a_row"]["cols_0_127"]
    a[0, 128:] = g["a_row"]["cols_128_255"]
    w = np.zeros((128, 256), np.float32)
    w[0, :128] = g["w_row0"]["cols_0_127"]
    w[0, 128:] = g["w_row0"]["cols_128_255"]
    qa, sa = quant.quant_act_1x128(a)
    qw, sw = quant.quant_w_128x128(w)
    assert list(sa[0]) == g["expected_scales_a"]
    assert list(sw[0]) == g["expected_scales_w"]
    c = gemm.block_scaled_gemm(qa, sa, qw, sw)
    assert c[0, 0] == g["expected_c00"]
    assert np.all(c[0, 1:] == 0)
    sa_bug = np.repeat(sa[:, :1], 2, axis=1)
    sw_bug = np.repeat(sw[:, :1], 2, axis=1)
    assert gemm.block_scaled_gemm(qa, sa_bug, qw, sw_bug)[0, 0] == g["single_scale_bug_c00"]


def _random_codes(r, shape):
    c = r.integers(0, 256, size=shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c & 0xF0, c).astype(np.uint8)   # no NaN codes


def _int_gemm(qa, ea, qw, ew):
    """Exact C with integer arithmetic: every finite E4M3 value is an integer
    multiple of 2^-9, scales are 2^ea / 2^ew."""
    na = np.rint(e4m3.decode(qa) * 512).astype(np.int64)
    nw = np.rint(e4m3.decode(qw) * 512).astype(np.int64)
    m, k = qa.shape
    c = np.zeros((m, qw.shape[0]), np.float64)
    for ch in range(k // 128):
        p = na[:, ch * 128:(ch + 1) * 128] @ nw[:, ch * 128:(ch + 1) * 128].T   # exact int64
        e = ea[:, ch][:, None] + np.repeat(ew[:, ch], 128)[None, :] - 18
        c += np.ldexp(p.astype(np.float64), e)
    return c


@pytest.mark.parametrize("m,n,k", [(5, 256, 384), (17, 384, 128), (1, 128, 1024)])
def test_gemm_is_integer_matmul_with_power_of_two_scales(m, n, k):
    r = np.random.default_rng(m * 1000 + n + k)
    qa = _random_codes(r, (m, k))
    qw = _random_codes(r, (n, k))
    # exponent spread <= 4 keeps every float64 sum below exact (< 2^53 units)
    ea = r.integers(-1, 2, size=(m, k // 128))
    ew = r.integers(-1, 2, size=(n // 128, k // 128))
    sa = np.ldexp(1.0, ea).astype(np.float32)
    sw = np.ldexp(1.0, ew).astype(np.float32)
    c = gemm.block_scaled_gemm(qa, sa, qw, sw)
    assert np.array_equal(c, _int_gemm(qa, ea, qw, ew))
    d = gemm.gemm_normaliser(qa, sa, qw, sw)
    assert np.all(np.abs(c) <= d * (1 + 1e-12))


def test_grouped_gemm_gathers_rows_and_picks_group_weights():
    r = np.random.default_rng(7)
    groups, n, k, rows_a = 3, 128, 256, 10
    qa = _random_codes(r, (rows_a, k))
    ea = r.integers(-2, 3, size=(rows_a, k // 128))
    qw = _random_codes(r, (groups, n, k))
    ew = r.integers(-2, 3, size=(groups, n // 128, k // 128))
    offsets = np.array([0, 4, 4, 9])
    a_rows = np.array([3, 3, 0, 9, 1, 2, 5, 7, 8])
    c, _ = gemm.grouped_gemm(qa, np.ldexp(1.0, ea).astype(np.float32), a_rows, offsets,
                             qw, np.ldexp(1.0, ew).astype(np.float32))
    for g in range(groups):
        for rr in range(offsets[g], offsets[g + 1]):
            src = a_rows[rr]
            want = _int_gemm(qa[src:src + 1], ea[src:src + 1], qw[g], ew[g])
            assert np.array_equal(c[rr:rr + 1], want)
