"""Pins of oracle.backward (V3 notes §6: the data-gradient GEMMs in FP8 on the
forward's 128x128 weight blocks, transposed)."""

import numpy as np

from dsmoe_inputs import normal_bf16
from oracle import backward as ob
from oracle import gemm as og
from oracle import quant as oq


def test_block_quantisation_commutes_with_transposition():
    """quant(W^T) == transpose(quant(W)): a block's amax, hence its scale and
    every code, is the same read row- or column-wise."""
    w = normal_bf16("bwd_w", (2, 256, 384), 0.02, seed=1)
    w[1, 130, 7] = np.float32(3.0)           # an outlier in one block
    q, s = oq.quant_w_128x128(w)
    qt, st = oq.quant_w_128x128(np.ascontiguousarray(np.swapaxes(w, 1, 2)))
    qb, sb = ob.transpose_blocks(q, s)
    assert np.array_equal(qt, qb)
    assert np.array_equal(st.view(np.uint32), sb.view(np.uint32))
    assert qb.shape == (2, 384, 256) and sb.shape == (2, 3, 2)


def test_adjoint_identity_fixes_the_orientation():
    """<dC, A_hat W_hat^T> = <dC_hat W_hat, A_hat> with dC_hat the 1x128
    codes of dC along N: the dgrad contracts the weight over its output axis.
    N != K, and a square case where W and W^T would both fit the shapes."""
    r = np.random.default_rng(3)
    for (m, n, k) in [(40, 256, 384), (33, 256, 256)]:
        a = normal_bf16("bwd_a", (m, k), 1.0, seed=m)
        w = normal_bf16("bwd_w2", (1, n, k), 0.02, seed=n + k)
        w[0] += np.float32(0.01) * r.standard_normal((n, k)).astype(np.float32)   # not symmetric
        dc = normal_bf16("bwd_dc", (m, n), 1.0, seed=k)
        qa, sa = oq.quant_act_1x128(a)
        qw, sw = oq.quant_w_128x128(w)
        qg, sg = oq.quant_act_1x128(dc)
        a_hat = og.dequant_act(qa, sa)
        dc_hat = og.dequant_act(qg, sg)
        w_hat = og.dequant_w(qw[0], sw[0])
        lhs = float(np.sum(dc_hat * (a_hat @ w_hat.T)))
        da, dnorm = ob.dgrad_grouped(qg, sg, None, [0, m], qw, sw)
        rhs = float(np.sum(da * a_hat))
        assert abs(lhs - rhs) <= 1e-12 * float(np.sum(np.abs(dc_hat) @ np.abs(w_hat) * np.abs(a_hat)))
        assert da.shape == (m, k) and np.all(dnorm >= np.abs(da))
        if n == k:   # using W instead of W^T gives another value
            wrong = float(np.sum((dc_hat @ w_hat.T) * a_hat))
            assert abs(wrong - lhs) > 1e-6 * abs(lhs)


def test_grouped_gather_matches_rows_one_by_one():
    """Rows gathered through g_rows into ragged groups: each output row is the
    gathered gradient row times its group's weight."""
    G, n, k = 3, 128, 256
    w = normal_bf16("bwd_wg", (G, n, k), 0.02, seed=4)
    dc = normal_bf16("bwd_dcg", (10, n), 1.0, seed=5)
    qw, sw = oq.quant_w_128x128(w)
    qg, sg = oq.quant_act_1x128(dc)
    rows = np.array([3, 0, 7, 7, 1, 9, 2], np.int64)
    offsets = [0, 2, 2, 7]
    da, _ = ob.dgrad_grouped(qg, sg, rows, offsets, qw, sw)
    dc_hat = og.dequant_act(qg, sg)
    for r, src in enumerate(rows):
        g = 0 if r < 2 else 2
        want = dc_hat[src] @ og.dequant_w(qw[g], sw[g])
        assert np.allclose(da[r], want, rtol=1e-12, atol=0)
