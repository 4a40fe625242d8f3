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


# ---------------------------------------------------------------------------
# Weight gradients, SwiGLU backward, gate and router gradients
# ---------------------------------------------------------------------------

def test_token_tiles_are_activation_tiles_of_the_transpose():
    """1x128 tiles along the rows: for a group of 256 rows the codes and
    scales are those of the 1x128 activation quantiser run on the transposed
    rows; a short last tile behaves as if zero-padded; an outlier moves only
    its own tile's scale (the group's other tiles and other columns keep
    theirs)."""
    v = normal_bf16("tok_v", (556, 256), 1.0, seed=2)
    offsets = [0, 256, 556]                       # 256 rows, then 300 = 128 + 128 + 44
    q, s = ob.quant_tokens_128(v, offsets)
    assert list(ob.chunk_offsets(offsets)) == [0, 2, 5] and s.shape == (5, 256)
    qt, st = oq.quant_act_1x128(np.ascontiguousarray(v[:256].T))     # [256 cols][256 rows]
    assert np.array_equal(q[:256], qt.T)
    assert np.array_equal(s[:2].view(np.uint32), st.T.view(np.uint32))
    tail = np.zeros((128, 256), np.float32)
    tail[:44] = v[512:556]
    qz, sz = oq.quant_act_1x128(np.ascontiguousarray(tail.T))
    assert np.array_equal(q[512:556], qz.T[:44]) and np.array_equal(s[4], sz[:, 0])
    w = v.copy()
    w[256 + 130, 7] = np.float32(80.0)            # group 1, tile 1, column 7
    q2, s2 = ob.quant_tokens_128(w, offsets)
    changed = np.argwhere(s2 != s)
    assert changed.tolist() == [[3, 7]]
    assert np.array_equal(q2[:256 + 128], q[:256 + 128]) and np.array_equal(q2[256 + 256:], q[256 + 256:])


def test_wgrad_is_the_adjoint_of_the_forward():
    """<dW_g, V> = <dC_hat, A_hat V^T> over each group's rows for any V: the
    weight gradient contracts the rows and has the weight's [N][K] shape.  A
    square case where dW^T would fit the shapes gives another value."""
    r = np.random.default_rng(8)
    for n, k in [(256, 384), (128, 128)]:
        offsets = [0, 70, 70, 333]                # a ragged group, an empty one, three tiles
        rows = offsets[-1]
        dc = normal_bf16("wg_dc", (rows, n), 1.0, seed=n)
        a = normal_bf16("wg_a", (rows, k), 1.0, seed=k + 1)
        qg, sg = ob.quant_tokens_128(dc, offsets)
        qa, sa = ob.quant_tokens_128(a, offsets)
        dw, dn = ob.wgrad_grouped(qg, sg, qa, sa, offsets)
        assert dw.shape == (3, n, k) and np.all(dw[1] == 0) and np.all(dn >= np.abs(dw))
        dc_hat = ob.dequant_tokens_128(qg, sg, offsets)
        a_hat = ob.dequant_tokens_128(qa, sa, offsets)
        for g in (0, 2):
            r0, r1 = offsets[g], offsets[g + 1]
            v = r.standard_normal((n, k))
            lhs = float(np.sum(dw[g] * v))
            rhs = float(np.sum(dc_hat[r0:r1] * (a_hat[r0:r1] @ v.T)))
            assert abs(lhs - rhs) <= 1e-11 * float(np.sum(dn[g] * np.abs(v)))
            if n == k:
                assert abs(float(np.sum(dw[g].T * v)) - lhs) > 1e-6 * abs(lhs)


def test_wgrad_integer_matmul():
    """Codes that are small integers with a +-448 in every tile column (so
    every scale is 1 and every code its own value): the weight gradient is the
    exact integer product of the operands, group by group."""
    r = np.random.default_rng(4)
    offsets = [0, 128, 200]
    rows, n, k = 200, 128, 256
    dc = r.integers(-15, 16, size=(rows, n)).astype(np.float32)
    a = r.integers(-15, 16, size=(rows, k)).astype(np.float32)
    for m in (dc, a):
        m[0] = 448.0
        m[128] = -448.0
    qg, sg = ob.quant_tokens_128(dc, offsets)
    qa, sa = ob.quant_tokens_128(a, offsets)
    assert np.all(sg == 1.0) and np.all(sa == 1.0)
    dw, _ = ob.wgrad_grouped(qg, sg, qa, sa, offsets)
    for g in range(2):
        r0, r1 = offsets[g], offsets[g + 1]
        want = dc[r0:r1].astype(np.int64).T @ a[r0:r1].astype(np.int64)
        assert np.array_equal(dw[g], want.astype(np.float64))


def test_swiglu_backward_finite_differences():
    """Each a_j depends on its own gate and up value only, so central
    differences per element pin both halves; at g = 0, silu' = 1/2 and
    silu = 0."""
    r = np.random.default_rng(5)
    n, inter = 6, 256
    h = r.standard_normal((n, 2 * inter)) * 3.0
    h[0, :inter] = 0.0
    da = r.standard_normal((n, inter))
    dh = ob.swiglu_backward(h, da)

    def act(g, u):
        return g / (1.0 + np.exp(-g)) * u

    g, u = h[:, :inter], h[:, inter:]
    eps = 1e-6
    fd_g = (act(g + eps, u) - act(g - eps, u)) / (2 * eps) * da
    fd_u = (act(g, u + eps) - act(g, u - eps)) / (2 * eps) * da
    assert np.allclose(dh[:, :inter], fd_g, rtol=1e-6, atol=1e-8)
    assert np.allclose(dh[:, inter:], fd_u, rtol=1e-6, atol=1e-8)
    assert np.array_equal(dh[0, :inter], 0.5 * da[0] * u[0]) and np.all(dh[0, inter:] == 0)


def test_gate_backward_finite_differences():
    """Routing held fixed: dlogits is the derivative of
    L(z) = sum_t sum_k gate_k(z) <dy_t, o_tk> with gate_k = s_k / sum s and
    s = sigmoid(z) (central differences in float64); unchosen experts get 0;
    an upstream gradient equal for all chosen experts gives no logit gradient
    (the gates sum to 1)."""
    from oracle import route as orr
    r = np.random.default_rng(6)
    T, E, H, K = 5, 16, 32, 4
    z = (r.standard_normal((T, E)) * 2.0).astype(np.float32)
    idx = orr.route(z, np.zeros(E, np.float32), 4, 2, K)["topk_idx"]
    dy = r.standard_normal((T, H))
    o = r.standard_normal((T, K, H))
    dgate, dz = ob.gate_backward(dy, o, idx, z, E)
    assert np.allclose(dgate, np.einsum("th,tkh->tk", dy, o), rtol=1e-14)

    def loss(zz):
        s = 1.0 / (1.0 + np.exp(-zz))
        s_sel = np.take_along_axis(s, idx.astype(np.int64), axis=1)
        return float(np.sum(s_sel / s_sel.sum(axis=1, keepdims=True) * dgate))

    z64 = z.astype(np.float64)
    eps = 1e-6
    for t in range(T):
        for e in range(E):
            zp, zm = z64.copy(), z64.copy()
            zp[t, e] += eps
            zm[t, e] -= eps
            fd = (loss(zp) - loss(zm)) / (2 * eps)
            assert abs(fd - dz[t, e]) <= 1e-5 * (1 + abs(fd)), (t, e, fd, dz[t, e])
        assert np.count_nonzero(dz[t]) <= K
    same = np.repeat(dgate[:, :1], K, axis=1)[:, :, None] * np.ones((1, 1, H)) / H
    _, dz0 = ob.gate_backward(np.ones((T, H)), same, idx, z, E)
    assert np.allclose(dz0, 0.0, atol=1e-15)
