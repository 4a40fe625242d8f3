"""GPU parity of dsmoe_route and dsmoe_update_bias against the oracle.

Both sides receive the same float32 logits, so expert choices, counts,
offsets, perm and inv must match bit for bit; gates are compared with an
absolute tolerance of 1e-6 (the GPU normalises in float32, the oracle in
float64).  The bias update is compared bit for bit.
"""

import numpy as np
import pytest
import torch

from dsmoe_inputs import zipf_logit_offsets
from gpu_util import banner, dev, host
from oracle import bias as ob
from oracle import route as orr

pytestmark = pytest.mark.gpu


def _dsmoe():
    import fp8_block_scaled_dsmoe_amd as d
    return d


def _run_and_compare(z: np.ndarray, b: np.ndarray, G: int, Mg: int, K: int, what: str):
    d = _dsmoe()
    T, E = z.shape
    banner(f"route {what} T={T} E={E} G={G} Mg={Mg} K={K}")
    out = d.route(dev(z), dev(b), G, Mg, K)
    want = orr.route(z, b, G, Mg, K)
    counts, offsets, perm, inv = orr.permute(want["topk_idx"], E)
    got_idx = host(out["topk_idx"])
    bad = np.nonzero(np.any(got_idx != want["topk_idx"], axis=1))[0]
    assert bad.size == 0, f"{what}: {bad.size} tokens differ, first {bad[:5].tolist()}: " \
                          f"{got_idx[bad[:2]].tolist()} vs {want['topk_idx'][bad[:2]].tolist()}"
    assert np.abs(host(out["gates"]) - want["gates"]).max(initial=0) <= 1e-6
    assert np.array_equal(host(out["counts"]), counts)
    assert np.array_equal(host(out["offsets"]), offsets)
    assert np.array_equal(host(out["perm"]), perm)
    assert np.array_equal(host(out["inv"]), inv)
    return out


def _golden_inputs(g):
    E = g["E"]
    z = np.full((len(g["tokens"]), E), g["logits_default"], np.float32)
    for t, tok in enumerate(g["tokens"]):
        for k, v in tok["logits"].items():
            if k == "all":
                z[t, :] = v
            else:
                z[t, int(k)] = v
    b = np.zeros(E, np.float32)
    for k, v in g["bias_nonzero"].items():
        b[int(k)] = v
    return z, b


def test_golden_routing_and_bias(golden):
    d = _dsmoe()
    g = golden("routing_c1.json")
    gb = golden("bias_update.json")
    z, b = _golden_inputs(g)
    out = _run_and_compare(z, b, g["G"], g["Mg"], g["K"], "golden")
    assert host(out["topk_idx"]).tolist() == [t["topk_idx"] for t in g["tokens"]]
    assert host(out["perm"]).tolist() == g["perm"]
    bt = dev(b)
    d.update_bias(bt, out["counts"], T=4, K=2, gamma=gb["gamma"])
    want_b = ob.update_bias(b, np.array(g["counts"], np.int32), 4, 2, gb["gamma"])
    assert np.array_equal(host(bt).view(np.uint32), want_b.view(np.uint32))
    out2 = d.route(dev(z[2:3]), bt, g["G"], g["Mg"], g["K"])
    assert host(out2["topk_idx"])[0].tolist() == gb["rerouted_token2_topk_idx"]


@pytest.mark.parametrize("T,E,G,Mg,K", [
    (1000, 256, 8, 4, 8),     # V3 geometry, ragged T
    (256, 16, 4, 2, 2),       # tiny geometry
    (333, 12, 3, 2, 3),       # E not a power of two
    (100, 64, 1, 1, 6),       # ungrouped
    (70, 1024, 64, 8, 32),    # largest E, G and K the library accepts
    (50, 1, 1, 1, 1),         # one expert
])
def test_random_logits_with_ties(T, E, G, Mg, K):
    r = np.random.default_rng(T + E)
    z = (r.standard_normal((T, E)) * 0.7).astype(np.float32)
    z[:: 3] = np.round(z[:: 3] * 2) / 2            # exact ties in a third of the tokens
    b = r.uniform(-0.01, 0.01, E).astype(np.float32)
    b[:: 5] = 0.0
    _run_and_compare(z, b, G, Mg, K, "random")


def test_v3_skewed_full_size():
    T, E = 32768, 256
    r = np.random.default_rng(7)
    z = (r.standard_normal((T, E)) * 0.5).astype(np.float32)
    z += zipf_logit_offsets(E, 1.1, 0.5)[None, :]
    b = r.uniform(-0.01, 0.01, E).astype(np.float32)
    out = _run_and_compare(z, b, 8, 4, 8, "v3 skew")
    counts = host(out["counts"])
    assert counts.sum() == T * 8
    assert counts.max() <= T


def test_empty_batch():
    d = _dsmoe()
    z = torch.empty((0, 16), dtype=torch.float32, device="cuda")
    out = d.route(z, dev(np.zeros(16, np.float32)), 4, 2, 2)
    assert host(out["counts"]).sum() == 0
    assert host(out["offsets"]).tolist() == [0] * 17


@pytest.mark.parametrize("T,K,E", [(4096, 8, 256), (12, 2, 16), (0, 8, 256), (64, 8, 256)])
def test_bias_update_matches_oracle(T, K, E):
    d = _dsmoe()
    r = np.random.default_rng(T + 1)
    b = r.uniform(-0.01, 0.01, E).astype(np.float32)
    counts = r.multinomial(T * K, np.ones(E) / E).astype(np.int32) if T else np.zeros(E, np.int32)
    if T and (T * K) % E == 0:
        counts[0] = T * K // E                      # exactly the mean load: sign 0
    banner(f"update_bias T={T} K={K} E={E}")
    bt = dev(b)
    d.update_bias(bt, dev(counts), T, K, 0.001)
    want = ob.update_bias(b, counts, T, K, 0.001)
    assert np.array_equal(host(bt).view(np.uint32), want.view(np.uint32))


def test_permute_with_4_byte_aligned_topk_buffer():
    """dsmoe_route requires only 4-byte alignment of its int32 buffers; with a
    topk_idx buffer that is not 16-byte aligned the permutation reads the
    entries one by one.  Same results as the oracle, over several 8192-entry
    slabs and a ragged last one."""
    import ctypes
    d = _dsmoe()
    T, E, G, Mg, K = 2500, 256, 8, 4, 8
    r = np.random.default_rng(23)
    z = (r.standard_normal((T, E)) * 0.7).astype(np.float32)
    b = r.uniform(-0.01, 0.01, E).astype(np.float32)
    want = orr.route(z, b, G, Mg, K)
    counts, offsets, perm, inv = orr.permute(want["topk_idx"], E)
    banner(f"route unaligned topk T={T}")
    zt, bt = dev(z), dev(b)
    topk_buf = torch.zeros((T * K + 4,), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, K), dtype=torch.float32, device="cuda")
    out = {n: torch.empty(s, dtype=torch.int32, device="cuda")
           for n, s in (("counts", (E,)), ("offsets", (E + 1,)), ("perm", (T * K,)), ("inv", (T, K)))}
    topk_ptr = ctypes.c_void_p(topk_buf.data_ptr() + 4)
    st = d.lib.dsmoe_route(ctypes.c_void_p(zt.data_ptr()), ctypes.c_void_p(bt.data_ptr()), T, E, G, Mg, K,
                           topk_ptr, ctypes.c_void_p(gates.data_ptr()),
                           *[ctypes.c_void_p(out[n].data_ptr()) for n in ("counts", "offsets", "perm", "inv")],
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, d.lib.dsmoe_status_str(st)
    torch.cuda.synchronize()
    assert np.array_equal(host(topk_buf)[1:1 + T * K].reshape(T, K), want["topk_idx"])
    assert np.array_equal(host(out["counts"]), counts)
    assert np.array_equal(host(out["offsets"]), offsets)
    assert np.array_equal(host(out["perm"]), perm)
    assert np.array_equal(host(out["inv"]), inv)
