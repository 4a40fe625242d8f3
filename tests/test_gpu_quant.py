"""GPU parity of dsmoe_quant_act_1x128 / dsmoe_quant_w_128x128 against the
oracle: FP8 codes and scales must match bit for bit."""

import numpy as np
import pytest
import torch

from dsmoe_inputs import bf16_round, dense_gemm_inputs_host, normal_bf16
from gpu_util import banner, dev, host
from oracle import quant as oq

pytestmark = pytest.mark.gpu


def _dsmoe():
    import fp8_block_scaled_dsmoe_amd as d
    return d


def _check_act(x32: np.ndarray, as_bf16: bool, what: str):
    d = _dsmoe()
    banner(f"quant_act {what} shape={x32.shape} bf16={as_bf16}")
    xt = dev(x32, torch.bfloat16 if as_bf16 else torch.float32)
    q, s = d.quant_act_1x128(xt)
    qo, so = oq.quant_act_1x128(x32)
    qg, sg = host(q), host(s)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32)), f"{what}: scales differ"
    bad = np.argwhere(qg != qo)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first {bad[:5].tolist()}"


def test_golden_tiles(golden):
    g = golden("quant_tiles.json")
    row = np.zeros((1, 256), np.float32)
    for k, v in g["tile0_nonzero"].items():
        row[0, int(k)] = float(v)
    for k, v in g["tile1_nonzero"].items():
        row[0, 128 + int(k)] = float(v)
    _check_act(row, True, "golden bf16")
    _check_act(row, False, "golden f32")


@pytest.mark.parametrize("rows,cols", [(1, 128), (300, 1024), (4096, 7168)])
def test_act_bf16_with_outliers(rows, cols):
    a, _ = dense_gemm_inputs_host(rows, 128, cols, seed=rows)
    _check_act(a, True, f"outliers {rows}x{cols}")


def test_act_f32_encoder_sweep():
    # tiles whose first element is 448 have scale exactly 1, so every other
    # element is encoded as given: sweep sign, every exponent that reaches the
    # E4M3 range (including float32 subnormals), every top-7 mantissa pattern,
    # and low bits at / just around the rounding midpoints
    r = np.random.default_rng(0)
    exps = np.arange(0, 136, dtype=np.uint32)            # biased float32 exponents 0..135 (< 512)
    mant_hi = np.arange(128, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = (exps[:, None, None] << 23) | mant_hi[None, :, None] | lows[None, None, :]
    bits = bits.reshape(-1)
    bits = np.concatenate([bits, bits | 0x80000000,
                           r.integers(0, 0x43E00000, size=200000, dtype=np.uint32)])
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448.0)]
    per = 127
    n_tiles = -(-vals.size // per)
    pad = np.zeros(n_tiles * per, np.float32)
    pad[:vals.size] = vals
    tiles = np.concatenate([np.full((n_tiles, 1), 448.0, np.float32), pad.reshape(n_tiles, per)], axis=1)
    cols = 1024
    n_rows = -(-tiles.size // cols)
    flat = np.zeros(n_rows * cols, np.float32)
    flat[:tiles.size] = tiles.reshape(-1)
    x = flat.reshape(n_rows, cols)
    # every tile of x starts with 448 (tile boundaries are 128-aligned)
    assert np.all(x.reshape(-1, 128)[: tiles.shape[0], 0] == 448.0)
    _check_act(x, False, "encoder sweep")


def test_act_zero_and_negative_zero_tiles():
    x = np.zeros((3, 256), np.float32)
    x[1, :128] = -0.0
    x[2, 128:] = bf16_round(np.linspace(-1e-38, 1e-38, 128).astype(np.float32))
    _check_act(x, False, "zero tiles")
    _check_act(x, True, "zero tiles")


def test_act_empty():
    d = _dsmoe()
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s = d.quant_act_1x128(x)
    assert q.shape == (0, 256) and s.shape == (0, 2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_weights_small(dtype):
    d = _dsmoe()
    w = normal_bf16("qw_small", (3, 384, 640), 0.02, seed=1)
    w[1, 5, 7] = 3.0    # an outlier in one block
    banner(f"quant_w small {dtype}")
    q, s = d.quant_w_128x128(dev(w, dtype))
    qo, so = oq.quant_w_128x128(w)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)


def test_weights_v3_expert_shape():
    d = _dsmoe()
    w13 = normal_bf16("qw_v3_w13", (1, 4096, 7168), 0.02, seed=2)
    banner("quant_w v3 expert w13")
    q, s = d.quant_w_128x128(dev(w13, torch.bfloat16))
    qo, so = oq.quant_w_128x128(w13)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)


def _near_rounding_points(amax: float, seed: int) -> np.ndarray:
    """float32 tiles [n][128] whose element 0 is `amax` (so every tile has
    s = fl32(amax / 448), not a power of two) and whose other elements put
    v / s within 3 float32 ulps of an E4M3 rounding point (the midpoint of two
    neighbouring codes), both signs, normal and subnormal codes alike."""
    from oracle import e4m3
    vals = e4m3.decode(np.arange(0, 127, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    s = np.float32(np.float32(amax) / np.float32(448.0))
    out = []
    for m in mids:
        v0 = np.float32(np.float64(m) * np.float64(s))
        for k in range(-3, 4):
            v = v0
            for _ in range(abs(k)):
                v = np.nextafter(v, np.float32(np.inf if k > 0 else -np.inf), dtype=np.float32)
            out += [v, -v]
    out = np.array(out, np.float32)
    out = out[np.random.default_rng(seed).permutation(len(out))]
    n = -(-len(out) // 127)
    body = np.zeros(n * 127, np.float32)
    body[:len(out)] = out
    x = np.empty((n, 128), np.float32)
    x[:, 0] = np.float32(amax)
    x[:, 1:] = body.reshape(n, 127)
    return x


@pytest.mark.parametrize("amax", [448 * 1.37, 448 * 0.731, 448 * 3.3e-3, 448 * 7.77e4, 1.0e-3])
def test_codes_near_rounding_points_with_a_general_scale(amax):
    """Every quotient v / s lies within a few float32 ulps of an E4M3 rounding
    point, with a scale that is not a power of two: the codes must be those of
    the IEEE quotient (a reciprocal multiply would get some of them wrong)."""
    d = _dsmoe()
    from oracle import granularity as og
    x = _near_rounding_points(amax, seed=int(amax * 1000) % 9973)
    banner(f"near rounding points amax={amax} tiles={x.shape[0]}")
    _check_act(x.reshape(-1, 256) if x.shape[0] % 2 == 0 else x, False, f"near-midpoint act amax={amax}")
    # the same values as 128x128 weight blocks
    nb = x.shape[0] // 128 * 128
    if nb:
        w = x[:nb].reshape(nb // 128, 128, 128).transpose(1, 0, 2).reshape(128, -1)
        wt = dev(np.ascontiguousarray(w), torch.float32)
        q, s = d.quant_w_128x128(wt)
        qo, so = oq.quant_w_128x128(w)
        assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
        assert np.array_equal(host(q), qo)
    # per row (each row holds amax) and per tensor
    q, s = d.quant_rows(dev(x, torch.float32))
    qo, so = og.quant_rows(x)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)
    q, s, _ = d.quant_tensor(dev(x, torch.float32))
    qo, so = og.quant_tensor(x)
    assert host(s)[0] == so and np.array_equal(host(q), qo)


def _codes_from_midpoints(absv: torch.Tensor, mids: torch.Tensor) -> torch.Tensor:
    """Code magnitudes of |v| from the sorted midpoints of neighbouring E4M3
    magnitudes: the number of midpoints below |v|, moved up to the even code
    where |v| sits exactly on a midpoint (ties to even: the low bit of a code
    is the low bit of its mantissa); 126 (0x7E, 448) for everything above
    the last midpoint."""
    n = torch.bucketize(absv, mids)                   # midpoints strictly below |v|
    on_mid = (n < mids.numel()) & (absv == mids[n.clamp(max=mids.numel() - 1)])
    return (n + (on_mid & (n % 2 == 1)).to(n.dtype)).to(torch.uint8)


def test_every_float_up_to_464_encodes_to_the_codes_the_midpoints_give():
    """Every float32 with |v| <= 464, both signs (2.28e9 values), through both
    encoders at scale 1 (dsmoe_e4m3_codes): the quantisers' integer encoder
    and the SwiGLU epilogue's packed conversion must give the code the
    oracle's 126 midpoints give (464 is the tie between 448 and the step
    past it, which goes to 448; beyond 448 both saturate)."""
    d = _dsmoe()
    from oracle import e4m3
    mags = e4m3.decode(np.arange(0, 127, dtype=np.uint8))          # 0 .. 448, increasing
    mids64 = (mags[:-1] + mags[1:]) / 2
    assert mids64.size == 126 and np.all(np.diff(mids64) > 0)
    mids32 = mids64.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids64)      # exact in float32
    # the rule above agrees with the oracle's encoder on the midpoints and their neighbours
    probe = np.concatenate([mids32, np.nextafter(mids32, np.float32(0)), np.nextafter(mids32, np.float32(1e9)),
                            np.float32([0.0, 448.0, 460.0, 464.0])])
    want_probe = e4m3.encode(probe)
    got_probe = _codes_from_midpoints(torch.from_numpy(probe), torch.from_numpy(mids32)).numpy()
    assert np.array_equal(got_probe, want_probe)
    mids = torch.from_numpy(mids32).cuda()
    top = int(np.float32(464.0).view(np.uint32))                  # 0x43E80000
    chunk = 1 << 28
    banner(f"e4m3 sweep of every float32 with |v| <= 464 ({2 * (top + 1)} values)")
    checked = 0
    for start in range(0, top + 1, chunk):
        end = min(top + 1, start + chunk)
        bits = torch.arange(start, end, dtype=torch.int32, device="cuda")
        pos = bits.view(torch.float32)
        want_mag = _codes_from_midpoints(pos, mids)
        for sign, x in ((0, pos), (0x80, -pos)):                  # negation flips only the sign bit
            want = want_mag | sign
            for conv in ("encoder", "packed"):
                q = d.e4m3_codes(x, conv)
                bad = (q != want).nonzero()
                if bad.numel():
                    i = int(bad[0, 0])
                    raise AssertionError(
                        f"{conv}: {bad.numel()} codes differ in bits [{start:#x}, {end:#x}) sign {sign:#x}; "
                        f"first: v={float(x[i])!r} (bits {int(bits[i]):#x}) gpu {int(q[i]):#04x} "
                        f"want {int(want[i]):#04x}")
            checked += end - start
        del bits, pos, want_mag
    torch.cuda.synchronize()
    assert checked == 2 * (top + 1)
    print(f"[parity] e4m3 sweep: {checked} values, both encoders, every code as the midpoints give", flush=True)
