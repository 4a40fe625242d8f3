"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/dsmoe.h declares, and rejects invalid arguments with
the documented status before touching any device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dsmoe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsmoe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    import fp8_block_scaled_dsmoe_amd as d
    names = _declared()
    assert len(names) == 27, names
    for n in names:
        assert hasattr(d.lib, n), f"{n} not exported"
    assert sorted(d.EXPORTED) == names


def test_status_strings_and_version():
    import fp8_block_scaled_dsmoe_amd as d
    assert d.lib.dsmoe_abi_version() == 1
    want = ["DSMOE_OK", "DSMOE_ERR_NULL", "DSMOE_ERR_SHAPE", "DSMOE_ERR_ALIGN", "DSMOE_ERR_DTYPE",
            "DSMOE_ERR_WORKSPACE", "DSMOE_ERR_DEVICE", "DSMOE_ERR_LAUNCH"]
    for i, w in enumerate(want):
        assert d.lib.dsmoe_status_str(i).decode() == w
    assert d.lib.dsmoe_status_str(99).decode() == "DSMOE_ERR_UNKNOWN"


def test_workspace_size_is_host_arithmetic():
    import fp8_block_scaled_dsmoe_amd as d
    desc = d.MoEDesc(7168, 2048, 256, 8, 4, 8, 1)
    ws = d.moe_workspace_bytes(desc, 4096)
    tk = 4096 * 8
    # the two largest regions: routed outputs (f32) and the FP8 SwiGLU output
    assert ws >= tk * 7168 * 4 + (tk + 4096) * 2048
    assert ws < 2 * (tk * 7168 * 4 + (tk + 4096) * 2048)
    assert d.moe_workspace_bytes(d.MoEDesc(7168, 2048, 256, 8, 4, 8, 1), 0) > 0
    assert d.moe_workspace_bytes(d.MoEDesc(100, 2048, 256, 8, 4, 8, 1), 4096) == 0   # H % 128
    assert d.moe_workspace_bytes(d.MoEDesc(7168, 2048, 256, 7, 4, 8, 1), 4096) == 0  # E % G
    assert d.moe_workspace_bytes(d.MoEDesc(7168, 2048, 256, 8, 1, 64, 1), 4096) == 0  # K > 32


def _vp(v):
    return ctypes.c_void_p(v)


ALIGNED = 1 << 20          # fake, never dereferenced: validation fails before any use
MISALIGNED = ALIGNED + 2


def test_quant_validation_errors():
    import fp8_block_scaled_dsmoe_amd as d
    L = d.lib
    assert L.dsmoe_quant_act_1x128(_vp(ALIGNED), 7, 4, 128, _vp(ALIGNED), _vp(ALIGNED), None) == 4
    assert L.dsmoe_quant_act_1x128(_vp(ALIGNED), 0, 4, 100, _vp(ALIGNED), _vp(ALIGNED), None) == 2
    assert L.dsmoe_quant_act_1x128(_vp(ALIGNED), 0, -1, 128, _vp(ALIGNED), _vp(ALIGNED), None) == 2
    assert L.dsmoe_quant_act_1x128(None, 0, 4, 128, _vp(ALIGNED), _vp(ALIGNED), None) == 1
    assert L.dsmoe_quant_act_1x128(_vp(MISALIGNED), 0, 4, 128, _vp(ALIGNED), _vp(ALIGNED), None) == 3
    assert L.dsmoe_quant_act_1x128(None, 0, 0, 128, None, None, None) == 0       # empty: no-op
    assert L.dsmoe_quant_w_128x128(_vp(ALIGNED), 0, 1, 130, 128, _vp(ALIGNED), _vp(ALIGNED), None) == 2
    assert L.dsmoe_quant_w_128x128(_vp(ALIGNED), 0, 1, 128, 128, None, _vp(ALIGNED), None) == 1
    assert L.dsmoe_quant_w_128x128(_vp(ALIGNED), 0, 1, 128, 128, _vp(ALIGNED), _vp(MISALIGNED), None) == 3
    a = _vp(ALIGNED)
    assert L.dsmoe_transpose_w_128x128(a, a, 1, 130, 128, a, a, None) == 2
    assert L.dsmoe_transpose_w_128x128(a, a, -1, 128, 128, a, a, None) == 2
    assert L.dsmoe_transpose_w_128x128(a, a, 1, 128, 128, None, a, None) == 1
    assert L.dsmoe_transpose_w_128x128(a, a, 1, 128, 128, _vp(MISALIGNED), a, None) == 3
    assert L.dsmoe_transpose_w_128x128(None, None, 0, 128, 128, None, None, None) == 0
    assert L.dsmoe_e4m3_codes(a, 8, 2, a, None) == 4                 # unknown converter
    assert L.dsmoe_e4m3_codes(a, -1, 0, a, None) == 2
    assert L.dsmoe_e4m3_codes(None, 8, 1, a, None) == 1
    assert L.dsmoe_e4m3_codes(_vp(MISALIGNED), 8, 0, a, None) == 3
    assert L.dsmoe_e4m3_codes(None, 0, 1, None, None) == 0           # empty: no-op


def test_granularity_validation_errors():
    import fp8_block_scaled_dsmoe_amd as d
    L = d.lib
    a = _vp(ALIGNED)
    # per-row: cols a multiple of 8, at most 32768
    assert L.dsmoe_quant_rows(a, 0, 4, 100, a, a, None) == 2
    assert L.dsmoe_quant_rows(a, 0, 4, 32768 + 8, a, a, None) == 2
    assert L.dsmoe_quant_rows(a, 0, 4, 0, a, a, None) == 2
    assert L.dsmoe_quant_rows(a, 3, 4, 128, a, a, None) == 4
    assert L.dsmoe_quant_rows(a, 0, 4, 128, a, None, None) == 1
    assert L.dsmoe_quant_rows(_vp(MISALIGNED), 0, 4, 128, a, a, None) == 3
    assert L.dsmoe_quant_rows(None, 0, 0, 128, None, None, None) == 0          # empty: no-op
    # per-tensor: n a multiple of 8; scale and amax always required
    assert L.dsmoe_quant_tensor(a, 0, 12, a, a, a, None) == 2
    assert L.dsmoe_quant_tensor(a, 0, -8, a, a, a, None) == 2
    assert L.dsmoe_quant_tensor(a, 0, 16, a, a, None, None) == 1
    assert L.dsmoe_quant_tensor(None, 0, 16, a, a, a, None) == 1
    assert L.dsmoe_quant_tensor(a, 0, 16, a, a, _vp(MISALIGNED), None) == 3
    # GEMM at a granularity
    G = L.dsmoe_fp8_gemm_granularity
    ws = d.gemm_granularity_workspace_bytes(64, 256, 512)
    assert ws >= 64 * 512 + 256 * 512 + 64 * 4 * 4 + 2 * 4 * 4
    assert d.gemm_granularity_workspace_bytes(64, 200, 512) == 0
    assert d.gemm_granularity_workspace_bytes(64, 256, 32768 + 128) == 0
    assert G(a, a, 0, 64, 256, 512, 3, a, a, ws, None) == 2                     # unknown granularity
    assert G(a, a, 2, 64, 256, 512, 0, a, a, ws, None) == 4
    assert G(a, a, 0, 64, 200, 512, 0, a, a, ws, None) == 2
    assert G(a, a, 0, 64, 256, 512, 0, a, a, ws - 1, None) == 5
    assert G(a, a, 0, 64, 256, 512, 0, a, None, ws, None) == 5
    assert G(a, None, 0, 64, 256, 512, 0, a, a, ws, None) == 1
    assert G(a, a, 0, 64, 256, 512, 0, a, _vp(ALIGNED + 16), ws, None) == 3    # workspace 256-aligned
    assert G(None, None, 0, 0, 256, 512, 1, None, None, 0, None) == 0          # M = 0: no-op


def test_serving_validation_errors():
    import fp8_block_scaled_dsmoe_amd as d
    L = d.lib
    a = _vp(ALIGNED)
    assert L.dsmoe_plan_replicas(a, 0, 4, a, a, None) == 2
    assert L.dsmoe_plan_replicas(a, 2000, 4, a, a, None) == 2
    assert L.dsmoe_plan_replicas(a, 256, -1, a, a, None) == 2
    assert L.dsmoe_plan_replicas(a, 256, 2000, a, a, None) == 2
    assert L.dsmoe_plan_replicas(a, 256, 32, None, a, None) == 1
    assert L.dsmoe_plan_replicas(a, 256, 32, a, _vp(MISALIGNED), None) == 3
    assert L.dsmoe_place_replicas(a, a, 8, 100, 128, a, 4, a, a, None) == 2
    assert L.dsmoe_place_replicas(a, a, 8, 128, 128, a, 70000, a, a, None) == 2
    assert L.dsmoe_place_replicas(a, a, 0, 128, 128, a, 4, a, a, None) == 2
    assert L.dsmoe_place_replicas(a, a, 8, 128, 128, None, 4, a, a, None) == 1
    assert L.dsmoe_place_replicas(a, a, 8, 128, 128, a, 4, _vp(MISALIGNED), a, None) == 3
    assert L.dsmoe_place_replicas(None, None, 8, 128, 128, None, 0, None, None, None) == 0   # no slots: no-op
    assert L.dsmoe_slot_offsets(a, 16, a, a, 15, -1, a, None) == 2                    # fewer slots than experts
    assert L.dsmoe_slot_offsets(a, 16, a, a, 16 + 1025, -1, a, None) == 2
    assert L.dsmoe_slot_offsets(a, 16, None, a, 20, -1, a, None) == 1
    desc = d.MoEDesc(512, 256, 16, 4, 2, 2, 1)
    assert d.moe_serving_workspace_bytes(desc, 256, 20) > d.moe_workspace_bytes(desc, 256)
    assert d.moe_serving_workspace_bytes(desc, 256, 15) == 0
    dc = desc._c()
    wc = d._Weights(*([ALIGNED] * 9))
    F = L.dsmoe_moe_forward_serving
    ws = d.moe_serving_workspace_bytes(desc, 256, 20)
    byref = ctypes.byref
    assert F(byref(dc), byref(wc), a, a, 15, a, a, 256, a, 0, a, a, ws, None, None) == 2       # n_slots < E
    assert F(byref(dc), byref(wc), None, a, 20, a, a, 256, a, 0, a, a, ws, None, None) == 1
    assert F(byref(dc), byref(wc), a, a, 20, a, a, 256, a, 0, a, a, ws - 1, None, None) == 5
    assert F(byref(dc), byref(wc), a, a, 20, a, a, 256, a, 9, a, a, ws, None, None) == 4
    null_events = (ctypes.c_void_p * 5)()
    dbg = d._Debug()
    dbg.stage_events = ctypes.cast(null_events, ctypes.POINTER(ctypes.c_void_p))
    assert F(byref(dc), byref(wc), a, a, 20, a, a, 256, a, 0, a, a, ws, byref(dbg), None) == 1
    dbg = d._Debug()
    dbg.qa = MISALIGNED                                                            # debug buffers 4-byte aligned
    assert F(byref(dc), byref(wc), a, a, 20, a, a, 256, a, 0, a, a, ws, byref(dbg), None) == 3


def test_route_and_bias_validation_errors():
    import fp8_block_scaled_dsmoe_amd as d
    L = d.lib
    p = [_vp(ALIGNED)] * 8
    assert L.dsmoe_route(p[0], p[1], 10, 16, 3, 2, 2, *p[2:], None) == 2        # E % G
    assert L.dsmoe_route(p[0], p[1], 10, 16, 4, 5, 2, *p[2:], None) == 2        # Mg > G
    assert L.dsmoe_route(p[0], p[1], 10, 16, 4, 2, 9, *p[2:], None) == 2        # K > Mg*E/G
    assert L.dsmoe_route(p[0], p[1], 10, 2048, 8, 4, 8, *p[2:], None) == 2      # E too large
    assert L.dsmoe_route(p[0], p[1], 10, 256, 8, 4, 33, *p[2:], None) == 2      # K too large
    assert L.dsmoe_route(None, p[1], 10, 16, 4, 2, 2, *p[2:], None) == 1
    assert L.dsmoe_route(p[0], p[1], 10, 16, 4, 2, 2, _vp(MISALIGNED), *p[3:], None) == 3
    assert L.dsmoe_update_bias(_vp(ALIGNED), _vp(ALIGNED), 0, 10, 2, 0.001, None) == 2
    assert L.dsmoe_update_bias(None, _vp(ALIGNED), 16, 10, 2, 0.001, None) == 1
    assert L.dsmoe_update_bias(_vp(ALIGNED), _vp(ALIGNED), 16, 10, 0, 0.001, None) == 2


def test_gemm_validation_errors():
    import fp8_block_scaled_dsmoe_amd as d
    L = d.lib
    a = _vp(ALIGNED)
    assert L.dsmoe_fp8_grouped_gemm(a, a, None, a, 1, 64, a, a, 100, 128, a, 0, None) == 2
    assert L.dsmoe_fp8_grouped_gemm(a, a, None, a, 0, 64, a, a, 128, 128, a, 0, None) == 2
    assert L.dsmoe_fp8_grouped_gemm(a, a, None, a, 1, 64, a, a, 128, 128, a, 5, None) == 4
    assert L.dsmoe_fp8_grouped_gemm(a, a, None, None, 1, 64, a, a, 128, 128, a, 0, None) == 1
    assert L.dsmoe_fp8_grouped_gemm(a, a, None, a, 1, 64, _vp(MISALIGNED), a, 128, 128, a, 0, None) == 3
    assert L.dsmoe_fp8_grouped_gemm(None, None, None, None, 1, 0, None, None, 128, 128, None, 0, None) == 0
    # the contraction length is at most 32768 (256 chunks of 128)
    assert L.dsmoe_fp8_grouped_gemm(a, a, None, a, 1, 64, a, a, 128, 32768 + 128, a, 0, None) == 2


def test_wgrad_validation_errors():
    import fp8_block_scaled_dsmoe_amd as d
    L = d.lib
    a = _vp(ALIGNED)
    # M, N multiples of 128, P a multiple of 128, a known output dtype
    assert L.dsmoe_fp8_wgrad_grouped(a, a, a, a, a, 1, 100, 128, 128, a, 0, None) == 2
    assert L.dsmoe_fp8_wgrad_grouped(a, a, a, a, a, 1, 128, 128, 100, a, 0, None) == 2
    assert L.dsmoe_fp8_wgrad_grouped(a, a, a, a, a, 0, 128, 128, 128, a, 0, None) == 2
    assert L.dsmoe_fp8_wgrad_grouped(a, a, a, a, a, 1, 128, 128, 128, a, 5, None) == 4
    # the kernel's per-lane offsets cover 128 rows of P bytes in 32 bits
    big = (1 << 32) // 128 // 128 * 128
    assert L.dsmoe_fp8_wgrad_grouped(a, a, a, a, a, 1, 128, 128, big, a, 0, None) == 2
    assert L.dsmoe_fp8_wgrad_grouped(a, a, a, a, None, 1, 128, 128, big - 128, a, 0, None) == 1


def test_moe_forward_validation_errors():
    import fp8_block_scaled_dsmoe_amd as d
    L = d.lib
    desc = d._Desc(7168, 2048, 256, 8, 4, 8, 1)
    w = d._Weights(*([ALIGNED] * 9))
    a = _vp(ALIGNED)
    need = L.dsmoe_moe_workspace_bytes(ctypes.byref(desc), 64)
    args = lambda **kw: dict(dict(d=ctypes.byref(desc), w=ctypes.byref(w), bias=a, x=a, T=64, y=a, yt=0,
                                  counts=a, ws=a, ws_bytes=need, dbg=None, stream=None), **kw)
    call = lambda kw: L.dsmoe_moe_forward(*args(**kw).values())
    assert call({"ws_bytes": need - 1}) == 5
    assert call({"ws": None}) == 5
    assert call({"yt": 3}) == 4
    assert call({"counts": None}) == 1
    assert call({"x": _vp(MISALIGNED)}) == 3
    bad = d._Desc(7168, 2048, 256, 8, 4, 8, 2)
    assert call({"d": ctypes.byref(bad)}) == 2
    w_null = d._Weights(*([ALIGNED] * 4 + [None] + [ALIGNED] * 4))
    assert call({"w": ctypes.byref(w_null)}) == 1


def test_noalloc_forward_rejects_calls_beyond_its_scratch():
    """dsmoe_moe_forward_noalloc runs on a fixed device array: the V3 shapes
    fit up to T = 256 tokens; larger calls are refused before anything is
    enqueued (checked on the host, no device touched)."""
    import fp8_block_scaled_dsmoe_amd as d
    L = d.lib
    desc = d._Desc(7168, 2048, 256, 8, 4, 8, 1)
    assert L.dsmoe_moe_workspace_bytes(ctypes.byref(desc), 256) <= d.NOALLOC_SCRATCH_BYTES
    assert L.dsmoe_moe_workspace_bytes(ctypes.byref(desc), 300) > d.NOALLOC_SCRATCH_BYTES
    w = d._Weights(*([ALIGNED] * 9))
    a = _vp(ALIGNED)
    F = L.dsmoe_moe_forward_noalloc
    assert F(ctypes.byref(desc), ctypes.byref(w), a, a, 300, a, 0, a, None, None) == 5      # DSMOE_ERR_WORKSPACE
    assert F(ctypes.byref(desc), ctypes.byref(w), a, a, 4096, a, 0, a, None, None) == 5
    bad = d._Desc(7168, 2048, 256, 8, 4, 8, 2)
    assert F(ctypes.byref(bad), ctypes.byref(w), a, a, 64, a, 0, a, None, None) == 2


C_PROGRAM = r"""
#include <stdio.h>
#include "dsmoe.h"
int main(void) {
  dsmoe_moe_desc d = {7168, 2048, 256, 8, 4, 8, 1};
  if (dsmoe_abi_version() != 1) return 1;
  if (dsmoe_moe_workspace_bytes(&d, 4096) == 0) return 2;
  if (dsmoe_moe_serving_workspace_bytes(&d, 64, 320) == 0) return 3;
  if (dsmoe_gemm_granularity_workspace_bytes(4096, 4096, 7168) == 0) return 4;
  if (dsmoe_quant_rows(NULL, DSMOE_BF16, 4, 100, NULL, NULL, NULL) != DSMOE_ERR_SHAPE) return 5;
  if (dsmoe_plan_replicas(NULL, 0, 0, NULL, NULL, NULL) != DSMOE_ERR_SHAPE) return 6;
  puts(dsmoe_status_str(DSMOE_ERR_WORKSPACE));
  return 0;
}
"""


def test_header_is_c99_and_links_from_c(tmp_path):
    """include/dsmoe.h is a C header: a C99 program compiles against it, links
    to libdsmoe.so and makes host-only calls (no device work)."""
    import shutil
    import subprocess
    import fp8_block_scaled_dsmoe_amd as d
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(d.LIB_PATH)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
                        os.path.join(ROOT, "include"), str(src), "-L", libdir, "-ldsmoe",
                        f"-Wl,-rpath,{libdir}", "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, (out.returncode, out.stderr)
    assert out.stdout.strip() == "DSMOE_ERR_WORKSPACE"
