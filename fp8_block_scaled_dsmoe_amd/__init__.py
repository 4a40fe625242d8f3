"""Python binding of libdsmoe.so: the DeepSeekMoE FFN layer forward on the
fine-grained FP8 recipe, as hand-written HIP kernels for MI355X (gfx950).

Argument marshalling only.  Every step runs inside the HIP library; PyTorch is
used for device memory and the current stream.  Each wrapper checks dtypes,
devices, contiguity and shapes, allocates outputs that were not passed in,
and calls the C function of the same name (include/dsmoe.h).  A non-zero
status raises DsmoeError.  There is no fallback: if the library is missing,
importing this package fails.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

__all__ = [
    "DsmoeError", "MoEDesc", "MoEWeights", "LIB_PATH", "lib",
    "quant_act_1x128", "quant_w_128x128", "route", "fp8_grouped_gemm",
    "moe_workspace_bytes", "moe_forward", "update_bias", "quantize_layer_weights",
    "quant_rows", "quant_tensor", "gemm_granularity_workspace_bytes", "fp8_gemm_granularity",
    "GRANULARITIES", "plan_replicas", "place_replicas", "place_layer_replicas", "slot_offsets",
    "moe_serving_workspace_bytes", "moe_forward_serving", "transpose_w_128x128", "e4m3_codes", "BF16", "F32",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsmoe.so")
BF16, F32 = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python fp8_block_scaled_dsmoe_amd/build.py` "
        "(hipcc, gfx950). There is no non-HIP fallback.")

lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _i32, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int, ctypes.c_size_t


class _Desc(ctypes.Structure):
    _fields_ = [("H", _i64), ("I", _i64), ("E", _i32), ("G", _i32), ("Mg", _i32), ("K", _i32),
                ("n_shared", _i32)]


class _Weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w13", "s13", "w2", "s2", "w13_sh", "s13_sh", "w2_sh", "s2_sh",
                                   "router_w")]


_DEBUG_BUFFERS = ("qx", "sx", "logits", "topk_idx", "gates", "offsets", "perm", "inv")


class _Debug(ctypes.Structure):
    _fields_ = [(n, _vp) for n in _DEBUG_BUFFERS] + [("stage_events", ctypes.POINTER(_vp))] + \
               [("qa", _vp), ("sa", _vp)]


STAGE_EVENTS = 8
STAGES = ("quant_x", "router_logits", "route_select", "permute", "gemm1_swiglu_requant",
          "gemm2_routed", "gemm2_shared_combine")


lib.dsmoe_status_str.restype = ctypes.c_char_p
lib.dsmoe_status_str.argtypes = [_int]
lib.dsmoe_abi_version.restype = _int
lib.dsmoe_abi_version.argtypes = []
lib.dsmoe_quant_act_1x128.restype = _int
lib.dsmoe_quant_act_1x128.argtypes = [_vp, _int, _i64, _i64, _vp, _vp, _vp]
lib.dsmoe_quant_w_128x128.restype = _int
lib.dsmoe_quant_w_128x128.argtypes = [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp]
lib.dsmoe_route.restype = _int
lib.dsmoe_route.argtypes = [_vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
lib.dsmoe_fp8_grouped_gemm.restype = _int
lib.dsmoe_fp8_grouped_gemm.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _vp, _vp, _i64, _i64, _vp, _int, _vp]
lib.dsmoe_moe_workspace_bytes.restype = _sz
lib.dsmoe_moe_workspace_bytes.argtypes = [ctypes.POINTER(_Desc), _i64]
lib.dsmoe_moe_forward.restype = _int
lib.dsmoe_moe_forward.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Weights), _vp, _vp, _i64, _vp,
                                  _int, _vp, _vp, _sz, ctypes.POINTER(_Debug), _vp]
lib.dsmoe_moe_forward_noalloc.restype = _int
lib.dsmoe_moe_forward_noalloc.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Weights), _vp, _vp, _i64, _vp,
                                          _int, _vp, ctypes.POINTER(_Debug), _vp]
NOALLOC_SCRATCH_BYTES = 80 << 20
lib.dsmoe_token_tiles.restype = _i64
lib.dsmoe_token_tiles.argtypes = [_i64, _i32]
lib.dsmoe_quant_tokens_128.restype = _int
lib.dsmoe_quant_tokens_128.argtypes = [_vp, _int, _i64, _i64, _vp, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _vp]
lib.dsmoe_fp8_wgrad_grouped.restype = _int
lib.dsmoe_fp8_wgrad_grouped.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _int, _vp]
lib.dsmoe_swiglu_backward.restype = _int
lib.dsmoe_swiglu_backward.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp]
lib.dsmoe_gate_backward.restype = _int
lib.dsmoe_gate_backward.argtypes = [_vp, _vp, _int, _vp, _vp, _vp, _i64, _i32, _i32, _i64, _vp, _vp, _vp]
lib.dsmoe_combine_rows.restype = _int
lib.dsmoe_combine_rows.argtypes = [_vp, _int, _vp, _i64, _i32, _i64, _i64, _vp, _vp]
lib.dsmoe_update_bias.restype = _int
lib.dsmoe_update_bias.argtypes = [_vp, _vp, _i32, _i64, _i32, ctypes.c_float, _vp]
lib.dsmoe_quant_rows.restype = _int
lib.dsmoe_quant_rows.argtypes = [_vp, _int, _i64, _i64, _vp, _vp, _vp]
lib.dsmoe_quant_tensor.restype = _int
lib.dsmoe_quant_tensor.argtypes = [_vp, _int, _i64, _vp, _vp, _vp, _vp]
lib.dsmoe_gemm_granularity_workspace_bytes.restype = _sz
lib.dsmoe_gemm_granularity_workspace_bytes.argtypes = [_i64, _i64, _i64]
lib.dsmoe_fp8_gemm_granularity.restype = _int
lib.dsmoe_fp8_gemm_granularity.argtypes = [_vp, _vp, _int, _i64, _i64, _i64, _int, _vp, _vp, _sz, _vp]
lib.dsmoe_plan_replicas.restype = _int
lib.dsmoe_plan_replicas.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp]
lib.dsmoe_place_replicas.restype = _int
lib.dsmoe_place_replicas.argtypes = [_vp, _vp, _i32, _i64, _i64, _vp, _i32, _vp, _vp, _vp]
lib.dsmoe_transpose_w_128x128.restype = _int
lib.dsmoe_transpose_w_128x128.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]
lib.dsmoe_e4m3_codes.restype = _int
lib.dsmoe_e4m3_codes.argtypes = [_vp, _i64, _int, _vp, _vp]
lib.dsmoe_slot_offsets.restype = _int
lib.dsmoe_slot_offsets.argtypes = [_vp, _i32, _vp, _vp, _i32, _i64, _vp, _vp]
lib.dsmoe_moe_serving_workspace_bytes.restype = _sz
lib.dsmoe_moe_serving_workspace_bytes.argtypes = [ctypes.POINTER(_Desc), _i64, _i32]
lib.dsmoe_moe_forward_serving.restype = _int
lib.dsmoe_moe_forward_serving.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Weights), _vp, _vp, _i32,
                                          _vp, _vp, _i64, _vp, _int, _vp, _vp, _sz, ctypes.POINTER(_Debug), _vp]
SERVING_STAGE_EVENTS = 5
SERVING_STAGES = ("quant_route_permute", "gemm1_swiglu_requant", "gemm2_routed_and_shared", "combine")

EXPORTED = ("dsmoe_status_str", "dsmoe_abi_version", "dsmoe_quant_act_1x128", "dsmoe_quant_w_128x128",
            "dsmoe_route", "dsmoe_fp8_grouped_gemm", "dsmoe_moe_workspace_bytes", "dsmoe_moe_forward",
            "dsmoe_update_bias", "dsmoe_quant_rows", "dsmoe_quant_tensor",
            "dsmoe_gemm_granularity_workspace_bytes", "dsmoe_fp8_gemm_granularity",
            "dsmoe_plan_replicas", "dsmoe_place_replicas", "dsmoe_slot_offsets", "dsmoe_moe_serving_workspace_bytes",
            "dsmoe_moe_forward_serving", "dsmoe_transpose_w_128x128", "dsmoe_moe_forward_noalloc",
            "dsmoe_token_tiles", "dsmoe_quant_tokens_128", "dsmoe_fp8_wgrad_grouped", "dsmoe_swiglu_backward",
            "dsmoe_gate_backward", "dsmoe_combine_rows", "dsmoe_e4m3_codes")

# dsmoe_granularity codes
GRANULARITIES = {"tensor": 0, "channel": 1, "block": 2}


class DsmoeError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {lib.dsmoe_status_str(status).decode()} ({status})")


def _check(status: int, call: str):
    if status != 0:
        raise DsmoeError(status, call)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _dtype_code(dtype) -> int:
    if dtype == torch.bfloat16:
        return BF16
    if dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {dtype}")


def _out_dtype(code: int):
    return torch.float32 if code == F32 else torch.bfloat16


# ---------------------------------------------------------------------------

def quant_act_1x128(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                    scale: Optional[torch.Tensor] = None):
    """x [rows][cols] bf16/f32 -> (q uint8 [rows][cols], scale f32 [rows][cols/128])."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    _dev(x, x.dtype, "x")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty((rows, cols // 128), dtype=torch.float32, device=x.device) if scale is None else scale
    _dev(q, torch.uint8, "q")
    _dev(scale, torch.float32, "scale")
    _check(lib.dsmoe_quant_act_1x128(_p(x), _dtype_code(x.dtype), rows, cols, _p(q), _p(scale), _stream()),
           "dsmoe_quant_act_1x128")
    return q, scale


def quant_w_128x128(w: torch.Tensor, q: Optional[torch.Tensor] = None,
                    scale: Optional[torch.Tensor] = None):
    """w [n_mats][N][K] (or [N][K]) -> (q uint8 same shape, scale f32 [n_mats][N/128][K/128])."""
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    if w3.dim() != 3:
        raise ValueError("w must be 2-D or 3-D")
    _dev(w3, w.dtype, "w")
    nm, n, k = w3.shape
    q = torch.empty(w3.shape, dtype=torch.uint8, device=w.device) if q is None else q.view(nm, n, k)
    scale = (torch.empty((nm, n // 128, k // 128), dtype=torch.float32, device=w.device)
             if scale is None else scale.view(nm, n // 128, k // 128))
    _dev(q, torch.uint8, "q")
    _dev(scale, torch.float32, "scale")
    _check(lib.dsmoe_quant_w_128x128(_p(w3), _dtype_code(w.dtype), nm, n, k, _p(q), _p(scale), _stream()),
           "dsmoe_quant_w_128x128")
    if squeeze:
        return q[0], scale[0]
    return q, scale


E4M3_CONVERTERS = {"encoder": 0, "packed": 1}


def e4m3_codes(x: torch.Tensor, converter: str = "encoder", q: Optional[torch.Tensor] = None):
    """float32 x (any shape) -> uint8 E4M3FN codes of x at scale 1, from the
    quantisers' integer encoder ("encoder") or the SwiGLU epilogue's packed
    conversion ("packed"); see dsmoe_e4m3_codes."""
    _dev(x, torch.float32, "x")
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if q is None else q
    _dev(q, torch.uint8, "q")
    if q.numel() != x.numel():
        raise ValueError("q must have as many elements as x")
    _check(lib.dsmoe_e4m3_codes(_p(x), x.numel(), E4M3_CONVERTERS[converter], _p(q), _stream()),
           "dsmoe_e4m3_codes")
    return q


def transpose_w_128x128(q: torch.Tensor, s: torch.Tensor):
    """Codes [n_mats][N][K] (or [N][K]) and their 128x128 scales -> those of
    W^T: codes [..][K][N], scales [..][K/128][N/128] (dsmoe_transpose_w_128x128)."""
    squeeze = q.dim() == 2
    q3 = q.unsqueeze(0) if squeeze else q
    s3 = s.unsqueeze(0) if squeeze else s
    _dev(q3, torch.uint8, "q")
    _dev(s3, torch.float32, "s")
    nm, n, k = q3.shape
    qt = torch.empty((nm, k, n), dtype=torch.uint8, device=q.device)
    st = torch.empty((nm, k // 128, n // 128), dtype=torch.float32, device=q.device)
    _check(lib.dsmoe_transpose_w_128x128(_p(q3), _p(s3), nm, n, k, _p(qt), _p(st), _stream()),
           "dsmoe_transpose_w_128x128")
    return (qt[0], st[0]) if squeeze else (qt, st)


def route(logits: torch.Tensor, bias: torch.Tensor, n_groups: int, groups_kept: int, top_k: int):
    """logits f32 [T][E], bias f32 [E] -> dict of topk_idx, gates, counts, offsets, perm, inv."""
    _dev(logits, torch.float32, "logits")
    _dev(bias, torch.float32, "bias")
    t, e = logits.shape
    dev = logits.device
    out = {
        "topk_idx": torch.empty((t, top_k), dtype=torch.int32, device=dev),
        "gates": torch.empty((t, top_k), dtype=torch.float32, device=dev),
        "counts": torch.empty((e,), dtype=torch.int32, device=dev),
        "offsets": torch.empty((e + 1,), dtype=torch.int32, device=dev),
        "perm": torch.empty((t * top_k,), dtype=torch.int32, device=dev),
        "inv": torch.empty((t, top_k), dtype=torch.int32, device=dev),
    }
    _check(lib.dsmoe_route(_p(logits), _p(bias), t, e, n_groups, groups_kept, top_k,
                           _p(out["topk_idx"]), _p(out["gates"]), _p(out["counts"]), _p(out["offsets"]),
                           _p(out["perm"]), _p(out["inv"]), _stream()), "dsmoe_route")
    return out


def fp8_grouped_gemm(a: torch.Tensor, a_scale: torch.Tensor, offsets: torch.Tensor, w: torch.Tensor,
                     w_scale: torch.Tensor, out_dtype=torch.bfloat16, a_rows: Optional[torch.Tensor] = None,
                     m_total: Optional[int] = None, c: Optional[torch.Tensor] = None):
    """Grouped block-scaled FP8 GEMM (see dsmoe_fp8_grouped_gemm).

    a uint8 [*][K], a_scale f32 [*][K/128], offsets int32 [G+1] (device),
    w uint8 [G][N][K], w_scale f32 [G][N/128][K/128]; a_rows int32 [M_total]
    or None.  m_total defaults to len(a_rows) or a.shape[0].
    """
    _dev(a, torch.uint8, "a")
    _dev(a_scale, torch.float32, "a_scale")
    _dev(offsets, torch.int32, "offsets")
    if w.dim() == 2:
        w = w.unsqueeze(0)
        w_scale = w_scale.unsqueeze(0)
    _dev(w, torch.uint8, "w")
    _dev(w_scale, torch.float32, "w_scale")
    if a_rows is not None:
        _dev(a_rows, torch.int32, "a_rows")
    g, n, k = w.shape
    if offsets.numel() != g + 1:
        raise ValueError("offsets must have G+1 entries")
    if m_total is None:
        m_total = a_rows.numel() if a_rows is not None else a.shape[0]
    if c is None:
        c = torch.empty((m_total, n), dtype=out_dtype, device=a.device)
    _dev(c, c.dtype, "c")
    _check(lib.dsmoe_fp8_grouped_gemm(_p(a), _p(a_scale), _p(a_rows), _p(offsets), g, m_total, _p(w),
                                      _p(w_scale), n, k, _p(c), _dtype_code(c.dtype), _stream()),
           "dsmoe_fp8_grouped_gemm")
    return c


def quant_rows(x: torch.Tensor, q: Optional[torch.Tensor] = None,
               scale: Optional[torch.Tensor] = None):
    """x [rows][cols] bf16/f32 -> (q uint8 [rows][cols], scale f32 [rows]): one
    scale per row over the whole row (see dsmoe_quant_rows)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    _dev(x, x.dtype, "x")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty((rows,), dtype=torch.float32, device=x.device) if scale is None else scale
    _dev(q, torch.uint8, "q")
    _dev(scale, torch.float32, "scale")
    _check(lib.dsmoe_quant_rows(_p(x), _dtype_code(x.dtype), rows, cols, _p(q), _p(scale), _stream()),
           "dsmoe_quant_rows")
    return q, scale


QUANT_TENSOR_SCRATCH_FLOATS = 2048


def quant_tensor(x: torch.Tensor, q: Optional[torch.Tensor] = None, scale: Optional[torch.Tensor] = None,
                 scratch: Optional[torch.Tensor] = None):
    """x (any shape) bf16/f32 -> (q uint8 same shape, scale f32 [1], amax f32 [1]):
    one scale for the whole tensor (see dsmoe_quant_tensor).  scratch: f32
    [QUANT_TENSOR_SCRATCH_FLOATS]; the returned amax is a view of its first
    element."""
    _dev(x, x.dtype, "x")
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty((1,), dtype=torch.float32, device=x.device) if scale is None else scale
    if scratch is None:
        scratch = torch.empty((QUANT_TENSOR_SCRATCH_FLOATS,), dtype=torch.float32, device=x.device)
    _dev(q, torch.uint8, "q")
    _dev(scale, torch.float32, "scale")
    _dev(scratch, torch.float32, "scratch")
    if q.numel() != x.numel():
        raise ValueError("q must have as many elements as x")
    if scratch.numel() < QUANT_TENSOR_SCRATCH_FLOATS:
        raise ValueError(f"scratch must hold {QUANT_TENSOR_SCRATCH_FLOATS} floats")
    _check(lib.dsmoe_quant_tensor(_p(x), _dtype_code(x.dtype), x.numel(), _p(q), _p(scale), _p(scratch),
                                  _stream()), "dsmoe_quant_tensor")
    return q, scale, scratch[:1]


def gemm_granularity_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(lib.dsmoe_gemm_granularity_workspace_bytes(m, n, k))


def fp8_gemm_granularity(a: torch.Tensor, w: torch.Tensor, granularity: str,
                         c: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """c f32 [M][N] = A W^T with A [M][K] and W [N][K] (bf16 or f32, same
    dtype) quantised to E4M3 at `granularity` ("tensor", "channel" or
    "block"); see dsmoe_fp8_gemm_granularity."""
    if granularity not in GRANULARITIES:
        raise ValueError(f"granularity must be one of {tuple(GRANULARITIES)}")
    if a.dim() != 2 or w.dim() != 2:
        raise ValueError("a and w must be 2-D")
    _dev(a, a.dtype, "a")
    _dev(w, a.dtype, "w")
    m, k = a.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("a and w must have the same K")
    c = torch.empty((m, n), dtype=torch.float32, device=a.device) if c is None else c
    _dev(c, torch.float32, "c")
    need = gemm_granularity_workspace_bytes(m, n, k)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=a.device)
    _dev(workspace, torch.uint8, "workspace")
    _check(lib.dsmoe_fp8_gemm_granularity(_p(a), _p(w), _dtype_code(a.dtype), m, n, k,
                                          GRANULARITIES[granularity], _p(c), _p(workspace),
                                          workspace.numel(), _stream()), "dsmoe_fp8_gemm_granularity")
    return c


@dataclasses.dataclass(frozen=True)
class MoEDesc:
    H: int
    I: int
    E: int
    G: int
    Mg: int
    K: int
    n_shared: int = 1

    def _c(self):
        return _Desc(self.H, self.I, self.E, self.G, self.Mg, self.K, self.n_shared)


@dataclasses.dataclass
class MoEWeights:
    """Quantised layer weights on the device (see dsmoe_moe_weights)."""
    w13: torch.Tensor
    s13: torch.Tensor
    w2: torch.Tensor
    s2: torch.Tensor
    w13_sh: Optional[torch.Tensor]
    s13_sh: Optional[torch.Tensor]
    w2_sh: Optional[torch.Tensor]
    s2_sh: Optional[torch.Tensor]
    router_w: torch.Tensor

    def _c(self):
        return _Weights(*[None if t is None else t.data_ptr() for t in (
            self.w13, self.s13, self.w2, self.s2, self.w13_sh, self.s13_sh, self.w2_sh, self.s2_sh,
            self.router_w)])


def quantize_layer_weights(w13: torch.Tensor, w2: torch.Tensor, router_w: torch.Tensor,
                           w13_sh: Optional[torch.Tensor] = None,
                           w2_sh: Optional[torch.Tensor] = None) -> MoEWeights:
    """Quantise bf16 expert weights with dsmoe_quant_w_128x128."""
    q13, s13 = quant_w_128x128(w13)
    q2, s2 = quant_w_128x128(w2)
    q13s = s13s = q2s = s2s = None
    if w13_sh is not None:
        q13s, s13s = quant_w_128x128(w13_sh)
        q2s, s2s = quant_w_128x128(w2_sh)
    return MoEWeights(q13, s13, q2, s2, q13s, s13s, q2s, s2s, router_w)


def moe_workspace_bytes(desc: MoEDesc, T: int) -> int:
    d = desc._c()
    return int(lib.dsmoe_moe_workspace_bytes(ctypes.byref(d), T))


def _debug_buffers(desc, T, dev, debug, stage_events, n_events):
    """(dict of device tensors or None, _Debug or None) for a forward call."""
    dbg = None
    dbg_c = None
    if debug:
        rows = T * desc.K + (T if desc.n_shared else 0)
        dbg = {
            "qx": torch.empty((T, desc.H), dtype=torch.uint8, device=dev),
            "sx": torch.empty((T, desc.H // 128), dtype=torch.float32, device=dev),
            "logits": torch.empty((T, desc.E), dtype=torch.float32, device=dev),
            "topk_idx": torch.empty((T, desc.K), dtype=torch.int32, device=dev),
            "gates": torch.empty((T, desc.K), dtype=torch.float32, device=dev),
            "offsets": torch.empty((desc.E + 1,), dtype=torch.int32, device=dev),
            "perm": torch.empty((T * desc.K,), dtype=torch.int32, device=dev),
            "inv": torch.empty((T, desc.K), dtype=torch.int32, device=dev),
            "qa": torch.empty((rows, desc.I), dtype=torch.uint8, device=dev),
            "sa": torch.empty((rows, desc.I // 128), dtype=torch.float32, device=dev),
        }
        dbg_c = _Debug(*[dbg[n].data_ptr() for n in _DEBUG_BUFFERS])
        dbg_c.qa = dbg["qa"].data_ptr()
        dbg_c.sa = dbg["sa"].data_ptr()
    if stage_events is not None:
        if len(stage_events) != n_events:
            raise ValueError(f"stage_events needs {n_events} handles")
        arr = (_vp * n_events)(*stage_events)
        if dbg_c is None:
            dbg_c = _Debug()
        dbg_c.stage_events = ctypes.cast(arr, ctypes.POINTER(_vp))
        dbg_c._keep = arr
    return dbg, dbg_c


def moe_forward(desc: MoEDesc, weights: MoEWeights, bias: torch.Tensor, x: torch.Tensor,
                out_dtype=torch.bfloat16, y: Optional[torch.Tensor] = None,
                counts: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                debug: bool = False, stage_events=None):
    """The layer forward (dsmoe_moe_forward).  Returns (y, counts, dbg) where
    dbg is a dict of intermediates when debug=True, else None.
    stage_events: optional sequence of STAGE_EVENTS raw hipEvent_t handles
    (ints) recorded around the stages (see dsmoe_moe_debug)."""
    _dev(x, torch.bfloat16, "x")
    _dev(bias, torch.float32, "bias")
    _dev(weights.router_w, torch.bfloat16, "router_w")
    T = x.shape[0]
    dev = x.device
    if y is None:
        y = torch.empty((T, desc.H), dtype=out_dtype, device=dev)
    if counts is None:
        counts = torch.empty((desc.E,), dtype=torch.int32, device=dev)
    need = moe_workspace_bytes(desc, T)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    dbg, dbg_c = _debug_buffers(desc, T, dev, debug, stage_events, STAGE_EVENTS)
    d = desc._c()
    wc = weights._c()
    _check(lib.dsmoe_moe_forward(ctypes.byref(d), ctypes.byref(wc), _p(bias), _p(x), T, _p(y),
                                 _dtype_code(y.dtype), _p(counts), _p(workspace), workspace.numel(),
                                 ctypes.byref(dbg_c) if dbg_c is not None else None, _stream()),
           "dsmoe_moe_forward")
    return y, counts, dbg


def moe_forward_noalloc(desc: MoEDesc, weights: MoEWeights, bias: torch.Tensor, x: torch.Tensor,
                        out_dtype=torch.bfloat16, y: Optional[torch.Tensor] = None,
                        counts: Optional[torch.Tensor] = None, debug: bool = False, stage_events=None):
    """The layer forward on the library's own device scratch
    (dsmoe_moe_forward_noalloc): no workspace; with y and counts given, the
    call allocates nothing.  Returns (y, counts, dbg) as moe_forward does."""
    _dev(x, torch.bfloat16, "x")
    _dev(bias, torch.float32, "bias")
    _dev(weights.router_w, torch.bfloat16, "router_w")
    T = x.shape[0]
    dev = x.device
    if y is None:
        y = torch.empty((T, desc.H), dtype=out_dtype, device=dev)
    if counts is None:
        counts = torch.empty((desc.E,), dtype=torch.int32, device=dev)
    dbg, dbg_c = _debug_buffers(desc, T, dev, debug, stage_events, STAGE_EVENTS)
    d = desc._c()
    wc = weights._c()
    _check(lib.dsmoe_moe_forward_noalloc(ctypes.byref(d), ctypes.byref(wc), _p(bias), _p(x), T, _p(y),
                                         _dtype_code(y.dtype), _p(counts),
                                         ctypes.byref(dbg_c) if dbg_c is not None else None, _stream()),
           "dsmoe_moe_forward_noalloc")
    return y, counts, dbg


def token_tiles(m_total: int, n_groups: int) -> int:
    """Upper bound on the 128-row token tiles of m_total rows in n_groups groups."""
    return int(lib.dsmoe_token_tiles(m_total, n_groups))


def quant_tokens_128(src: torch.Tensor, offsets: torch.Tensor, m_total: Optional[int] = None,
                     rows: Optional[torch.Tensor] = None, row_scale: Optional[torch.Tensor] = None):
    """1x128 tiles along the rows of each group (dsmoe_quant_tokens_128).

    src bf16/f32 [n_src][C]; offsets int32 [G+1] (device); rows int32
    [m_total] (source row per output row) or None; row_scale f32 [m_total]
    or None.  Returns (qt uint8 [C][P], scales f32 [P/128][C], chunk_off
    int32 [G+1])."""
    if src.dtype not in (torch.bfloat16, torch.float32) or not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous bf16 or f32 CUDA tensor")
    _dev(offsets, torch.int32, "offsets")
    if rows is not None:
        _dev(rows, torch.int32, "rows")
    if row_scale is not None:
        _dev(row_scale, torch.float32, "row_scale")
    G = offsets.numel() - 1
    n_src, C = src.shape
    if m_total is None:
        m_total = rows.numel() if rows is not None else n_src
    P = 128 * token_tiles(m_total, G)
    dev = src.device
    qt = torch.empty((C, max(P, 128)), dtype=torch.uint8, device=dev)
    sc = torch.empty((max(P, 128) // 128, C), dtype=torch.float32, device=dev)
    cho = torch.empty((G + 1,), dtype=torch.int32, device=dev)
    _check(lib.dsmoe_quant_tokens_128(_p(src), _dtype_code(src.dtype), n_src, C, _p(rows), _p(row_scale),
                                      _p(offsets), G, m_total, _p(cho), _p(qt), _p(sc), _stream()),
           "dsmoe_quant_tokens_128")
    return qt[:, :P], sc[:P // 128], cho


def fp8_wgrad_grouped(at: torch.Tensor, sa: torch.Tensor, bt: torch.Tensor, sb: torch.Tensor,
                      chunk_off: torch.Tensor, out_dtype=torch.float32, c: Optional[torch.Tensor] = None):
    """Per-group weight gradient c[g] = A_g B_g^T over the group's token tiles
    (dsmoe_fp8_wgrad_grouped); at/sa and bt/sb from quant_tokens_128 on the
    same offsets.  Returns c [G][M][N]."""
    _dev(at, torch.uint8, "at")
    _dev(bt, torch.uint8, "bt")
    _dev(sa, torch.float32, "sa")
    _dev(sb, torch.float32, "sb")
    _dev(chunk_off, torch.int32, "chunk_off")
    G = chunk_off.numel() - 1
    M, P = at.shape
    N = bt.shape[0]
    if bt.shape[1] != P:
        raise ValueError("at and bt must span the same token tiles")
    if c is None:
        c = torch.empty((G, M, N), dtype=out_dtype, device=at.device)
    # the codes' rows are P apart: pass the strided views' base with P as the stride
    _check(lib.dsmoe_fp8_wgrad_grouped(_p(at), _p(sa), _p(bt), _p(sb), _p(chunk_off), G, M, N,
                                       at.stride(0), _p(c), _dtype_code(c.dtype), _stream()),
           "dsmoe_fp8_wgrad_grouped")
    return c


def swiglu_backward(h: torch.Tensor, da: torch.Tensor, row_gate: Optional[torch.Tensor] = None,
                    recompute_a: bool = False):
    """SwiGLU backward on the recomputed activation (dsmoe_swiglu_backward).
    h f32 [rows][2I], da f32 [rows][I], row_gate f32 [rows] or None.
    Returns (dh f32 [rows][2I], a f32 [rows][I] or None)."""
    _dev(h, torch.float32, "h")
    _dev(da, torch.float32, "da")
    if row_gate is not None:
        _dev(row_gate, torch.float32, "row_gate")
    rows, I = da.shape
    dh = torch.empty((rows, 2 * I), dtype=torch.float32, device=h.device)
    a = torch.empty((rows, I), dtype=torch.float32, device=h.device) if recompute_a else None
    _check(lib.dsmoe_swiglu_backward(_p(h), _p(da), _p(row_gate), rows, I, _p(dh), _p(a), _stream()),
           "dsmoe_swiglu_backward")
    return dh, a


def gate_backward(dy: torch.Tensor, o: torch.Tensor, inv: torch.Tensor, topk_idx: torch.Tensor,
                  logits: torch.Tensor):
    """Gradients of the gates and the router logits (dsmoe_gate_backward).
    dy bf16 [T][H]; o bf16/f32 [T*K][H] ungated expert outputs; inv, topk_idx
    int32 [T][K]; logits f32 [T][E].  Returns (dgate f32 [T][K], dlogits f32
    [T][E])."""
    _dev(dy, torch.bfloat16, "dy")
    _dev(inv, torch.int32, "inv")
    _dev(topk_idx, torch.int32, "topk_idx")
    _dev(logits, torch.float32, "logits")
    T, H = dy.shape
    K = topk_idx.shape[1]
    E = logits.shape[1]
    dgate = torch.empty((T, K), dtype=torch.float32, device=dy.device)
    dlogits = torch.empty((T, E), dtype=torch.float32, device=dy.device)
    _check(lib.dsmoe_gate_backward(_p(dy), _p(o), _dtype_code(o.dtype), _p(inv), _p(topk_idx), _p(logits), T, E,
                                   K, H, _p(dgate), _p(dlogits), _stream()), "dsmoe_gate_backward")
    return dgate, dlogits


def combine_rows(o: torch.Tensor, inv: torch.Tensor, shared0: int = -1, y: Optional[torch.Tensor] = None):
    """y[t] = o[shared0 + t] (if shared0 >= 0) + sum_k o[inv[t][k]] in float32
    (dsmoe_combine_rows); o and y bf16 or f32."""
    _dev(inv, torch.int32, "inv")
    T, K = inv.shape
    H = o.shape[1]
    if y is None:
        y = torch.empty((T, H), dtype=o.dtype, device=o.device)
    _check(lib.dsmoe_combine_rows(_p(o), _dtype_code(o.dtype), _p(inv), T, K, H, shared0, _p(y), _stream()),
           "dsmoe_combine_rows")
    return y


def expert_rows(dbg: dict, T: int, K: int, n_shared: int = 1):
    """The forward's row structure over the routed groups and the shared one
    (index plumbing only): offsets [E+1+n_shared], perm [T*K + n_shared*T]
    (row -> token) and the row gates (gate of each routed row, 1 for the
    shared expert's rows), from a debug dict of moe_forward."""
    dev = dbg["perm"].device
    rows = T * K + (T if n_shared else 0)
    off, perm = dbg["offsets"], dbg["perm"]
    rg = torch.ones((rows,), dtype=torch.float32, device=dev)
    rg[dbg["inv"].reshape(-1).long()] = dbg["gates"].reshape(-1)
    if n_shared:
        off = torch.cat([off, torch.tensor([rows], dtype=torch.int32, device=dev)])
        perm = torch.cat([perm, torch.arange(T, dtype=torch.int32, device=dev)])
    return off, perm, rg


def moe_backward_experts(dbg: dict, x: torch.Tensor, dy: torch.Tensor, w, wt, T: int, K: int,
                         n_shared: int = 1, wgrad_dtype=torch.float32, stage_events=None):
    """The FP8 backward of the routed experts and the shared one, as a chain of
    the library's calls on the forward's intermediates (dbg from moe_forward
    with debug=True: routing, x codes, codes of a).

    x bf16 [T][H] (the layer input), dy bf16 [T][H] (gradient of y);
    w = (q13, s13, q2, s2) and wt = their block transposes, over the routed
    experts followed by the shared one.  Steps: h = x W13^T recomputed (the
    SwiGLU input) and the ungated expert outputs o = a W2^T; the gate and
    router-logit gradients; the dgrad of the down projection; the SwiGLU
    backward (recomputing a); the dgrad of the gate/up projection, summed per
    token; the weight gradients dW2 and dW13 on 1x128 tiles along each
    expert's tokens.  stage_events: optional 9 torch.cuda.Events recorded at
    the start and after each of the 8 steps.  Returns a dict of device
    tensors: h, o, dgate, dlogits, da, dh, a, dx, dw2, dw13."""
    off, perm, rg = expert_rows(dbg, T, K, n_shared)
    rows = perm.numel()
    q13, s13, q2, s2 = w
    q13t, s13t, q2t, s2t = wt
    ev = stage_events or [None] * 9
    mark = lambda i: ev[i].record() if ev[i] is not None else None
    out = {}
    mark(0)
    out["h"] = fp8_grouped_gemm(dbg["qx"], dbg["sx"], off, q13, s13, out_dtype=torch.float32, a_rows=perm,
                                m_total=rows)
    out["o"] = fp8_grouped_gemm(dbg["qa"], dbg["sa"], off, q2, s2, out_dtype=torch.float32, m_total=rows)
    mark(1)
    out["dgate"], out["dlogits"] = gate_backward(dy, out["o"], dbg["inv"], dbg["topk_idx"], dbg["logits"])
    mark(2)
    qdy, sdy = quant_act_1x128(dy)
    out["da"] = fp8_grouped_gemm(qdy, sdy, off, q2t, s2t, out_dtype=torch.float32, a_rows=perm, m_total=rows)
    mark(3)
    out["dh"], out["a"] = swiglu_backward(out["h"], out["da"], rg, recompute_a=True)
    mark(4)
    qdh, sdh = quant_act_1x128(out["dh"])
    dx_rows = fp8_grouped_gemm(qdh, sdh, off, q13t, s13t, out_dtype=torch.float32, m_total=rows)
    out["dx"] = combine_rows(dx_rows, dbg["inv"], shared0=T * K if n_shared else -1)
    mark(5)
    qdo, sdo, cho = quant_tokens_128(dy, off, m_total=rows, rows=perm, row_scale=rg)
    qa_t, sa_t, _ = quant_tokens_128(out["a"], off)
    qdh_t, sdh_t, _ = quant_tokens_128(out["dh"], off)
    qx_t, sx_t, _ = quant_tokens_128(x, off, m_total=rows, rows=perm)
    mark(6)
    out["dw2"] = fp8_wgrad_grouped(qdo, sdo, qa_t, sa_t, cho, out_dtype=wgrad_dtype)
    mark(7)
    out["dw13"] = fp8_wgrad_grouped(qdh_t, sdh_t, qx_t, sx_t, cho, out_dtype=wgrad_dtype)
    mark(8)
    return out


BACKWARD_STAGES = ("recompute_h_and_o", "gate_router_grad", "dgrad_down", "swiglu_backward",
                   "dgrad_gate_up_and_sum", "token_tiles", "wgrad_w2", "wgrad_w13")


def plan_replicas(counts: torch.Tensor, n_extra: int):
    """counts int32 [E] (device) -> (slot_first int32 [E+1], slot_expert int32
    [E + n_extra]) on the device (dsmoe_plan_replicas)."""
    _dev(counts, torch.int32, "counts")
    e = counts.numel()
    slot_first = torch.empty((e + 1,), dtype=torch.int32, device=counts.device)
    slot_expert = torch.empty((e + n_extra,), dtype=torch.int32, device=counts.device)
    _check(lib.dsmoe_plan_replicas(_p(counts), e, n_extra, _p(slot_first), _p(slot_expert), _stream()),
           "dsmoe_plan_replicas")
    return slot_first, slot_expert


def place_replicas(w: torch.Tensor, w_scale: torch.Tensor, slot_expert: torch.Tensor):
    """w uint8 [E][N][K], w_scale f32 [E][N/128][K/128] -> (w_slots [S][N][K],
    s_slots [S][N/128][K/128]) with slot s holding expert slot_expert[s]
    (dsmoe_place_replicas)."""
    _dev(w, torch.uint8, "w")
    _dev(w_scale, torch.float32, "w_scale")
    _dev(slot_expert, torch.int32, "slot_expert")
    e, n, k = w.shape
    S = slot_expert.numel()
    w_slots = torch.empty((S, n, k), dtype=torch.uint8, device=w.device)
    s_slots = torch.empty((S, n // 128, k // 128), dtype=torch.float32, device=w.device)
    _check(lib.dsmoe_place_replicas(_p(w), _p(w_scale), e, n, k, _p(slot_expert), S, _p(w_slots), _p(s_slots),
                                    _stream()), "dsmoe_place_replicas")
    return w_slots, s_slots


def place_layer_replicas(weights: "MoEWeights", slot_expert: torch.Tensor) -> "MoEWeights":
    """The layer's weights with W13 and W2 laid out over the slots of a plan;
    the shared expert and the router are shared with `weights`."""
    w13, s13 = place_replicas(weights.w13, weights.s13, slot_expert)
    w2, s2 = place_replicas(weights.w2, weights.s2, slot_expert)
    return MoEWeights(w13, s13, w2, s2, weights.w13_sh, weights.s13_sh, weights.w2_sh, weights.s2_sh,
                      weights.router_w)


def slot_offsets(offsets: torch.Tensor, slot_first: torch.Tensor, slot_expert: torch.Tensor,
                 extra_rows: int = -1):
    """Group offsets of the slots of a plan (dsmoe_slot_offsets): int32
    [S + 2], the last entry meaningful only when extra_rows >= 0."""
    for t, n in ((offsets, "offsets"), (slot_first, "slot_first"), (slot_expert, "slot_expert")):
        _dev(t, torch.int32, n)
    e = offsets.numel() - 1
    S = slot_expert.numel()
    phys = torch.empty((S + 2,), dtype=torch.int32, device=offsets.device)
    _check(lib.dsmoe_slot_offsets(_p(offsets), e, _p(slot_first), _p(slot_expert), S, extra_rows, _p(phys),
                                  _stream()), "dsmoe_slot_offsets")
    return phys


def moe_serving_workspace_bytes(desc: "MoEDesc", T: int, n_slots: int) -> int:
    d = desc._c()
    return int(lib.dsmoe_moe_serving_workspace_bytes(ctypes.byref(d), T, n_slots))


def moe_forward_serving(desc: "MoEDesc", slot_weights: "MoEWeights", slot_first: torch.Tensor,
                        slot_expert: torch.Tensor, bias: torch.Tensor, x: torch.Tensor,
                        out_dtype=torch.bfloat16, y: Optional[torch.Tensor] = None,
                        counts: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        debug: bool = False, stage_events=None):
    """The layer forward over the slots of a replica plan, the shared expert
    as one more routed group (dsmoe_moe_forward_serving).  Returns (y, counts,
    dbg) as moe_forward does.  stage_events: optional SERVING_STAGE_EVENTS raw
    hipEvent_t handles (ints)."""
    _dev(x, torch.bfloat16, "x")
    _dev(bias, torch.float32, "bias")
    _dev(slot_first, torch.int32, "slot_first")
    _dev(slot_expert, torch.int32, "slot_expert")
    T = x.shape[0]
    S = slot_expert.numel()
    dev = x.device
    if y is None:
        y = torch.empty((T, desc.H), dtype=out_dtype, device=dev)
    if counts is None:
        counts = torch.empty((desc.E,), dtype=torch.int32, device=dev)
    need = moe_serving_workspace_bytes(desc, T, S)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    dbg, dbg_c = _debug_buffers(desc, T, dev, debug, stage_events, SERVING_STAGE_EVENTS)
    d = desc._c()
    wc = slot_weights._c()
    _check(lib.dsmoe_moe_forward_serving(ctypes.byref(d), ctypes.byref(wc), _p(slot_first), _p(slot_expert), S,
                                         _p(bias), _p(x), T, _p(y), _dtype_code(y.dtype), _p(counts),
                                         _p(workspace), workspace.numel(),
                                         ctypes.byref(dbg_c) if dbg_c is not None else None, _stream()),
           "dsmoe_moe_forward_serving")
    return y, counts, dbg


def update_bias(bias: torch.Tensor, counts: torch.Tensor, T: int, K: int, gamma: float = 0.001):
    """In-place aux-loss-free bias update (dsmoe_update_bias)."""
    _dev(bias, torch.float32, "bias")
    _dev(counts, torch.int32, "counts")
    _check(lib.dsmoe_update_bias(_p(bias), _p(counts), bias.numel(), T, K, float(gamma), _stream()),
           "dsmoe_update_bias")
    return bias
