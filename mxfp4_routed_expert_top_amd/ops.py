"""Python binding of libmoe_mxfp4.so (ctypes): argument marshalling only.

Every function has the name of the C entry point it calls (without the
``moe_`` prefix), takes torch tensors that live on the GPU, passes their
device pointers and the current HIP stream, and raises ``MoeError`` on a
non-OK status.  Nothing here computes any step of the layer; there is no
CPU fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_mxfp4.so")
DEBUG_LIB_PATH = os.path.join(PKG, "libmoe_mxfp4_debug.so")   # the MOE_DEBUG build

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_DEVICE = range(5)
ACT_BF16, ACT_MXFP4, ACT_MXFP4_BLOCKED = 0, 1, 2
W_MXFP4, W_MXFP8 = 0, 1            # expert weight formats
SRC_F32, SRC_BF16 = 0, 1
TILE_M = 32

_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGS = {
    "moe_status_string": (ctypes.c_char_p, [_I32]),
    "moe_debug_flags": (ctypes.c_uint32, [_I32]),
    "moe_route_topk": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "moe_mxfp4_forward_router": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                        _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_gemm_workspace_size": (_SZ, [_I32, _I32, _I32, _I32]),
    "moe_route_topk_gemm": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _SZ,
                                   _P]),
    "moe_align_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "moe_align_sort": (_I32, [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_align": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P,
                               _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_quantize": (_I32, [_P, _I32, _I64, _I64, _P, _P, _P]),
    "moe_mxfp4_quantize_blocked": (_I32, [_P, _I32, _I64, _I64, _P, _I32, _I64, _P, _P, _P]),
    "moe_expert_gate_up": (_I32, [_P, _P, _I32, _P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _I32,
                                  _I32, _I32, _P, _P]),
    "moe_expert_gate_up_quant": (_I32, [_P, _P, _I32, _P, _P, _P, _P, _I32, _P, _P, _I32, _I32,
                                        _I32, _I32, _I32, _P, _P, _P]),
    "moe_expert_down": (_I32, [_P, _P, _I32, _P, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _I32,
                               _I32, _P, _P]),
    "moe_combine": (_I32, [_P, _P, _P, _I32, _I32, _I32, _P, _P]),
    "moe_residual_rmsnorm": (_I32, [_P, _I32, _P, _P, ctypes.c_float, _I32, _I32, _P, _P, _P]),
    "moe_gemm_tile_m": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "moe_mxfp4_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "moe_mxfp4_forward": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                 _I32, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_forward_layers": (_I32, [_P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                        _I32, _P, _P, _SZ, _P]),
    "moe_mxfp4_forward_layers_norm": (_I32, [_P, _I32, _P, _P, ctypes.c_float, _P, _I32, _I32,
                                             _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ,
                                             _P]),
    "moe_mxfp8_quantize": (_I32, [_P, _I32, _I64, _I64, _P, _P, _P]),
    "moe_weights_to_native": (_I32, [_P, _I32, _I64, _I64, _P, _P]),
    "moe_mxfp8_expert_gate_up": (_I32, [_P, _P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _I32,
                                        _I32, _P, _P]),
    "moe_mxfp8_expert_down": (_I32, [_P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                     _P, _P]),
    "moe_mxfp8_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "moe_mxfp8_gemm_tile_m": (_I32, [_I32, _I32, _I32, _I32, _I32]),
    "moe_mxfp8_forward": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                 _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_forward_noalloc": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                         _I32, _I32, _P, _P, _P, _P]),
}
EXPORTS = tuple(_SIGS)


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} returned {status_string(status)} ({status})")


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m mxfp4_routed_expert_top_amd.build --all`")
    l = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        f = getattr(l, name)
        f.restype, f.argtypes = res, args
    return l


def lib() -> ctypes.CDLL:
    """Load libmoe_mxfp4.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path: str = DEBUG_LIB_PATH):
    """Inside the block every call of this module goes to another build of
    the library (by default the bound-checking debug build); raises if it
    has not been built."""
    global _lib
    saved = lib()
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = saved


def debug_flags(reset: bool = True) -> int:
    """moe_debug_flags: the debug build's bound-check bits since the last
    reset (0 in the release build)."""
    return int(lib().moe_debug_flags(1 if reset else 0))


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _dt(t, dtype, name):
    if t is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")


# ------------------------------------------------------------------ stages --

def route_topk(logits, gate_logits, K: int, shared: int, renormalize: int = 1,
               topk_ids=None, topk_weights=None, stream=None):
    """moe_route_topk: logits fp32 [T, E], gate fp32 [T] -> (ids int32 [T, K'], w fp32 [T, K'])."""
    _dt(logits, torch.float32, "logits")
    _dt(gate_logits, torch.float32, "gate_logits")
    T, E = logits.shape
    Kp = K + shared
    if topk_ids is None:
        topk_ids = torch.empty(T, Kp, dtype=torch.int32, device=logits.device)
    if topk_weights is None:
        topk_weights = torch.empty(T, Kp, dtype=torch.float32, device=logits.device)
    _check("moe_route_topk", lib().moe_route_topk(
        _ptr(logits), _ptr(gate_logits), T, E, K, shared, renormalize, _ptr(topk_ids),
        _ptr(topk_weights), _stream(stream)))
    return topk_ids, topk_weights


def route_gemm_workspace_size(T: int, H: int, E: int, shared: int) -> int:
    return int(lib().moe_route_gemm_workspace_size(T, H, E, shared))


def route_topk_gemm(x, router_w, K: int, shared: int, renormalize: int = 1, topk_ids=None,
                    topk_weights=None, logits_out=None, workspace=None, stream=None):
    """moe_route_topk_gemm: x bf16 [T, H], router_w bf16 [E + shared, H] (row E = the
    shared expert's gate vector) -> (ids int32 [T, K'], w fp32 [T, K'], logits or None)."""
    _dt(x, torch.bfloat16, "x")
    _dt(router_w, torch.bfloat16, "router_w")
    T, H = x.shape
    E = router_w.shape[0] - shared
    Kp = K + shared
    if topk_ids is None:
        topk_ids = torch.empty(T, Kp, dtype=torch.int32, device=x.device)
    if topk_weights is None:
        topk_weights = torch.empty(T, Kp, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(1, route_gemm_workspace_size(T, H, E, shared)),
                                dtype=torch.uint8, device=x.device)
    _check("moe_route_topk_gemm", lib().moe_route_topk_gemm(
        _ptr(x), _ptr(router_w), T, H, E, K, shared, renormalize, _ptr(topk_ids),
        _ptr(topk_weights), _ptr(logits_out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return topk_ids, topk_weights, logits_out


def align_workspace_size(T: int, Kp: int, Ep: int) -> int:
    return int(lib().moe_align_workspace_size(T, Kp, Ep))


def align_sort(topk_ids, Ep: int, tile_m: int = TILE_M, out=None, stream=None):
    """moe_align_sort -> dict(counts, offsets, sorted, inv, tiles, num_tiles, workspace).
    `out` may hold preallocated tensors of those names (see alloc_align)."""
    _dt(topk_ids, torch.int32, "topk_ids")
    T, Kp = topk_ids.shape
    A = T * Kp
    if out is None:
        out = alloc_align(T, Kp, Ep, topk_ids.device, tile_m)
    if out["tiles"].shape[0] < (A + tile_m - 1) // tile_m + Ep:
        raise ValueError("tile table too small for this tile_m")
    out["tile_m"] = tile_m
    _check("moe_align_sort", lib().moe_align_sort(
        _ptr(topk_ids), T, Kp, Ep, tile_m, _ptr(out["counts"]), _ptr(out["offsets"]),
        _ptr(out["sorted"]) if A else None, _ptr(out["inv"]) if A else None,
        _ptr(out["tiles"]), _ptr(out["num_tiles"]), _ptr(out["workspace"]),
        out["workspace"].numel(), _stream(stream)))
    return out


def route_align(logits, gate_logits, K: int, shared: int, renormalize: int = 1,
                tile_m: int = TILE_M, topk_ids=None, topk_weights=None, out=None, stream=None):
    """moe_route_align: route_topk then align_sort on its ids in one call (one launch
    for a small batch) -> (ids, w, dict as align_sort returns)."""
    _dt(logits, torch.float32, "logits")
    _dt(gate_logits, torch.float32, "gate_logits")
    T, E = logits.shape
    Kp, Ep = K + shared, E + shared
    A = T * Kp
    dev = logits.device
    if topk_ids is None:
        topk_ids = torch.empty(T, Kp, dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty(T, Kp, dtype=torch.float32, device=dev)
    if out is None:
        out = alloc_align(T, Kp, Ep, dev, tile_m)
    if out["tiles"].shape[0] < (A + tile_m - 1) // tile_m + Ep:
        raise ValueError("tile table too small for this tile_m")
    out["tile_m"] = tile_m
    _check("moe_route_align", lib().moe_route_align(
        _ptr(logits), _ptr(gate_logits), T, E, K, shared, renormalize, tile_m, _ptr(topk_ids),
        _ptr(topk_weights), _ptr(out["counts"]), _ptr(out["offsets"]),
        _ptr(out["sorted"]) if A else None, _ptr(out["inv"]) if A else None,
        _ptr(out["tiles"]), _ptr(out["num_tiles"]), _ptr(out["workspace"]),
        out["workspace"].numel(), _stream(stream)))
    return topk_ids, topk_weights, out


def alloc_align(T: int, Kp: int, Ep: int, device, tile_m: int = TILE_M) -> dict:
    A = T * Kp
    i32 = dict(dtype=torch.int32, device=device)
    ws_bytes = align_workspace_size(T, Kp, Ep)
    return dict(counts=torch.empty(Ep, **i32), offsets=torch.empty(Ep + 1, **i32),
                sorted=torch.empty(max(A, 1), **i32)[:A], inv=torch.empty(max(A, 1), **i32)[:A],
                tiles=torch.empty((A + tile_m - 1) // tile_m + Ep, 2, **i32),
                num_tiles=torch.empty(1, **i32),
                workspace=torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=device))


def mxfp4_quantize(src, packed=None, scales=None, stream=None):
    """moe_mxfp4_quantize: fp32 or bf16 [..., cols] -> (packed uint8 [..., cols/2], scales uint8 [..., cols/32])."""
    if src.dtype == torch.float32:
        dt = SRC_F32
    elif src.dtype == torch.bfloat16:
        dt = SRC_BF16
    else:
        raise TypeError("src must be float32 or bfloat16")
    cols = src.shape[-1]
    rows = src.numel() // cols if cols else 0
    lead = src.shape[:-1]
    if packed is None:
        packed = torch.empty(*lead, cols // 2, dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty(*lead, cols // 32, dtype=torch.uint8, device=src.device)
    _check("moe_mxfp4_quantize", lib().moe_mxfp4_quantize(
        _ptr(src), dt, rows, cols, _ptr(packed), _ptr(scales), _stream(stream)))
    return packed, scales


def mxfp4_quantize_blocked(src, row_map=None, Kp: int = 1, out_rows=None, packed=None,
                           scales=None, stream=None):
    """moe_mxfp4_quantize_blocked: fp32 or bf16 [rows, cols] -> (packed uint8
    [R, cols/2], scales uint8 [R, cols/32]) in the blocked row order, R =
    out_rows rounded up to 16; row_map (int32 [rows * Kp], e.g. a grouping's
    inv) sends source row t to output rows row_map[t * Kp + k]."""
    if src.dtype == torch.float32:
        dt = SRC_F32
    elif src.dtype == torch.bfloat16:
        dt = SRC_BF16
    else:
        raise TypeError("src must be float32 or bfloat16")
    rows, cols = src.shape
    if out_rows is None:
        out_rows = rows * Kp if row_map is not None else rows
    r16 = (out_rows + 15) // 16 * 16
    if packed is None:
        packed = torch.empty(r16, cols // 2, dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty(r16, cols // 32, dtype=torch.uint8, device=src.device)
    if row_map is not None:
        _dt(row_map, torch.int32, "row_map")
        if row_map.numel() < rows * Kp:
            raise ValueError("row_map needs rows * Kp entries")
    _check("moe_mxfp4_quantize_blocked", lib().moe_mxfp4_quantize_blocked(
        _ptr(src), dt, rows, cols, _ptr(row_map), Kp, out_rows, _ptr(packed), _ptr(scales),
        _stream(stream)))
    return packed, scales


def mxfp8_quantize(src, codes=None, scales=None, stream=None):
    """moe_mxfp8_quantize: fp32 or bf16 [..., cols] -> (codes uint8 [..., cols], scales uint8 [..., cols/32])."""
    if src.dtype == torch.float32:
        dt = SRC_F32
    elif src.dtype == torch.bfloat16:
        dt = SRC_BF16
    else:
        raise TypeError("src must be float32 or bfloat16")
    cols = src.shape[-1]
    rows = src.numel() // cols if cols else 0
    lead = src.shape[:-1]
    if codes is None:
        codes = torch.empty(*lead, cols, dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty(*lead, cols // 32, dtype=torch.uint8, device=src.device)
    _check("moe_mxfp8_quantize", lib().moe_mxfp8_quantize(
        _ptr(src), dt, rows, cols, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def weights_to_native(codes, wfmt: int = W_MXFP4, out=None, stream=None):
    """moe_weights_to_native: row-major weight codes uint8 [..., rows, row_bytes]
    (one matrix or experts stacked along the leading dims) -> the GEMM kernels'
    native code order, same shape and size."""
    _dt(codes, torch.uint8, "codes")
    if codes.dim() < 2:
        raise ValueError("codes must be [..., rows, row_bytes]")
    row_bytes = codes.shape[-1]
    cols = row_bytes if wfmt == W_MXFP8 else 2 * row_bytes
    rows = codes.numel() // row_bytes if row_bytes else 0
    if out is None:
        out = torch.empty_like(codes)
    _check("moe_weights_to_native", lib().moe_weights_to_native(
        _ptr(codes), wfmt, rows, cols, _ptr(out), _stream(stream)))
    return out


def quantize_weights(w, codes, scales, wfmt: int = W_MXFP4, stream=None):
    """Pack float expert weights [rows, K] for the GEMMs: quantise (MXFP4 or
    MXFP8, row-major), then put the codes into the native order (codes
    [rows, K/2] or [rows, K]; scales [rows, K/32] stay row-major)."""
    quant = mxfp8_quantize if wfmt == W_MXFP8 else mxfp4_quantize
    rm, _ = quant(w, scales=scales, stream=stream)
    weights_to_native(rm, wfmt, out=codes, stream=stream)
    return codes, scales


def gemm_tile_m(T: int, Kp: int, Ep: int, H: int, I: int, act_fmt: int = ACT_BF16) -> int:
    """moe_gemm_tile_m: the GEMM tile rows mxfp4_forward uses for these shapes."""
    return int(lib().moe_gemm_tile_m(T, Kp, Ep, H, I, act_fmt))


def expert_gate_up(act, act_scale, act_fmt: int, align: dict, w13, w13_scale, T: int, H: int,
                   I: int, Ep: int, Kp: int, h=None, stream=None):
    """moe_expert_gate_up -> h bf16 [T*Kp, I] in sorted row order (align["tile_m"]-row tiles)."""
    if h is None:
        h = torch.empty(T * Kp, I, dtype=torch.bfloat16, device=w13.device)
    _check("moe_expert_gate_up", lib().moe_expert_gate_up(
        _ptr(act), _ptr(act_scale), act_fmt, _ptr(align["sorted"]), _ptr(align["offsets"]),
        _ptr(align["tiles"]), _ptr(align["num_tiles"]), align["tile_m"], _ptr(w13),
        _ptr(w13_scale), T, H, I, Ep, Kp, _ptr(h), _stream(stream)))
    return h


def expert_gate_up_quant(act, act_scale, align: dict, w13, w13_scale, T: int, H: int, I: int,
                         Ep: int, Kp: int, h_packed=None, h_scale=None, stream=None,
                         act_fmt: int = ACT_MXFP4_BLOCKED):
    """moe_expert_gate_up_quant (MXFP4 activations, blocked or per token) ->
    (h_packed uint8 [R, I/2], h_scale uint8 [R, I/32]) in the blocked row
    order, R = T*Kp rounded up to 16."""
    r16 = (T * Kp + 15) // 16 * 16
    if h_packed is None:
        h_packed = torch.empty(r16, I // 2, dtype=torch.uint8, device=w13.device)
    if h_scale is None:
        h_scale = torch.empty(r16, I // 32, dtype=torch.uint8, device=w13.device)
    _dt(h_packed, torch.uint8, "h_packed")
    _dt(h_scale, torch.uint8, "h_scale")
    _check("moe_expert_gate_up_quant", lib().moe_expert_gate_up_quant(
        _ptr(act), _ptr(act_scale), act_fmt, _ptr(align["sorted"]), _ptr(align["offsets"]),
        _ptr(align["tiles"]), _ptr(align["num_tiles"]), align["tile_m"], _ptr(w13),
        _ptr(w13_scale), T, H, I, Ep, Kp, _ptr(h_packed), _ptr(h_scale), _stream(stream)))
    return h_packed, h_scale


def expert_down(h, h_scale, act_fmt: int, align: dict, w2, w2_scale, T: int, H: int, I: int,
                Ep: int, Kp: int, y=None, stream=None):
    """moe_expert_down -> staged y (uint8 [staged_y_bytes(T*Kp, H)]), rows in sorted order."""
    if y is None:
        y = torch.empty(staged_y_bytes(T * Kp, H), dtype=torch.uint8, device=w2.device)
    _dt(y, torch.uint8, "y")
    _check("moe_expert_down", lib().moe_expert_down(
        _ptr(h), _ptr(h_scale), act_fmt, _ptr(align["offsets"]), _ptr(align["tiles"]),
        _ptr(align["num_tiles"]), align["tile_m"], _ptr(w2), _ptr(w2_scale), T, H, I, Ep, Kp,
        _ptr(y), _stream(stream)))
    return y


def mxfp8_gemm_tile_m(T: int, Kp: int, Ep: int, H: int, I: int) -> int:
    """moe_mxfp8_gemm_tile_m: the GEMM tile rows mxfp8_forward uses for these shapes."""
    return int(lib().moe_mxfp8_gemm_tile_m(T, Kp, Ep, H, I))


def mxfp8_expert_gate_up(x, align: dict, w13, w13_scale, T: int, H: int, I: int, Ep: int,
                         Kp: int, h=None, stream=None):
    """moe_mxfp8_expert_gate_up (MXFP8 weights, bf16 x) -> h bf16 [T*Kp, I], sorted rows."""
    _dt(x, torch.bfloat16, "x")
    if h is None:
        h = torch.empty(T * Kp, I, dtype=torch.bfloat16, device=w13.device)
    _check("moe_mxfp8_expert_gate_up", lib().moe_mxfp8_expert_gate_up(
        _ptr(x), _ptr(align["sorted"]), _ptr(align["offsets"]), _ptr(align["tiles"]),
        _ptr(align["num_tiles"]), align["tile_m"], _ptr(w13), _ptr(w13_scale), T, H, I, Ep, Kp,
        _ptr(h), _stream(stream)))
    return h


def mxfp8_expert_down(h, align: dict, w2, w2_scale, T: int, H: int, I: int, Ep: int, Kp: int,
                      y=None, stream=None):
    """moe_mxfp8_expert_down (MXFP8 weights, bf16 h) -> staged y, sorted rows."""
    _dt(h, torch.bfloat16, "h")
    if y is None:
        y = torch.empty(staged_y_bytes(T * Kp, H), dtype=torch.uint8, device=w2.device)
    _dt(y, torch.uint8, "y")
    _check("moe_mxfp8_expert_down", lib().moe_mxfp8_expert_down(
        _ptr(h), _ptr(align["offsets"]), _ptr(align["tiles"]), _ptr(align["num_tiles"]),
        align["tile_m"], _ptr(w2), _ptr(w2_scale), T, H, I, Ep, Kp, _ptr(y), _stream(stream)))
    return y


def combine(y, topk_weights, inv, T: int, H: int, Kp: int, out=None, stream=None):
    """moe_combine: staged y of T*Kp rows -> out bf16 [T, H]."""
    _dt(y, torch.uint8, "y")
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=y.device)
    _check("moe_combine", lib().moe_combine(
        _ptr(y), _ptr(topk_weights), _ptr(inv), T, H, Kp, _ptr(out), _stream(stream)))
    return out


NORM_MAX_RANKS = 8


def residual_rmsnorm(partials, gamma, eps: float, residual=None, residual_out=None, out=None,
                     stream=None):
    """moe_residual_rmsnorm: the G partial outputs (a list of bf16 [T, H]
    tensors) summed, residual added, RMSNorm with gamma (bf16 [H]).  Returns
    (out, residual_out); residual_out may be the residual tensor itself
    (updated in place) or None (not written)."""
    G = len(partials)
    T, H = partials[0].shape
    for p in partials:
        _dt(p, torch.bfloat16, "partials")
        if tuple(p.shape) != (T, H):
            raise ValueError("partials: every one of shape [T, H]")
    _dt(gamma, torch.bfloat16, "gamma")
    _dt(residual, torch.bfloat16, "residual")
    _dt(residual_out, torch.bfloat16, "residual_out")
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=partials[0].device)
    ptrs = (ctypes.c_void_p * G)(*[_ptr(p) for p in partials])
    _check("moe_residual_rmsnorm", lib().moe_residual_rmsnorm(
        ptrs, G, _ptr(residual), _ptr(gamma), float(eps), T, H, _ptr(residual_out), _ptr(out),
        _stream(stream)))
    return out, residual_out


# ------------------------------------------------------------ whole layer --

def staged_y_bytes(A: int, H: int) -> int:
    """Bytes of the staged y between moe_expert_down and moe_combine
    (MOE_STAGED_Y_BYTES): fp16 [A, H] and one exponent byte per 32 columns."""
    return A * H * 2 + A * (H // 32)


def workspace_size(T, H, I, E, K, shared, act_fmt) -> int:
    return int(lib().moe_mxfp4_workspace_size(T, H, I, E, K, shared, act_fmt))


def mxfp4_forward(x, router_logits, shared_gate_logits, w13, w13_scale, w2, w2_scale, I: int,
                  E: int, K: int, shared: int, act_fmt: int = ACT_BF16, out=None, topk_ids=None,
                  topk_weights=None, workspace=None, stream=None):
    """moe_mxfp4_forward: the whole layer.  x bf16 [T, H] -> out bf16 [T, H]."""
    _dt(x, torch.bfloat16, "x")
    _dt(router_logits, torch.float32, "router_logits")
    T, H = x.shape
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    need = workspace_size(T, H, I, E, K, shared, act_fmt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check("moe_mxfp4_forward", lib().moe_mxfp4_forward(
        _ptr(x), _ptr(router_logits), _ptr(shared_gate_logits), _ptr(w13), _ptr(w13_scale),
        _ptr(w2), _ptr(w2_scale), T, H, I, E, K, shared, act_fmt, _ptr(out), _ptr(topk_ids),
        _ptr(topk_weights), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def mxfp4_forward_noalloc(x, router_logits, shared_gate_logits, w13, w13_scale, w2, w2_scale,
                          I: int, E: int, K: int, shared: int, act_fmt: int = ACT_BF16, out=None,
                          topk_ids=None, topk_weights=None, stream=None):
    """moe_mxfp4_forward_noalloc: the whole layer with the library's own
    device scratch instead of a workspace.  x bf16 [T, H] -> out bf16 [T, H]."""
    _dt(x, torch.bfloat16, "x")
    _dt(router_logits, torch.float32, "router_logits")
    T, H = x.shape
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    _check("moe_mxfp4_forward_noalloc", lib().moe_mxfp4_forward_noalloc(
        _ptr(x), _ptr(router_logits), _ptr(shared_gate_logits), _ptr(w13), _ptr(w13_scale),
        _ptr(w2), _ptr(w2_scale), T, H, I, E, K, shared, act_fmt, _ptr(out), _ptr(topk_ids),
        _ptr(topk_weights), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20      # MOE_NOALLOC_SCRATCH_BYTES


def mxfp4_forward_router(x, router_w, w13, w13_scale, w2, w2_scale, I: int, E: int, K: int,
                         shared: int, act_fmt: int = ACT_BF16, out=None, topk_ids=None,
                         topk_weights=None, logits_out=None, workspace=None, stream=None):
    """moe_mxfp4_forward_router: the whole layer routed from x through the router
    GEMM (router_w bf16 [E + shared, H]).  x bf16 [T, H] -> out bf16 [T, H]."""
    _dt(x, torch.bfloat16, "x")
    _dt(router_w, torch.bfloat16, "router_w")
    T, H = x.shape
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    need = workspace_size(T, H, I, E, K, shared, act_fmt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check("moe_mxfp4_forward_router", lib().moe_mxfp4_forward_router(
        _ptr(x), _ptr(router_w), _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), T, H, I,
        E, K, shared, act_fmt, _ptr(out), _ptr(topk_ids), _ptr(topk_weights), _ptr(logits_out),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def mxfp8_workspace_size(T, H, I, E, K, shared) -> int:
    return int(lib().moe_mxfp8_workspace_size(T, H, I, E, K, shared))


def mxfp8_forward(x, router_logits, shared_gate_logits, w13, w13_scale, w2, w2_scale, I: int,
                  E: int, K: int, shared: int, out=None, topk_ids=None, topk_weights=None,
                  workspace=None, stream=None):
    """moe_mxfp8_forward: the whole layer over MXFP8 weights, bf16 activations."""
    _dt(x, torch.bfloat16, "x")
    _dt(router_logits, torch.float32, "router_logits")
    T, H = x.shape
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    need = mxfp8_workspace_size(T, H, I, E, K, shared)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check("moe_mxfp8_forward", lib().moe_mxfp8_forward(
        _ptr(x), _ptr(router_logits), _ptr(shared_gate_logits), _ptr(w13), _ptr(w13_scale),
        _ptr(w2), _ptr(w2_scale), T, H, I, E, K, shared, _ptr(out), _ptr(topk_ids),
        _ptr(topk_weights), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


class _Layer(ctypes.Structure):
    """moe_mxfp4_layer: one layer's router rows and MXFP4 expert weights."""
    _fields_ = [("router_w", _P), ("w13", _P), ("w13_scale", _P), ("w2", _P), ("w2_scale", _P)]


def mxfp4_forward_layers(x, layers, I: int, E: int, K: int, shared: int,
                         act_fmt: int = ACT_BF16, prefetch: int = 0, out=None, workspace=None,
                         stream=None):
    """moe_mxfp4_forward_layers: len(layers) layers back to back, each a
    (router_w, w13, w13_scale, w2, w2_scale) tuple of device tensors; layer 0
    reads x, each later layer the previous layer's output.  -> out bf16 [T, H]."""
    _dt(x, torch.bfloat16, "x")
    T, H = x.shape
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    need = workspace_size(T, H, I, E, K, shared, act_fmt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    arr = (_Layer * max(len(layers), 1))()
    for i, (wr, w13, w13s, w2, w2s) in enumerate(layers):
        _dt(wr, torch.bfloat16, "router_w")
        arr[i] = _Layer(_ptr(wr), _ptr(w13), _ptr(w13s), _ptr(w2), _ptr(w2s))
    _check("moe_mxfp4_forward_layers", lib().moe_mxfp4_forward_layers(
        _ptr(x), len(layers), ctypes.cast(arr, _P), T, H, I, E, K, shared, act_fmt, prefetch,
        _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def mxfp4_forward_layers_norm(x, layers, gammas, eps: float, residual, I: int, E: int, K: int,
                              shared: int, act_fmt: int = ACT_BF16, prefetch: int = 0, out=None,
                              workspace=None, stream=None):
    """moe_mxfp4_forward_layers_norm: the layers of mxfp4_forward_layers with
    residual += layer output and out = RMSNorm(residual) * gammas[l] after
    each (residual, bf16 [T, H], updated in place).  -> out bf16 [T, H]."""
    _dt(x, torch.bfloat16, "x")
    _dt(residual, torch.bfloat16, "residual")
    T, H = x.shape
    if len(gammas) != len(layers):
        raise ValueError("one gamma per layer")
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    need = workspace_size(T, H, I, E, K, shared, act_fmt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    arr = (_Layer * max(len(layers), 1))()
    for i, (wr, w13, w13s, w2, w2s) in enumerate(layers):
        _dt(wr, torch.bfloat16, "router_w")
        arr[i] = _Layer(_ptr(wr), _ptr(w13), _ptr(w13s), _ptr(w2), _ptr(w2s))
    for g in gammas:
        _dt(g, torch.bfloat16, "gammas")
    garr = (ctypes.c_void_p * max(len(gammas), 1))(*[_ptr(g) for g in gammas])
    _check("moe_mxfp4_forward_layers_norm", lib().moe_mxfp4_forward_layers_norm(
        _ptr(x), len(layers), ctypes.cast(arr, _P), garr, float(eps), _ptr(residual), T, H, I, E,
        K, shared, act_fmt, prefetch, _ptr(out), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return out


def alloc_stages(T: int, H: int, I: int, E: int, K: int, shared: int, act_fmt: int,
                 device) -> dict:
    """Preallocated outputs of every stage of one pass (for forward_stages)."""
    Kp, Ep, A = K + shared, E + shared, T * (K + shared)
    b = dict(ids=torch.empty(T, Kp, dtype=torch.int32, device=device),
             w=torch.empty(T, Kp, dtype=torch.float32, device=device),
             align=alloc_align(T, Kp, Ep, device),
             h=torch.empty(A, I, dtype=torch.bfloat16, device=device),
             y=torch.empty(staged_y_bytes(A, H), dtype=torch.uint8, device=device),
             out=torch.empty(T, H, dtype=torch.bfloat16, device=device))
    if act_fmt == ACT_MXFP4:
        # per token / sorted row, or sorted rows in the blocked order (tiled GEMMs)
        u8 = dict(dtype=torch.uint8, device=device)
        A16 = (A + 15) // 16 * 16
        b.update(xq=torch.empty(A16, H // 2, **u8), xs=torch.empty(A16, H // 32, **u8),
                 hq=torch.empty(A16, I // 2, **u8), hs=torch.empty(A16, I // 32, **u8))
    return b


def forward_stages(x, router_logits, shared_gate_logits, w13, w13_scale, w2, w2_scale, I: int,
                   E: int, K: int, shared: int, act_fmt: int = ACT_BF16, bufs=None, stream=None,
                   events=None, wfmt: int = W_MXFP4, fuse_h_quant: bool = False):
    """The same pass as mxfp4_forward (mxfp8_forward for wfmt = W_MXFP8), one
    C entry point per stage, keeping every intermediate (in `bufs` if given,
    see alloc_stages).  `events`, if given, maps a stage name (route, align,
    quant_x, gate_up, quant_h, down, combine) to a (start, end) pair of
    torch.cuda.Event recorded around it.  W4A4 on the tiled kernels writes
    the bf16 h and quantises it as a stage of its own, unless fuse_h_quant
    (the forward's own path: moe_expert_gate_up_quant, no bf16 h)."""
    if wfmt == W_MXFP8 and act_fmt != ACT_BF16:
        raise ValueError("MXFP8 weights take bf16 activations")
    T, H = x.shape
    Kp, Ep = K + shared, E + shared
    b = alloc_stages(T, H, I, E, K, shared, act_fmt, x.device) if bufs is None else bufs
    st = torch.cuda.current_stream() if stream is None else stream

    def rec(name, i):
        if events and name in events:
            events[name][i].record(st)

    rec("route", 0)
    route_topk(router_logits, shared_gate_logits, K, shared, topk_ids=b["ids"],
               topk_weights=b["w"], stream=stream)
    rec("route", 1)
    rec("align", 0)
    tm = (mxfp8_gemm_tile_m(T, Kp, Ep, H, I) if wfmt == W_MXFP8 else
          gemm_tile_m(T, Kp, Ep, H, I, act_fmt))
    align_sort(b["ids"], Ep, tile_m=tm, out=b["align"], stream=stream)
    rec("align", 1)
    act, act_s, gemm_act = x, None, act_fmt
    blk = act_fmt == ACT_MXFP4 and tm != TILE_M      # tiled GEMMs: blocked sorted rows
    if act_fmt == ACT_MXFP4:
        rec("quant_x", 0)
        if blk:
            mxfp4_quantize_blocked(x, b["align"]["inv"], Kp, T * Kp, b["xq"], b["xs"],
                                   stream=stream)
            gemm_act = ACT_MXFP4_BLOCKED
        else:
            mxfp4_quantize(x, b["xq"][:T], b["xs"][:T], stream=stream)
        rec("quant_x", 1)
        act, act_s = b["xq"], b["xs"]
    fused = blk and fuse_h_quant
    rec("gate_up", 0)
    if wfmt == W_MXFP8:
        mxfp8_expert_gate_up(x, b["align"], w13, w13_scale, T, H, I, Ep, Kp, h=b["h"], stream=stream)
    elif fused:
        expert_gate_up_quant(act, act_s, b["align"], w13, w13_scale, T, H, I, Ep, Kp,
                             h_packed=b["hq"], h_scale=b["hs"], stream=stream)
    else:
        expert_gate_up(act, act_s, gemm_act, b["align"], w13, w13_scale, T, H, I, Ep, Kp, h=b["h"],
                       stream=stream)
    rec("gate_up", 1)
    hin, hin_s = b["h"], None
    if fused:
        hin, hin_s = b["hq"], b["hs"]
    elif act_fmt == ACT_MXFP4:
        rec("quant_h", 0)
        if blk:
            mxfp4_quantize_blocked(b["h"], packed=b["hq"], scales=b["hs"], stream=stream)
        else:
            mxfp4_quantize(b["h"], b["hq"][:T * Kp], b["hs"][:T * Kp], stream=stream)
        rec("quant_h", 1)
        hin, hin_s = b["hq"], b["hs"]
    rec("down", 0)
    if wfmt == W_MXFP8:
        mxfp8_expert_down(hin, b["align"], w2, w2_scale, T, H, I, Ep, Kp, y=b["y"], stream=stream)
    else:
        expert_down(hin, hin_s, gemm_act, b["align"], w2, w2_scale, T, H, I, Ep, Kp, y=b["y"],
                    stream=stream)
    rec("down", 1)
    rec("combine", 0)
    combine(b["y"], b["w"], b["align"]["inv"], T, H, Kp, out=b["out"], stream=stream)
    rec("combine", 1)
    return b
