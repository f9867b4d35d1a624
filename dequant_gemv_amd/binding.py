"""ctypes binding of ``libdqg.so`` (the C ABI in ``include/dqg.h``).

Argument marshalling only: every function checks dtypes, devices, shapes and contiguity,
passes ``data_ptr()`` values and the current torch stream to the C entry point of the
same name and raises on a non-zero status.  All arithmetic runs in the HIP kernels.
PyTorch serves as the device allocator and stream provider; outputs and workspaces are
allocated with torch when the caller does not pass them.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DQG_LIBRARY names another build of the same library (the host-sanitizer build that the
# CPU tests load); the in-tree libdqg.so otherwise
LIB_PATH = os.environ.get("DQG_LIBRARY") or os.path.join(_HERE, "libdqg.so")

DQG_OK = 0
DQG_ERR_INVALID_ARG = -1
DQG_ERR_UNSUPPORTED = -2
DQG_ERR_MISALIGNED = -3
DQG_ERR_WORKSPACE = -4
DQG_ERR_HIP = -5
FMT_INT4 = 0
FMT_FP4_E2M1 = 1
FMT_FP8_E4M3 = 2
FMT_INT2 = 3
FMT_FEXC = 4
PATH_FORCE_GEMV = 0x100
PATH_FORCE_MFMA = 0x200
PATH_NO_FUSED = 0x400

# (name, restype, argtypes) for every symbol the header declares
_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t
SIGNATURES = {
    "dqg_abi_version": (_I, []),
    "dqg_status_string": (ctypes.c_char_p, [_I]),
    "topk_route": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_fp4_ffn_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "moe_fp4_ffn": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _Z,
                         _P]),
    "moe_fp4_layer": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P,
                           _Z, _P]),
    "router_logits_workspace_bytes": (_Z, [_I, _I, _I]),
    "router_logits": (_I, [_P, _I, _I, _I, _P, _P, _P, _Z, _P]),
    "moe_fp4_layer_from_hidden": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _I, _P, _P,
                                       _P, _P, _P, _P, _Z, _P]),
    "moe_fp4_layer_mixed": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _I, _P,
                                 _P, _P, _P, _P, _Z, _P]),
    "packed_gemv_int4_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "packed_gemv_int4": (_I, [_P, _I, _I, _I, _P, _P, _I, _P, _P, _Z, _P]),
    "packed_gemv_int4_noalloc": (_I, [_P, _I, _I, _I, _P, _P, _I, _P, _P, _P]),
    "packed_gemv_int4_prepack_sizes": (_I, [_I, _I, _I, ctypes.POINTER(_Z), ctypes.POINTER(_Z)]),
    "packed_gemv_int4_prepack": (_I, [_P, _P, _I, _I, _I, _P, _P, _P]),
    "packed_gemv_int4_tiled": (_I, [_P, _I, _I, _I, _P, _P, _I, _P, _P, _Z, _P]),
    "packed_dequant_f32": (_I, [_P, _P, _I, _I, _I, _I, _P, _P]),
    "dqg_stream_read": (_I, [_P, _Z, _P, _P]),
}


class DqgError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m dequant_gemv_amd.build`"
                          " (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


LIB = _load()


def status_string(status: int) -> str:
    return LIB.dqg_status_string(int(status)).decode()


def abi_version() -> int:
    return int(LIB.dqg_abi_version())


def _check(fn: str, status: int):
    if status != DQG_OK:
        raise DqgError(fn, status)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, name: str, itemsize: int, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.element_size() != itemsize:
        raise TypeError(f"{name} must have {itemsize}-byte elements, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


# ---------------------------------------------------------------------------------------
def topk_route(logits: torch.Tensor, k: int, ids: Optional[torch.Tensor] = None,
               weights: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    T, E = logits.shape
    _need(logits, "logits", 4)
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _need(ids, "ids", 4, (T, k), logits.device)
    _need(weights, "weights", 4, (T, k), logits.device)
    _check("topk_route", LIB.topk_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(weights),
                                        _stream(logits)))
    return ids, weights


def moe_fp4_ffn_workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(LIB.moe_fp4_ffn_workspace_bytes(T, H, I, E, k))


def moe_workspace(T: int, H: int, I: int, E: int, k: int, device) -> torch.Tensor:
    n = moe_fp4_ffn_workspace_bytes(T, H, I, E, k)
    if n == 0:
        raise ValueError("unsupported MoE sizes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _moe_shapes(x, w_gate_up, s_gate_up, w_down, s_down, group, fmt):
    T, H = x.shape
    E, hp, two_i = w_gate_up.shape
    I = two_i // 2
    b = 1 if fmt == FMT_FP8_E4M3 else 2   # K indices per stored byte
    if hp * b != H:
        raise ValueError(f"w_gate_up must be [E, H/{b}, 2I]" if b > 1 else "w_gate_up must be [E, H, 2I]")
    _need(x, "x", 2)
    _need(w_gate_up, "w_gate_up", 1, (E, H // b, 2 * I), x.device)
    _need(s_gate_up, "s_gate_up", 2, (E, H // group, 2 * I), x.device)
    _need(w_down, "w_down", 1, (E, I // b, H), x.device)
    _need(s_down, "s_down", 2, (E, I // group, H), x.device)
    return T, H, I, E


def moe_fp4_ffn(x, ids, weights, w_gate_up, s_gate_up, w_down, s_down, group: int, fmt: int,
                residual=None, out=None, workspace=None, flags: int = 0) -> torch.Tensor:
    T, H, I, E = _moe_shapes(x, w_gate_up, s_gate_up, w_down, s_down, group, fmt)
    k = ids.shape[1]
    _need(ids, "ids", 4, (T, k), x.device)
    _need(weights, "weights", 4, (T, k), x.device)
    if residual is not None:
        _need(residual, "residual", 2, (T, H), x.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", 2, (T, H), x.device)
    if workspace is None:
        workspace = moe_workspace(T, H, I, E, k, x.device)
    _need(workspace, "workspace", 1, None, x.device)
    _check("moe_fp4_ffn", LIB.moe_fp4_ffn(
        _ptr(x), T, H, I, E, k, _ptr(ids), _ptr(weights), _ptr(w_gate_up), _ptr(s_gate_up),
        _ptr(w_down), _ptr(s_down), group, fmt | flags, _ptr(residual), _ptr(out),
        _ptr(workspace), workspace.numel(), _stream(x)))
    return out


def moe_fp4_layer(x, logits, k: int, w_gate_up, s_gate_up, w_down, s_down, group: int, fmt: int,
                  residual=None, out=None, ids_out=None, weights_out=None, workspace=None,
                  flags: int = 0) -> torch.Tensor:
    T, H, I, E = _moe_shapes(x, w_gate_up, s_gate_up, w_down, s_down, group, fmt)
    _need(logits, "logits", 4, (T, E), x.device)
    if residual is not None:
        _need(residual, "residual", 2, (T, H), x.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", 2, (T, H), x.device)
    if ids_out is not None:
        _need(ids_out, "ids_out", 4, (T, k), x.device)
    if weights_out is not None:
        _need(weights_out, "weights_out", 4, (T, k), x.device)
    if workspace is None:
        workspace = moe_workspace(T, H, I, E, k, x.device)
    _need(workspace, "workspace", 1, None, x.device)
    _check("moe_fp4_layer", LIB.moe_fp4_layer(
        _ptr(x), _ptr(logits), T, H, I, E, k, _ptr(w_gate_up), _ptr(s_gate_up), _ptr(w_down),
        _ptr(s_down), group, fmt | flags, _ptr(residual), _ptr(out), _ptr(ids_out),
        _ptr(weights_out), _ptr(workspace), workspace.numel(), _stream(x)))
    return out


def router_logits_workspace_bytes(T: int, H: int, E: int) -> int:
    return int(LIB.router_logits_workspace_bytes(T, H, E))


def router_logits_workspace(T: int, H: int, E: int, device) -> torch.Tensor:
    n = router_logits_workspace_bytes(T, H, E)
    if n == 0:
        raise ValueError("unsupported router sizes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def router_logits(x, w_router, logits=None, workspace=None) -> torch.Tensor:
    T, H = x.shape
    E = w_router.shape[1]
    _need(x, "x", 2)
    _need(w_router, "w_router", 2, (H, E), x.device)
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _need(logits, "logits", 4, (T, E), x.device)
    if workspace is None:
        workspace = router_logits_workspace(T, H, E, x.device)
    _need(workspace, "workspace", 1, None, x.device)
    _check("router_logits", LIB.router_logits(
        _ptr(x), T, H, E, _ptr(w_router), _ptr(logits), _ptr(workspace), workspace.numel(),
        _stream(x)))
    return logits


def moe_fp4_layer_from_hidden(x, w_router, k: int, w_gate_up, s_gate_up, w_down, s_down,
                              group: int, fmt: int, residual=None, out=None, logits_out=None,
                              ids_out=None, weights_out=None, workspace=None,
                              flags: int = 0) -> torch.Tensor:
    T, H, I, E = _moe_shapes(x, w_gate_up, s_gate_up, w_down, s_down, group, fmt)
    _need(w_router, "w_router", 2, (H, E), x.device)
    if residual is not None:
        _need(residual, "residual", 2, (T, H), x.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", 2, (T, H), x.device)
    if logits_out is not None:
        _need(logits_out, "logits_out", 4, (T, E), x.device)
    if ids_out is not None:
        _need(ids_out, "ids_out", 4, (T, k), x.device)
    if weights_out is not None:
        _need(weights_out, "weights_out", 4, (T, k), x.device)
    if workspace is None:
        workspace = moe_workspace(T, H, I, E, k, x.device)
    _need(workspace, "workspace", 1, None, x.device)
    _check("moe_fp4_layer_from_hidden", LIB.moe_fp4_layer_from_hidden(
        _ptr(x), _ptr(w_router), T, H, I, E, k, _ptr(w_gate_up), _ptr(s_gate_up), _ptr(w_down),
        _ptr(s_down), group, fmt | flags, _ptr(residual), _ptr(out), _ptr(logits_out),
        _ptr(ids_out), _ptr(weights_out), _ptr(workspace), workspace.numel(), _stream(x)))
    return out


def moe_fp4_layer_mixed(x, logits, k: int, w_gate_up, s_gate_up, w_down, s_down,
                        expert_formats, group: int, codebooks=None, residual=None, out=None,
                        ids_out=None, weights_out=None, workspace=None,
                        flags: int = 0) -> torch.Tensor:
    """FP4 layer whose experts marked FMT_INT2 / FMT_FEXC in expert_formats (uint8 [E]) hold
    INT2 or FE-XC codes in the first quarter of their slab (codebooks bf16 [E, 2, 2, 256, 8])."""
    T, H, I, E = _moe_shapes(x, w_gate_up, s_gate_up, w_down, s_down, group, FMT_FP4_E2M1)
    _need(logits, "logits", 4, (T, E), x.device)
    _need(expert_formats, "expert_formats", 1, (E,), x.device)
    if codebooks is not None:
        _need(codebooks, "codebooks", 2, (E, 2, 2, 256, 8), x.device)
    if residual is not None:
        _need(residual, "residual", 2, (T, H), x.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", 2, (T, H), x.device)
    if ids_out is not None:
        _need(ids_out, "ids_out", 4, (T, k), x.device)
    if weights_out is not None:
        _need(weights_out, "weights_out", 4, (T, k), x.device)
    if workspace is None:
        workspace = moe_workspace(T, H, I, E, k, x.device)
    _need(workspace, "workspace", 1, None, x.device)
    _check("moe_fp4_layer_mixed", LIB.moe_fp4_layer_mixed(
        _ptr(x), _ptr(logits), T, H, I, E, k, _ptr(w_gate_up), _ptr(s_gate_up), _ptr(w_down),
        _ptr(s_down), _ptr(expert_formats), _ptr(codebooks), group, FMT_FP4_E2M1 | flags,
        _ptr(residual),
        _ptr(out), _ptr(ids_out), _ptr(weights_out), _ptr(workspace), workspace.numel(),
        _stream(x)))
    return out


def packed_gemv_int4_workspace_bytes(T: int, K: int, N: int, group: int) -> int:
    return int(LIB.packed_gemv_int4_workspace_bytes(T, K, N, group))


def gemv_workspace(T: int, K: int, N: int, group: int, device) -> Optional[torch.Tensor]:
    n = packed_gemv_int4_workspace_bytes(T, K, N, group)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def packed_gemv_int4(x, w, s, group: int, y=None, workspace=None) -> torch.Tensor:
    T, K = x.shape
    N = w.shape[1]
    _need(x, "x", 2)
    _need(w, "w", 1, (K // 2, N), x.device)
    _need(s, "s", 2, (K // group, N), x.device)
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", 2, (T, N), x.device)
    if workspace is not None:
        _need(workspace, "workspace", 1, None, x.device)
    _check("packed_gemv_int4", LIB.packed_gemv_int4(
        _ptr(x), T, K, N, _ptr(w), _ptr(s), group, _ptr(y), _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(x)))
    return y


def packed_gemv_int4_noalloc(x, w, s, group: int, y=None, status=None) -> torch.Tensor:
    """The allocation-free GEMV entry point: split partials in the library's device array.
    ``y`` (bf16 [T, N]) and ``status`` (int32, one element) are optional device tensors; when
    ``y`` is None it is allocated here with torch (the C call itself allocates nothing)."""
    T, K = x.shape
    N = w.shape[1]
    _need(x, "x", 2)
    _need(w, "w", 1, (K // 2, N), x.device)
    _need(s, "s", 2, (K // group, N), x.device)
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", 2, (T, N), x.device)
    if status is not None:
        _need(status, "status", 4, (1,), x.device)
    _check("packed_gemv_int4_noalloc", LIB.packed_gemv_int4_noalloc(
        _ptr(x), T, K, N, _ptr(w), _ptr(s), group, _ptr(y), _ptr(status), _stream(x)))
    return y


def packed_gemv_int4_prepack_sizes(K: int, N: int, group: int):
    wb, sb = _Z(0), _Z(0)
    _check("packed_gemv_int4_prepack_sizes",
           LIB.packed_gemv_int4_prepack_sizes(K, N, group, ctypes.byref(wb), ctypes.byref(sb)))
    return int(wb.value), int(sb.value)


def packed_gemv_int4_prepack(w, s, group: int, w_tiled=None, s_tiled=None):
    """Prepacked copies (flat uint8 weights, flat bf16 scales) of an INT4 matrix w [K/2, N]
    and its scales s [K/G, N]; returns (w_tiled, s_tiled)."""
    Kp, N = w.shape
    K = 2 * Kp
    _need(w, "w", 1)
    _need(s, "s", 2, (K // group, N), w.device)
    wb, sb = packed_gemv_int4_prepack_sizes(K, N, group)
    if w_tiled is None:
        w_tiled = torch.empty(wb, dtype=torch.uint8, device=w.device)
    if s_tiled is None:
        s_tiled = torch.empty(sb // 2, dtype=torch.bfloat16, device=w.device)
    _need(w_tiled, "w_tiled", 1, (wb,), w.device)
    _need(s_tiled, "s_tiled", 2, (sb // 2,), w.device)
    _check("packed_gemv_int4_prepack", LIB.packed_gemv_int4_prepack(
        _ptr(w), _ptr(s), K, N, group, _ptr(w_tiled), _ptr(s_tiled), _stream(w)))
    return w_tiled, s_tiled


def packed_gemv_int4_tiled(x, w_tiled, s_tiled, N: int, group: int, y=None,
                           workspace=None) -> torch.Tensor:
    """The GEMV of packed_gemv_int4 on prepacked weights (packed_gemv_int4_prepack); T <= 4.
    ``workspace``: as for packed_gemv_int4 (``gemv_workspace(T, K, N, group, device)``)."""
    T, K = x.shape
    _need(x, "x", 2)
    wb, sb = packed_gemv_int4_prepack_sizes(K, N, group)
    _need(w_tiled, "w_tiled", 1, (wb,), x.device)
    _need(s_tiled, "s_tiled", 2, (sb // 2,), x.device)
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", 2, (T, N), x.device)
    if workspace is not None:
        _need(workspace, "workspace", 1, None, x.device)
    _check("packed_gemv_int4_tiled", LIB.packed_gemv_int4_tiled(
        _ptr(x), T, K, N, _ptr(w_tiled), _ptr(s_tiled), group, _ptr(y), _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(x)))
    return y


def packed_dequant_f32(w, s, group: int, fmt: int, out=None) -> torch.Tensor:
    Kp, N = w.shape
    K = Kp if fmt == FMT_FP8_E4M3 else 2 * Kp
    _need(w, "w", 1)
    _need(s, "s", 2, (K // group, N), w.device)
    if out is None:
        out = torch.empty((K, N), dtype=torch.float32, device=w.device)
    _need(out, "out", 4, (K, N), w.device)
    _check("packed_dequant_f32", LIB.packed_dequant_f32(
        _ptr(w), _ptr(s), K, N, group, fmt, _ptr(out), _stream(w)))
    return out


def stream_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Measurement aid: one streaming read of ``buf`` (uint8, contiguous, size a multiple of
    16) on the current stream; ``sink`` is a one-element int32 device tensor."""
    _need(buf, "buf", 1)
    _need(sink, "sink", 4, (1,), buf.device)
    _check("dqg_stream_read", LIB.dqg_stream_read(_ptr(buf), buf.numel(), _ptr(sink), _stream(buf)))
