"""C-ABI checks that need no GPU: the library loads, exports every function that
include/dqg.h declares, and rejects bad arguments on the host before any launch.

Every call below fails validation, so nothing is ever enqueued (fake device addresses
are never dereferenced; the stream is NULL)."""
import ctypes
import os
import re

import pytest

from dequant_gemv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "dqg.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_header_lists_expected_entry_points():
    fns = header_functions()
    for name in ("topk_route", "moe_fp4_ffn", "moe_fp4_layer", "packed_gemv_int4",
                 "packed_dequant_f32", "moe_fp4_ffn_workspace_bytes",
                 "packed_gemv_int4_workspace_bytes", "dqg_status_string", "dqg_abi_version",
                 "router_logits", "router_logits_workspace_bytes", "moe_fp4_layer_from_hidden",
                 "moe_fp4_layer_mixed"):
        assert name in fns


def test_library_exports_every_header_function():
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name
        assert name in B.SIGNATURES, name


def test_abi_version_and_status_strings():
    assert B.abi_version() == 2
    assert B.status_string(0) == "DQG_OK"
    assert B.status_string(-3) == "DQG_ERR_MISALIGNED"
    assert B.status_string(12345) == "DQG_ERR_UNKNOWN"


def test_workspace_queries():
    q30 = B.moe_fp4_ffn_workspace_bytes(1, 2048, 768, 128, 8)
    assert q30 > 0 and q30 % 256 == 0
    assert B.moe_fp4_ffn_workspace_bytes(64, 2048, 768, 128, 8) > q30
    assert B.moe_fp4_ffn_workspace_bytes(1, 2048, 768, 8, 9) == 0      # k > E
    assert B.moe_fp4_ffn_workspace_bytes(1, 2000, 768, 128, 8) == 0    # H % 64
    assert B.moe_fp4_ffn_workspace_bytes(0, 2048, 768, 128, 8) == 0
    big = B.packed_gemv_int4_workspace_bytes(1, 5120, 34816, 128)        # K splits
    assert big > 0 and big % 256 == 0
    assert B.packed_gemv_int4_workspace_bytes(1, 5120, 8192, 128) > 0    # K split
    assert B.packed_gemv_int4_workspace_bytes(1, 5120, 100, 128) == 0    # N % 64


A = 0x10000  # fake, 16-byte aligned device address (never dereferenced)
MIS = A + 8  # misaligned


def _moe(**kw):
    args = dict(x=A, T=1, H=256, I=128, E=8, k=2, ids=A, w=A, wgu=A, sgu=A, wd=A, sd=A, group=32,
                fmt=0, res=0, out=A, ws=A, wsb=1 << 30)
    args.update(kw)
    a = args
    return B.LIB.moe_fp4_ffn(a["x"], a["T"], a["H"], a["I"], a["E"], a["k"], a["ids"], a["w"],
                             a["wgu"], a["sgu"], a["wd"], a["sd"], a["group"], a["fmt"], a["res"],
                             a["out"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), B.DQG_ERR_INVALID_ARG),
    (dict(ids=0), B.DQG_ERR_INVALID_ARG),
    (dict(out=0), B.DQG_ERR_INVALID_ARG),
    (dict(T=0), B.DQG_ERR_INVALID_ARG),
    (dict(k=9), B.DQG_ERR_INVALID_ARG),
    (dict(k=0), B.DQG_ERR_INVALID_ARG),
    (dict(fmt=7), B.DQG_ERR_UNSUPPORTED),
    (dict(fmt=0x800), B.DQG_ERR_UNSUPPORTED),
    (dict(fmt=B.PATH_FORCE_GEMV | B.PATH_FORCE_MFMA), B.DQG_ERR_INVALID_ARG),
    (dict(group=64), B.DQG_ERR_UNSUPPORTED),
    (dict(H=250), B.DQG_ERR_UNSUPPORTED),
    (dict(I=96), B.DQG_ERR_UNSUPPORTED),
    (dict(E=5000, k=2), B.DQG_ERR_UNSUPPORTED),
    (dict(x=MIS), B.DQG_ERR_MISALIGNED),
    (dict(sd=MIS), B.DQG_ERR_MISALIGNED),
    (dict(res=MIS), B.DQG_ERR_MISALIGNED),
    (dict(ws=0), B.DQG_ERR_WORKSPACE),
    (dict(wsb=100), B.DQG_ERR_WORKSPACE),
])
def test_moe_validation_rejects_before_launch(kw, status):
    assert _moe(**kw) == status


def test_moe_layer_validation():
    f = B.LIB.moe_fp4_layer
    ok = dict(x=A, lg=A, T=1, H=256, I=128, E=8, k=2)
    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["lg"], a["T"], a["H"], a["I"], a["E"], a["k"], A, A, A, A, 32, 1, 0, A,
                 0, 0, A, 1 << 30, None)
    assert call(lg=0) == B.DQG_ERR_INVALID_ARG
    assert call(k=9) == B.DQG_ERR_INVALID_ARG
    assert call(x=MIS) == B.DQG_ERR_MISALIGNED
    assert call(lg=A + 2) == B.DQG_ERR_MISALIGNED


def test_fp8_validation():
    # FP8 runs on both paths; an expert matrix of 2 H I bytes must fit 32-bit offsets
    f = B.LIB.moe_fp4_layer
    def layer(T, fmt, H=256, I=128):
        return f(A, A, T, H, I, 8, 2, A, A, A, A, 32, fmt, 0, A, 0, 0, A, 1 << 40, None)
    assert layer(16, B.FMT_FP8_E4M3, H=32768, I=65536) == B.DQG_ERR_UNSUPPORTED  # 2 H I > 2^31
    assert layer(1, 3) == B.DQG_ERR_UNSUPPORTED                                 # no format 3
    assert _moe(fmt=B.FMT_FP8_E4M3, H=32768, I=65536) == B.DQG_ERR_UNSUPPORTED
    d = B.LIB.packed_dequant_f32
    assert d(A, A, 64, 64, 32, 3, A, None) == B.DQG_ERR_UNSUPPORTED


def test_mixed_layer_validation():
    f = B.LIB.moe_fp4_layer_mixed
    def call(T=1, fmt=B.FMT_FP4_E2M1, tab=A, lg=A, cb=0, I=128):
        return f(A, lg, T, 256, I, 8, 2, A, A, A, A, tab, cb, 32, fmt, 0, A, 0, 0, A, 1 << 30, None)
    assert call(tab=0) == B.DQG_ERR_INVALID_ARG
    assert call(lg=0) == B.DQG_ERR_INVALID_ARG
    assert call(fmt=B.FMT_INT4) == B.DQG_ERR_UNSUPPORTED          # FP4 base only
    assert call(fmt=B.FMT_FP8_E4M3, T=16) == B.DQG_ERR_UNSUPPORTED
    assert call(lg=A + 2) == B.DQG_ERR_MISALIGNED
    assert call(lg=A + 2, T=16) == B.DQG_ERR_MISALIGNED           # multi-launch calls too
    assert call(tab=A + 1) == B.DQG_ERR_MISALIGNED                # table read as words
    assert call(tab=A + 1, T=16) == B.DQG_ERR_MISALIGNED
    assert call(cb=A + 8, I=512) == B.DQG_ERR_MISALIGNED
    assert call(cb=A + 8, T=16) == B.DQG_ERR_MISALIGNED


def test_router_validation():
    f = B.LIB.router_logits
    q = B.router_logits_workspace_bytes(1, 2048, 128)
    assert q == 16 * 128 * 4                                  # 16 row splits x 128 logits
    assert B.router_logits_workspace_bytes(4, 2048, 128) == 4 * q
    assert B.router_logits_workspace_bytes(1, 2048, 60) == 0  # E % 8
    assert B.router_logits_workspace_bytes(1, 2044, 64) == 0  # H % 8
    assert B.router_logits_workspace_bytes(1, 2048, 8192) == 0
    assert f(0, 1, 2048, 128, A, A, A, q, None) == B.DQG_ERR_INVALID_ARG
    assert f(A, 0, 2048, 128, A, A, A, q, None) == B.DQG_ERR_INVALID_ARG
    assert f(A, 1, 2048, 60, A, A, A, q, None) == B.DQG_ERR_UNSUPPORTED
    assert f(MIS, 1, 2048, 128, A, A, A, q, None) == B.DQG_ERR_MISALIGNED
    assert f(A, 1, 2048, 128, A, A, A, q - 4, None) == B.DQG_ERR_WORKSPACE
    assert f(A, 1, 2048, 128, A, A, 0, q, None) == B.DQG_ERR_WORKSPACE


def test_moe_layer_from_hidden_validation():
    f = B.LIB.moe_fp4_layer_from_hidden
    ok = dict(x=A, wr=A, T=1, H=256, I=128, E=8, k=2, lo=0)
    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["wr"], a["T"], a["H"], a["I"], a["E"], a["k"], A, A, A, A, 32, 1, 0, A,
                 a["lo"], 0, 0, A, 1 << 30, None)
    assert call(wr=0) == B.DQG_ERR_INVALID_ARG
    assert call(k=9) == B.DQG_ERR_INVALID_ARG
    assert call(E=12, k=2) == B.DQG_ERR_UNSUPPORTED          # E % 8
    assert call(wr=MIS) == B.DQG_ERR_MISALIGNED
    assert call(lo=A + 2) == B.DQG_ERR_MISALIGNED
    # the MoE workspace query covers the router's partial rows and logits
    assert B.moe_fp4_ffn_workspace_bytes(64, 2048, 768, 128, 8) >= 64 * 17 * 128 * 4


def test_topk_validation():
    f = B.LIB.topk_route
    assert f(0, 1, 8, 2, A, A, None) == B.DQG_ERR_INVALID_ARG
    assert f(A, 1, 8, 9, A, A, None) == B.DQG_ERR_INVALID_ARG
    assert f(A, 0, 8, 2, A, A, None) == B.DQG_ERR_INVALID_ARG
    assert f(A, 1, 8, 0, A, A, None) == B.DQG_ERR_INVALID_ARG
    assert f(A, 1, 8000, 2, A, A, None) == B.DQG_ERR_UNSUPPORTED
    assert f(A, 1, 64, 33, A, A, None) == B.DQG_ERR_UNSUPPORTED
    assert f(A + 1, 1, 8, 2, A, A, None) == B.DQG_ERR_MISALIGNED


def test_gemv_validation():
    f = B.LIB.packed_gemv_int4
    assert f(0, 1, 5120, 256, A, A, 128, A, 0, 0, None) == B.DQG_ERR_INVALID_ARG
    assert f(A, 0, 5120, 256, A, A, 128, A, 0, 0, None) == B.DQG_ERR_INVALID_ARG
    assert f(A, 1, 5120, 100, A, A, 128, A, 0, 0, None) == B.DQG_ERR_UNSUPPORTED
    assert f(A, 1, 5100, 256, A, A, 128, A, 0, 0, None) == B.DQG_ERR_UNSUPPORTED
    assert f(A, 1, 5120, 256, A, A, 64, A, 0, 0, None) == B.DQG_ERR_UNSUPPORTED
    assert f(A, 1, 5120, 256, MIS, A, 128, A, 0, 0, None) == B.DQG_ERR_MISALIGNED
    # a workspace that is given but too small is an error (NULL means "no K split")
    assert f(A, 1, 5120, 8192, A, A, 128, A, A, 16, None) == B.DQG_ERR_WORKSPACE


def test_tiled_gemv_sizes_and_validation():
    """Prepacked sizes (tiles of 128 columns, the last padded) and host-side rejection before
    any launch."""
    wb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    q = B.LIB.packed_gemv_int4_prepack_sizes
    assert q(5120, 34816, 128, ctypes.byref(wb), ctypes.byref(sb)) == B.DQG_OK
    assert wb.value == 5120 // 2 * 34816 and sb.value == 5120 // 128 * 34816 * 2
    assert q(96, 320, 32, ctypes.byref(wb), ctypes.byref(sb)) == B.DQG_OK
    assert wb.value == 3 * 96 * 64 and sb.value == 3 * 3 * 256   # 3 tiles, 64 columns padded
    assert q(5120, 100, 128, ctypes.byref(wb), ctypes.byref(sb)) == B.DQG_ERR_UNSUPPORTED
    assert q(5120, 256, 128, None, ctypes.byref(sb)) == B.DQG_ERR_INVALID_ARG
    p = B.LIB.packed_gemv_int4_prepack
    assert p(0, A, 5120, 256, 128, A, A, None) == B.DQG_ERR_INVALID_ARG
    assert p(A, A, 5120, 100, 128, A, A, None) == B.DQG_ERR_UNSUPPORTED
    assert p(A, A, 5120, 256, 128, MIS, A, None) == B.DQG_ERR_MISALIGNED
    f = B.LIB.packed_gemv_int4_tiled
    assert f(0, 1, 5120, 256, A, A, 128, A, 0, 0, None) == B.DQG_ERR_INVALID_ARG
    assert f(A, 5, 5120, 256, A, A, 128, A, 0, 0, None) == B.DQG_ERR_UNSUPPORTED   # T > 4
    assert f(A, 1, 5120, 100, A, A, 128, A, 0, 0, None) == B.DQG_ERR_UNSUPPORTED
    assert f(A, 1, 5120, 256, A, MIS, 128, A, 0, 0, None) == B.DQG_ERR_MISALIGNED
    # a workspace that is given but too small is an error (NULL means "no K split")
    assert f(A, 1, 5120, 8192, A, A, 128, A, A, 16, None) == B.DQG_ERR_WORKSPACE


def test_dequant_validation():
    f = B.LIB.packed_dequant_f32
    assert f(0, A, 64, 64, 32, 0, A, None) == B.DQG_ERR_INVALID_ARG
    assert f(A, A, 64, 64, 32, 5, A, None) == B.DQG_ERR_UNSUPPORTED
    assert f(A, A, 48, 64, 32, 0, A, None) == B.DQG_ERR_UNSUPPORTED
    assert f(A, A, 64, 24, 32, 0, A, None) == B.DQG_ERR_UNSUPPORTED
    assert f(A, MIS, 64, 64, 32, 0, A, None) == B.DQG_ERR_MISALIGNED


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        B.topk_route(torch.zeros(1, 8), 2)


def test_noalloc_gemv_host_checks():
    """The allocation-free GEMV validates on the host before it touches the device: bad
    arguments, and partials beyond its 16 MiB scratch (T = 16, N = 65536: 6 K splits x 16 x
    65536 x 4 bytes = 25 MB) return an error and launch nothing."""
    f = B.LIB.packed_gemv_int4_noalloc
    assert f(0, 1, 5120, 8192, A, A, 128, A, None, None) == B.DQG_ERR_INVALID_ARG
    assert f(A, 1, 5120, 100, A, A, 128, A, None, None) == B.DQG_ERR_UNSUPPORTED
    assert f(MIS, 1, 5120, 8192, A, A, 128, A, None, None) == B.DQG_ERR_MISALIGNED
    assert f(A, 1, 5120, 8192, A, A, 128, A, A + 2, None) == B.DQG_ERR_MISALIGNED
    assert f(A, 16, 5120, 65536, A, A, 128, A, None, None) == B.DQG_ERR_WORKSPACE


@pytest.mark.parametrize("H,I,E,k", [(2048, 768, 128, 8), (2048, 512, 512, 10), (256, 128, 8, 2)])
def test_moe_workspace_size_is_monotonic_in_T(H, I, E, k):
    """The workspace layout is chosen as the largest token capacity whose size fits, so the
    size must never shrink as T grows (otherwise one workspace would get different layouts
    for different T and leave data where another layout expects zeros)."""
    prev = 0
    for T in list(range(1, 65)) + list(range(65, 65536 // k + 1, 37)) + [65536 // k]:
        n = B.moe_fp4_ffn_workspace_bytes(T, H, I, E, k)
        assert n >= prev, (T, n, prev)
        prev = n
