"""Helpers for the GPU parity tests: host <-> device copies of the generator's arrays and
the elementwise tolerance check (|gpu - oracle| <= 1e-2 * rms(oracle) + 1 bf16 ulp)."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda"


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy array -> device tensor with the same bytes (uint16 travels as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def check_bf16(gpu_bits: np.ndarray, oracle: np.ndarray, rel: float = 1e-2, what: str = ""):
    """The tolerance of the method: per element |diff| <= rel * rms(oracle) + ulp_bf16."""
    g = bf16_f64(gpu_bits)
    o = np.asarray(oracle, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    rms = float(np.sqrt(np.mean(np.square(o)))) if o.size else 0.0
    bound = rel * rms + ulp_bf16(o)
    err = np.abs(g - o)
    ratio = err / bound
    worst = int(np.argmax(ratio)) if ratio.size else 0
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    assert np.all(err <= bound), (
        f"{what}: {int(np.sum(err > bound))} of {err.size} elements out of tolerance; worst "
        f"index {np.unravel_index(worst, o.shape)} gpu={g.flat[worst]!r} "
        f"oracle={o.flat[worst]!r} bound={bound.flat[worst]!r} rms={rms!r}")
    return float(ratio.max()) if ratio.size else 0.0


def upload_layer(L, experts=None):
    """Device copies of one MoE layer's packed buffers.  With ``experts`` only those slabs
    are copied (the rest stay zero; the kernels only read routed experts)."""
    if experts is None:
        return {k: dev(getattr(L, k)) for k in ("w_gu", "s_gu", "w_d", "s_d")}
    out = {}
    for k in ("w_gu", "s_gu", "w_d", "s_d"):
        a = getattr(L, k)
        t = torch.zeros(a.shape, dtype=torch.uint8 if a.dtype == np.uint8 else torch.int16,
                        device=DEV)
        for e in sorted(set(int(v) for v in np.asarray(experts).ravel())):
            t[e].copy_(dev(a[e]))
        out[k] = t
    return out


def check_chain(gpu_bits: np.ndarray, oracle: np.ndarray, n_layers: int, rel: float = 1e-2,
                what: str = "", elementwise: bool = True):
    """Tolerance for an L-layer residual chain x_{l+1} = bf16(x_l + MoE_l(x_l)) run
    independently on both sides.  Each side rounds every layer's output to bf16, and one
    rounding decision that falls differently (values within fp32 noise of a bf16
    midpoint) shifts later layers' inputs, so the per-layer bound does not compose.
    Checked instead: the method's relative tolerance in norm,
    rms(gpu - oracle) <= rel * rms(oracle), and per element at most one bf16 ulp per
    layer on top of the per-layer bound."""
    g = bf16_f64(gpu_bits)
    o = np.asarray(oracle, dtype=np.float64)
    rms = float(np.sqrt(np.mean(np.square(o))))
    err = np.abs(g - o)
    rms_err = float(np.sqrt(np.mean(np.square(err))))
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    assert rms_err <= rel * rms, f"{what}: rms error {rms_err!r} > {rel} * rms {rms!r}"
    if not elementwise:
        return rms_err / rms
    bound = rel * rms + n_layers * ulp_bf16(np.maximum(np.abs(o), np.abs(g)))
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond {n_layers} ulps + "
                           f"{rel} * rms; worst {err.max()!r}")
    return rms_err / rms


GUARD = 4096      # canary bytes on each side of a guarded buffer (keeps 256-byte alignment)
CANARY = 0xA5


def guarded(shape, dtype, zero: bool = False):
    """A device buffer of ``shape``/``dtype`` inside canary bands of GUARD bytes on each
    side.  Returns ``(view, check)``; ``check()`` asserts that no kernel wrote outside the
    view.  ``zero`` zero-fills the view (workspaces)."""
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    base = torch.full((GUARD + n + GUARD,), CANARY, dtype=torch.uint8, device=DEV)
    view = base[GUARD:GUARD + n].view(dtype).view(shape)
    if zero:
        view.zero_()

    def check():
        torch.cuda.synchronize()
        lo, hi = base[:GUARD], base[GUARD + n:]
        assert bool((lo == CANARY).all()) and bool((hi == CANARY).all()), \
            "a kernel wrote outside its buffer (canary band changed)"
    return view, check


def guarded_workspace(nbytes: int):
    """A zero-filled workspace of nbytes (uint8) inside canary bands."""
    return guarded((nbytes,), torch.uint8, zero=True)
