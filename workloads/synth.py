"""Seeded synthetic inputs for the packed-MoE decode FFN and the dense packed GEMV.

This module only draws random numbers and encodes them into the storage formats the
library consumes (bf16 bit patterns, packed 4-bit codes, bf16 group scales).  It holds
none of the method's arithmetic: no decode of a code back to a value, no product, no
softmax.  Both the CPU oracle (``oracle/``) and the GPU path's tests and benchmark draw
their inputs from here, so that the two sides see the same bytes.

Storage layouts (FireEcho page, "The Goliath Kernel: Why It's Fast": all experts of a
layer in one contiguous ``[E, K//2, N]`` byte buffer, low nibble taken first):

* packed weights ``u8 [E, K/2, N]``: byte ``[e, r, n]`` holds K index ``2r`` in bits 0-3
  and K index ``2r+1`` in bits 4-7; N is the contiguous axis.
* group scales ``bf16 [E, K/G, N]`` (stored as uint16 bit patterns), same orientation.
* fused gate_up: columns ``[0, I)`` are gate, ``[I, 2I)`` are up.

Draw order for one MoE layer (fixed so a layer is reproducible from its seed): x, logits,
the per-expert bias or the expert permutation, then for each expert in index order its
gate_up codes, gate_up scales, down codes, down scales.  Layer ``l`` of a stack uses seed
``1000 * seed + l``.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

FMT_INT4 = 0  # value = (nibble - 8) * scale
FMT_FP4 = 1   # value = E2M1(nibble) * scale
FMT_FP8 = 2   # value = E4M3(byte) * scale, one byte per weight
FMT_INT2 = 3  # value = (code - 2) * scale, four codes per byte (per-expert cold format)
FMT_FEXC = 4  # value = (C1[c1] + C2[c2])[i] * scale, 2 codes per 8 weights (codebook format)


# --------------------------------------------------------------------------------------
# bit-pattern encoders (inputs only)
# --------------------------------------------------------------------------------------
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    a32 = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a32.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_view_f32(bits) -> np.ndarray:
    """Reinterpret bf16 bit patterns as float32 (exact widening).  Used by generators
    that need to know the stored scale value, e.g. the quantizer below."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes ``[..., K, N]`` (values 0..15) into bytes ``[..., K/2, N]``:
    even K index in the low nibble, odd K index in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-2] % 2 == 0
    lo = c[..., 0::2, :]
    hi = c[..., 1::2, :]
    return (lo | (hi << 4)).astype(np.uint8)


# --------------------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------------------
@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    E: int
    H: int
    I: int
    k: int
    fmt: int
    group: int
    scale_lo: float
    scale_hi: float
    logits: str = "normal"          # "normal" | "normal+bias" | "zipf"
    bias_sigma: float = 0.5
    zipf_s: float = 1.1
    layers: int = 1
    residual: bool = False          # chained stack: x_{l+1} = bf16(x_l + MoE_l(x_l))
    int2_frac: float = 0.0          # share of experts stored as INT2 (cold experts)
    fexc_frac: float = 0.0          # share of experts stored as FE-XC codebook codes

    def with_T(self, T: int) -> "MoEConfig":
        return replace(self, T=T)

    @property
    def kb(self) -> int:
        """K indices per stored byte (2 for the 4-bit formats, 1 for FP8)."""
        return 1 if self.fmt == FMT_FP8 else 2

    @property
    def bytes_per_expert(self) -> int:
        """Packed weight + scale bytes of one expert (gate_up and down)."""
        H, I, G, b = self.H, self.I, self.group, self.kb
        return (H // b) * (2 * I) + (H // G) * (2 * I) * 2 + (I // b) * H + (I // G) * H * 2


@dataclass(frozen=True)
class GemvConfig:
    name: str
    T: int
    K: int
    N: int
    group: int = 128
    w_sigma: float = 0.02

    @property
    def weight_bytes(self) -> int:
        return (self.K // 2) * self.N + (self.K // self.group) * self.N * 2


TINY = MoEConfig("tiny", T=1, E=8, H=256, I=128, k=2, fmt=FMT_INT4, group=32,
                 scale_lo=0.005, scale_hi=0.02)
Q30 = MoEConfig("q30", T=1, E=128, H=2048, I=768, k=8, fmt=FMT_FP4, group=32,
                scale_lo=0.002, scale_hi=0.01)
Q30_BATCH = replace(Q30, name="q30_batch", T=16, logits="normal+bias")
Q30_FP8 = replace(Q30, name="q30_fp8", fmt=FMT_FP8)
Q30_MIXED = replace(Q30, name="q30_mixed", int2_frac=0.5)
Q30_CODEBOOK = replace(Q30, name="q30_codebook", int2_frac=0.25, fexc_frac=0.25)
W512 = MoEConfig("w512", T=1, E=512, H=2048, I=512, k=10, fmt=FMT_FP4, group=32,
                 scale_lo=0.002, scale_hi=0.01, logits="zipf", layers=48, residual=True)
GEMV_N = (256, 8192, 34816)
GEMV_T = (1, 4)


def gemv_config(N: int, T: int = 1) -> GemvConfig:
    return GemvConfig(f"gemv_n{N}_t{T}", T=T, K=5120, N=N)


# --------------------------------------------------------------------------------------
# MoE layer inputs
# --------------------------------------------------------------------------------------
@dataclass
class MoELayer:
    cfg: MoEConfig
    seed: int
    x: Optional[np.ndarray]      # uint16 [T, H] bf16 bits (None for layers > 0 of a stack)
    logits: np.ndarray           # float32 [T, E]
    w_gu: np.ndarray             # uint8  [E, H/2, 2I]
    s_gu: np.ndarray             # uint16 [E, H/G, 2I]
    w_d: np.ndarray              # uint8  [E, I/2, H]
    s_d: np.ndarray              # uint16 [E, I/G, H]
    meta: dict = field(default_factory=dict)
    expert_fmt: Optional[np.ndarray] = None  # uint8 [E] per-expert format (mixed layers)
    codebooks: Optional[np.ndarray] = None   # uint16 bf16 [E, 2, 2, 256, 8] (FE-XC experts)


def fp8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """FP8 E4M3 weight codes: N(0, 2) values rounded to E4M3 (nearest-even, by torch's
    float8_e4m3fn cast; input encoding only).  |value| < 448, so no NaN code appears."""
    import torch
    v = (2.0 * rng.standard_normal(shape)).astype(np.float32)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _scales(rng: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    return f32_to_bf16_bits(rng.uniform(lo, hi, size=shape))


def make_logits(cfg: MoEConfig, rng: np.random.Generator, T: int) -> np.ndarray:
    E = cfg.E
    if cfg.logits == "normal":
        lg = rng.standard_normal((T, E))
    elif cfg.logits == "normal+bias":
        noise = rng.standard_normal((T, E))
        bias = rng.normal(0.0, cfg.bias_sigma, size=E)
        lg = noise + bias[None, :]
    elif cfg.logits == "zipf":
        noise = rng.standard_normal((T, E))
        perm = rng.permutation(E)
        lg = -cfg.zipf_s * np.log1p(perm.astype(np.float64))[None, :] + noise
    else:
        raise ValueError(cfg.logits)
    return lg.astype(np.float32)


def make_moe_layer(cfg: MoEConfig, seed: int = 0, layer: int = 0, with_x: bool = True,
                   experts: Optional[np.ndarray] = None) -> MoELayer:
    """One MoE layer drawn from ``default_rng(1000*seed + layer)`` (plain ``seed`` for a
    single layer).  ``experts`` (optional) restricts which expert slabs are drawn; the
    others are left zero.  The draw order is unchanged, so drawn slabs are identical
    to a full draw."""
    s = seed if cfg.layers == 1 else 1000 * seed + layer
    rng = np.random.default_rng(s)
    T, E, H, I, G = cfg.T, cfg.E, cfg.H, cfg.I, cfg.group
    x = f32_to_bf16_bits(rng.standard_normal((T, H))) if with_x else None
    if not with_x:
        rng.standard_normal((T, H))  # keep the draw order identical
    logits = make_logits(cfg, rng, T)
    b = cfg.kb
    w_gu = np.zeros((E, H // b, 2 * I), np.uint8)
    s_gu = np.zeros((E, H // G, 2 * I), np.uint16)
    w_d = np.zeros((E, I // b, H), np.uint8)
    s_d = np.zeros((E, I // G, H), np.uint16)
    codes = fp8_codes if cfg.fmt == FMT_FP8 else \
        (lambda g, shape: g.integers(0, 256, size=shape, dtype=np.uint8))
    efmt = expert_formats(cfg, seed, layer)
    want = None if experts is None else set(int(e) for e in np.asarray(experts).ravel())
    for e in range(E):
        sub = rng.spawn(1)[0]
        if want is not None and e not in want:
            continue
        if efmt is not None and efmt[e] in (FMT_INT2, FMT_FEXC):  # codes: first K/4 rows
            w_gu[e, : H // 4] = codes(sub, (H // 4, 2 * I))
            s_gu[e] = _scales(sub, (H // G, 2 * I), cfg.scale_lo, cfg.scale_hi)
            w_d[e, : I // 4] = codes(sub, (I // 4, H))
            s_d[e] = _scales(sub, (I // G, H), cfg.scale_lo, cfg.scale_hi)
            continue
        w_gu[e] = codes(sub, (H // b, 2 * I))
        s_gu[e] = _scales(sub, (H // G, 2 * I), cfg.scale_lo, cfg.scale_hi)
        w_d[e] = codes(sub, (I // b, H))
        s_d[e] = _scales(sub, (I // G, H), cfg.scale_lo, cfg.scale_hi)
    return MoELayer(cfg, seed, x, logits, w_gu, s_gu, w_d, s_d, meta={"rng_seed": s},
                    expert_fmt=efmt, codebooks=make_codebooks(cfg, seed, layer))


def make_codebooks(cfg: MoEConfig, seed: int = 0, layer: int = 0) -> Optional[np.ndarray]:
    """FE-XC codebooks of every expert (gate_up and down, two codebooks each, 256 entries of
    8): bf16 N(0, 2), from their own stream ``default_rng([seed, layer, 0xC0])``; None when
    the layer has no FE-XC experts."""
    if cfg.fexc_frac <= 0:
        return None
    rng = np.random.default_rng([seed, layer, 0xC0])
    return f32_to_bf16_bits(2.0 * rng.standard_normal((cfg.E, 2, 2, 256, 8)))


def expert_formats(cfg: MoEConfig, seed: int = 0, layer: int = 0) -> Optional[np.ndarray]:
    """Per-expert formats of a mixed layer: round(int2_frac E) experts, drawn from their own
    stream ``default_rng([seed, layer, 0x12])``, are INT2, the rest the layer's format; None
    when the layer has no INT2 experts."""
    if cfg.int2_frac <= 0 and cfg.fexc_frac <= 0:
        return None
    n2 = int(round(cfg.int2_frac * cfg.E))
    nx = int(round(cfg.fexc_frac * cfg.E))
    cold = np.random.default_rng([seed, layer, 0x12]).permutation(cfg.E)
    f = np.full(cfg.E, cfg.fmt, np.uint8)
    f[cold[:n2]] = FMT_INT2
    f[cold[n2:n2 + nx]] = FMT_FEXC
    return f


# --------------------------------------------------------------------------------------
# dense GEMV inputs
# --------------------------------------------------------------------------------------
def quantize_int4_groups(w: np.ndarray, group: int):
    """Symmetric INT4 group quantization of ``w [K, N]`` along K (input encoding only).

    Per group of ``group`` K indices and column n: ``s = bf16(absmax / 7)`` (1 when the
    group is all zero), ``q = clamp(rint(w / s), -8, 7)``, stored nibble ``q + 8``.
    Returns ``(codes uint8 [K, N] in 0..15, scale bits uint16 [K/G, N])``.
    """
    K, N = w.shape
    assert K % group == 0
    wg = w.reshape(K // group, group, N)
    absmax = np.abs(wg).max(axis=1)
    s_bits = f32_to_bf16_bits(absmax / 7.0)
    s_bits = np.where(absmax == 0, f32_to_bf16_bits(np.ones_like(absmax)), s_bits)
    s_val = bf16_bits_view_f32(s_bits).astype(np.float64)
    q = np.clip(np.rint(wg / s_val[:, None, :]), -8, 7).astype(np.int16)
    codes = (q + 8).astype(np.uint8).reshape(K, N)
    return codes, s_bits.astype(np.uint16)


@dataclass
class GemvInputs:
    cfg: GemvConfig
    seed: int
    x: np.ndarray   # uint16 [T, K]
    w: np.ndarray   # uint8  [K/2, N]
    s: np.ndarray   # uint16 [K/G, N]


def make_gemv(cfg: GemvConfig, seed: int = 0) -> GemvInputs:
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(rng.standard_normal((cfg.T, cfg.K)))
    w = rng.normal(0.0, cfg.w_sigma, size=(cfg.K, cfg.N)).astype(np.float32)
    codes, s = quantize_int4_groups(w, cfg.group)
    return GemvInputs(cfg, seed, x, pack_nibbles(codes), s)


def random_packed(rng: np.random.Generator, K: int, N: int, group: int, lo=0.002, hi=0.01):
    """Uniform random packed codes ``[K/2, N]`` and bf16 scales ``[K/G, N]``."""
    return (rng.integers(0, 256, size=(K // 2, N), dtype=np.uint8),
            _scales(rng, (K // group, N), lo, hi))


def make_routing(rng: np.random.Generator, T: int, E: int, k: int):
    """A routing given as input (for calls that take ids and weights): per token k
    distinct experts drawn uniformly, weights from a flat Dirichlet (positive, summing to
    about 1), as int32 [T, k] and float32 [T, k]."""
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), size=T).astype(np.float32)
    return ids, w


def make_router_weights(H: int, E: int, seed: int = 0, layer: int = 0) -> np.ndarray:
    """A bf16 router weight ``W_r [H, E]`` (uint16 bits) drawn i.i.d. N(0, 1/sqrt(H)) from its
    own stream ``default_rng([seed, layer, 0x52])`` (the layer draws are unchanged), so that
    an N(0, 1) hidden state gives logits of about unit spread, like the logits the other
    workloads draw directly."""
    rng = np.random.default_rng([seed, layer, 0x52])
    return f32_to_bf16_bits(rng.normal(0.0, 1.0 / np.sqrt(H), size=(H, E)))


def moe_layer_logits(cfg: MoEConfig, seed: int = 0, layer: int = 0) -> np.ndarray:
    """The logits make_moe_layer(cfg, seed, layer) draws, without drawing the experts."""
    s = seed if cfg.layers == 1 else 1000 * seed + layer
    rng = np.random.default_rng(s)
    rng.standard_normal((cfg.T, cfg.H))
    return make_logits(cfg, rng, cfg.T)
