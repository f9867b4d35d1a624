"""CPU oracle for the packed-MoE 4-bit decode FFN and the dense packed INT4 GEMV.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links this
module; only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` do.  It shares no code with the HIP library under ``dequant_gemv_amd/``.

Plain, slow and deliberately unfused: every step is the textbook definition, evaluated in
float64 with numpy, one expert and one token at a time.  A matrix product is the only
library primitive used.  Because every dequantized weight is exact (a code with at most
3 significant bits times a bf16 scale with 8), the GPU path computes the same products;
it differs from this oracle only in fp32 summation order and the final bf16 rounding.

What each function follows (page titles as printed at the head of each page):

* packed layout and nibble order -- FireEcho, "The Goliath Kernel: Why It's Fast": all
  experts of a layer in one contiguous ``[E, K//2, N]`` buffer; the low nibble (``& 0xF``)
  is taken before the high nibble (``>> 4``), dequantized by multiplying with a scale.
* FP4 values -- FireEcho, "Quantization Formats" names the FP4 format only; its element
  type is read as OCP Microscaling E2M1 (sign bit, 2 exponent bits with bias 1, 1 mantissa
  bit; exponent field 0 is subnormal).
* FP8 values -- the same table lists an 8-bit "Goliath FP8" format (there used for the KV
  cache); as a weight format its element is read as OCP FP8 E4M3 (sign bit, 4 exponent bits
  with bias 7, 3 mantissa bits; exponent field 0 is subnormal; S.1111.111 is NaN and there
  is no infinity), one byte per weight, ``[E, K, N]`` with the same bf16 group scales.
* INT2 cold experts -- the same table lists a scalar 2-bit INT2 format for the coldest
  experts next to the 4-bit format of the hot ones (an engine that demotes experts by age).
  The pages give no zero point or packing; read as: code n in 0..3 means n - 2, four codes
  per byte with K index 4r + i in bits 2i..2i+1 of byte row r (low bits first, like the
  nibbles), the same bf16 group scales.  A layer may mix formats per expert (a table of E
  entries); every expert keeps the 4-bit slab ``[K/2, N]`` and an INT2 expert's ``[K/4, N]``
  bytes fill the first K/4 rows of its slab.
* FE-XC codebook experts -- the same table lists FE-XC, a 2-bit codebook format "2x8" for
  cold experts.  Read as additive quantization with two codebooks: a group of 8 consecutive
  K indices of one column is C1[c1] + C2[c2], two bf16 vectors of length 8 picked by two
  8-bit codes, times the bf16 group scale; codes ``[K/8, 2, N]`` (codebook m of group g in
  byte row 2g + m) fill the first K/4 rows of the slab; each expert matrix has its own pair
  of codebooks ``[2, 256, 8]``.
* INT4 values -- symmetric, ``nibble - 8``; the page's simplified snippet multiplies the
  raw nibble by the scale, which is not used (it is labelled a simplification).
* group scales -- one bf16 scale per ``group`` consecutive K indices and per column.
* expert IDs read per token -- FireEcho, "The Goliath Kernel" (a launch reads the expert
  IDs and indexes the packed buffer); top-k on the raw logits, ties to the lower index,
  weights = softmax over the selected k.
* fused gate_up then SiLU(gate) * up -- FireEcho, "Speed Optimization History" step 2
  (gate and up as one matmul); FastInfer, "Confirmed elementwise SwiGLU scheduling"
  (the fused operation is SiLU(gate) * up).  Columns ``[0, I)`` are gate, ``[I, 2I)`` up.
* dense GEMV -- FastInfer, "Specialized matrix-vector result" (a vector times a stored
  weight matrix, FP32-or-better products and reductions); the weight is the packed INT4
  ``[K/2, N]`` layout above with group 128.
* router logits from the hidden state -- FireEcho, "Architecture": the MoE FFN is a packed
  MoE with fused dispatch.  The pages do not spell out the router; it is read as the
  plain linear router of an MoE layer, ``logits = x W_r`` with a bf16 ``W_r [H, E]`` and no
  bias, and the selection is made on those logits (here in float64) by the top-k rule
  above.

Every function here is pinned by ``tests/test_oracle_pins.py`` against hand-worked decode
tables, closed forms, library special cases, invariants and exact-rational brute force.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

FMT_INT4 = 0
FMT_FP4 = 1
FMT_FP8 = 2
FMT_INT2 = 3
FMT_FEXC = 4


# ------------------------------------------------------------------------------------
# element decode
# ------------------------------------------------------------------------------------
def e2m1_value(code: int) -> float:
    """OCP MX E2M1: bit 3 sign, bits 2-1 exponent (bias 1), bit 0 mantissa.
    Exponent field 0 is subnormal: value = mantissa * 0.5."""
    sign = (code >> 3) & 1
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:
        mag = 0.5 * man
    else:
        mag = (2.0 ** (exp - 1)) * (1.0 + 0.5 * man)
    return math.copysign(mag, -1.0 if sign else 1.0)


def e4m3_value(code: int) -> float:
    """OCP FP8 E4M3: bit 7 sign, bits 6-3 exponent (bias 7), bits 2-0 mantissa.  Exponent
    field 0 is subnormal: value = mantissa / 8 * 2**-6.  Exponent 15 with mantissa 7 is NaN;
    exponent 15 otherwise is an ordinary binade (no infinity), up to 448."""
    sign = (code >> 7) & 1
    exp = (code >> 3) & 15
    man = code & 7
    if exp == 15 and man == 7:
        return math.nan
    if exp == 0:
        mag = (man / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return math.copysign(mag, -1.0 if sign else 1.0)


def int2_value(code: int) -> float:
    """INT2: stored code n in 0..3 means n - 2."""
    return float(code - 2)


def int4_value(code: int) -> float:
    """Symmetric INT4: stored nibble n means n - 8."""
    return float(code - 8)


def decode_table(fmt: int) -> np.ndarray:
    """Value of every code: 16 entries (4-bit formats) or 256 (FP8; NaN codes give NaN)."""
    if fmt == FMT_FP8:
        return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    if fmt == FMT_INT2:
        return np.array([int2_value(c) for c in range(4)], dtype=np.float64)
    if fmt not in (FMT_FP4, FMT_INT4):
        raise ValueError(fmt)
    fn = e2m1_value if fmt == FMT_FP4 else int4_value
    return np.array([fn(c) for c in range(16)], dtype=np.float64)


def codes_per_byte(fmt: int) -> int:
    """K indices per stored byte: 2 for the 4-bit formats, 1 for FP8, 4 for INT2."""
    return {FMT_FP8: 1, FMT_INT2: 4}.get(fmt, 2)


def unpack_codes2(packed: np.ndarray) -> np.ndarray:
    """INT2 bytes ``[K/4, N]`` -> codes ``[K, N]``: bits 2i..2i+1 of byte row r give K index
    4r + i."""
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty((4 * p.shape[0], p.shape[1]), dtype=np.uint8)
    for i in range(4):
        codes[i::4, :] = (p >> (2 * i)) & 3
    return codes


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round_to_bits(v) -> np.ndarray:
    """Round float64 values to bfloat16, nearest-even, straight from float64 (one
    rounding); return uint16 bit patterns.  Used only to form a chained layer's input."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                       # v = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                  # below 2**-126 the bf16 quantum is fixed
    quantum = np.ldexp(1.0, e - 8)           # 8 significant bits
    r = np.rint(v / quantum) * quantum       # exact scaling; rint is ties-to-even
    f32 = r.astype(np.float32)               # exact: r fits bf16 (finite inputs)
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Bytes ``[..., K/2, N]`` -> codes ``[..., K, N]``: byte row r gives K index 2r from
    its low nibble and 2r+1 from its high nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    shape = p.shape[:-2] + (2 * p.shape[-2], p.shape[-1])
    codes = np.empty(shape, dtype=np.uint8)
    codes[..., 0::2, :] = p & 0x0F
    codes[..., 1::2, :] = p >> 4
    return codes


def dequant(packed: np.ndarray, scale_bits: np.ndarray, group: int, fmt: int,
            cols: Optional[np.ndarray] = None) -> np.ndarray:
    """Dequantize one packed matrix ``[K/2, N]`` (FP8: ``[K, N]``, one code per byte) with
    scales ``[K/G, N]`` into float64 ``[K, N]``:
    ``W[k, n] = value(code[k, n]) * scale[k // group, n]``.
    ``cols`` optionally selects output columns (for sampled checks of large N)."""
    if cols is not None:
        packed = packed[:, cols]
        scale_bits = scale_bits[:, cols]
    if fmt == FMT_FP8:
        codes = np.asarray(packed, dtype=np.uint8)
    elif fmt == FMT_INT2:
        codes = unpack_codes2(packed)
    else:
        codes = unpack_codes(packed)
    K = codes.shape[0]
    assert K % group == 0 and scale_bits.shape[0] == K // group
    vals = decode_table(fmt)[codes]
    if np.isnan(vals).any():
        raise ValueError("NaN weight code")
    scales = np.repeat(bf16_to_f64(scale_bits), group, axis=0)
    return vals * scales


# ------------------------------------------------------------------------------------
# routing
# ------------------------------------------------------------------------------------
def topk_route(logits: np.ndarray, k: int, dtype=np.float32):
    """Per token: the k largest raw logits (ties to the lower expert index; -0.0 and +0.0
    tie), in rank order, and weights = softmax over those k logits.  The logits are taken
    in ``dtype``: float32 for logits handed to the library as fp32, float64 for logits the
    oracle computes itself from the hidden state.
    Returns ``(ids int32 [T, k], weights float64 [T, k])``."""
    lg = np.asarray(logits, dtype=dtype)
    T, E = lg.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    if not np.all(np.isfinite(lg)):
        raise ValueError("logits must be finite")
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        row = [float(v) for v in lg[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))[:k]
        sel = np.array([row[e] for e in order], dtype=np.float64)
        ex = np.exp(sel - sel[0])
        ids[t] = order
        w[t] = ex / ex.sum()
    return ids, w


# ------------------------------------------------------------------------------------
# expert FFN
# ------------------------------------------------------------------------------------
def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g / (1 + exp(-g)); for very negative g exp overflows to inf and the
    quotient is (-)0, which is the correctly rounded limit."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def dequant_fexc(codes: np.ndarray, codebooks_bits: np.ndarray, scale_bits: np.ndarray,
                 group: int) -> np.ndarray:
    """FE-XC: codes ``[K/8, 2, N]`` (or the slab rows holding them), codebooks bf16
    ``[2, 256, 8]``, scales ``[K/G, N]`` -> float64 ``[K, N]``:
    ``W[8g + i, n] = (C[0][c0(g, n)][i] + C[1][c1(g, n)][i]) * scale[(8g + i) // group, n]``."""
    K = scale_bits.shape[0] * group
    N = scale_bits.shape[1]
    c = np.asarray(codes, dtype=np.uint8)[: K // 4].reshape(K // 8, 2, N).astype(np.int64)
    C = bf16_to_f64(codebooks_bits)                      # [2, 256, 8]
    W = C[0][c[:, 0, :]] + C[1][c[:, 1, :]]              # [K/8, N, 8]
    W = W.transpose(0, 2, 1).reshape(K, N)
    return W * np.repeat(bf16_to_f64(scale_bits), group, axis=0)


class ExpertCache:
    """Dequantized experts of one layer, built on first use (the oracle never fuses).
    ``expert_fmt`` (optional, [E]) gives each expert's format; an INT2 or FE-XC expert's codes
    are the first K/4 byte rows of its slab; ``codebooks`` (bf16 ``[E, 2, 2, 256, 8]``: gate_up
    then down) serve the FE-XC experts."""

    def __init__(self, w_gu, s_gu, w_d, s_d, group: int, fmt: int, expert_fmt=None,
                 codebooks=None):
        self.w_gu, self.s_gu, self.w_d, self.s_d = w_gu, s_gu, w_d, s_d
        self.group, self.fmt = group, fmt
        self.codebooks = codebooks
        self.expert_fmt = None if expert_fmt is None else np.asarray(expert_fmt)
        self._gu: Dict[int, np.ndarray] = {}
        self._d: Dict[int, np.ndarray] = {}

    def _fmt(self, e: int) -> int:
        return self.fmt if self.expert_fmt is None else int(self.expert_fmt[e])

    def _deq(self, w, s, e: int, mat: int) -> np.ndarray:
        f = self._fmt(e)
        if f == FMT_FEXC:
            return dequant_fexc(w, self.codebooks[e][mat], s, self.group)
        if f == FMT_INT2:
            w = w[: (s.shape[0] * self.group) // 4]
        return dequant(w, s, self.group, f)

    def gate_up(self, e: int) -> np.ndarray:
        if e not in self._gu:
            self._gu[e] = self._deq(self.w_gu[e], self.s_gu[e], e, 0)
        return self._gu[e]

    def down(self, e: int) -> np.ndarray:
        if e not in self._d:
            self._d[e] = self._deq(self.w_d[e], self.s_d[e], e, 1)
        return self._d[e]


def expert_ffn(x_row: np.ndarray, W_gu: np.ndarray, W_d: np.ndarray) -> np.ndarray:
    """One expert on one token: [g | u] = x W_gu; h = SiLU(g) * u; y = h W_d."""
    I = W_gu.shape[1] // 2
    gu = x_row @ W_gu
    g, u = gu[:I], gu[I:]
    h = silu(g) * u
    return h @ W_d


def moe_ffn(x_bits, ids, weights, w_gu, s_gu, w_d, s_d, group: int, fmt: int,
            residual_bits=None, cache: Optional[ExpertCache] = None,
            expert_fmt=None, codebooks=None) -> np.ndarray:
    """out[t] = residual[t] + sum_j weights[t, j] * FFN_{ids[t, j]}(x[t]), j ascending.
    Returns the unrounded float64 ``[T, H]``."""
    x = bf16_to_f64(x_bits)
    T, H = x.shape
    ids = np.asarray(ids)
    wts = np.asarray(weights, dtype=np.float64)
    c = cache or ExpertCache(w_gu, s_gu, w_d, s_d, group, fmt, expert_fmt, codebooks)
    out = np.zeros((T, H), dtype=np.float64) if residual_bits is None else \
        bf16_to_f64(residual_bits).copy()
    for t in range(T):
        acc = np.zeros(H, dtype=np.float64)
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            acc += wts[t, j] * expert_ffn(x[t], c.gate_up(e), c.down(e))
        out[t] += acc
    return out


def moe_layer(x_bits, logits, k: int, w_gu, s_gu, w_d, s_d, group: int, fmt: int,
              residual_bits=None, cache: Optional[ExpertCache] = None, expert_fmt=None,
              codebooks=None):
    """Route, then the expert FFN and the weighted combine.
    Returns ``(out float64 [T, H], ids, weights)``."""
    ids, w = topk_route(logits, k)
    out = moe_ffn(x_bits, ids, w, w_gu, s_gu, w_d, s_d, group, fmt, residual_bits, cache,
                  expert_fmt, codebooks)
    return out, ids, w


def router_logits(x_bits, wr_bits) -> np.ndarray:
    """logits[t, e] = sum_c x[t, c] * W_r[c, e] over the bf16 hidden state ``x [T, H]`` and
    the bf16 router weight ``W_r [H, E]`` (uint16 bit patterns), in float64.
    Returns ``float64 [T, E]``."""
    return bf16_to_f64(x_bits) @ bf16_to_f64(wr_bits)


def moe_layer_from_hidden(x_bits, wr_bits, k: int, w_gu, s_gu, w_d, s_d, group: int, fmt: int,
                          residual_bits=None, cache: Optional[ExpertCache] = None):
    """The router on the hidden state, top-k on its float64 logits, then the expert FFN
    and the weighted combine.  Returns ``(out float64 [T, H], ids, weights, logits)``."""
    logits = router_logits(x_bits, wr_bits)
    ids, w = topk_route(logits, k, dtype=np.float64)
    out = moe_ffn(x_bits, ids, w, w_gu, s_gu, w_d, s_d, group, fmt, residual_bits, cache)
    return out, ids, w, logits


def moe_stack(x_bits, layers: Sequence, k: int, group: int, fmt: int):
    """Chained layers with a residual stream: x_{l+1} = bf16(x_l + MoE_l(x_l)).
    ``layers`` yields objects with ``logits, w_gu, s_gu, w_d, s_d``.
    Returns ``(bits of the last layer's input, float64 output of the last layer)``."""
    x = np.asarray(x_bits, dtype=np.uint16)
    out = None
    for L in layers:
        out, _, _ = moe_layer(x, L.logits, k, L.w_gu, L.s_gu, L.w_d, L.s_d, group, fmt,
                              residual_bits=x)
        last_in = x
        x = bf16_round_to_bits(out)
    return last_in, out


# ------------------------------------------------------------------------------------
# dense packed GEMV
# ------------------------------------------------------------------------------------
def packed_gemv(x_bits, w_packed, s_bits, group: int, fmt: int = FMT_INT4,
                cols: Optional[np.ndarray] = None) -> np.ndarray:
    """y[t, n] = sum_k x[t, k] * W[k, n] with W the dequantized packed matrix.
    Returns the unrounded float64 ``[T, N]`` (or ``[T, len(cols)]``)."""
    x = bf16_to_f64(x_bits)
    W = dequant(w_packed, s_bits, group, fmt, cols)
    return x @ W
