"""Exact-rational brute force for tiny MoE layers and GEMVs (test-side only).

Independent of ``oracle/``: element values come from the hand-typed golden decode table,
gate/up and GEMV sums are exact ``fractions.Fraction`` arithmetic, and only SiLU, the
softmax and the final conversion use float64 (``math.exp``, ``math.fsum``).  Top-k is a
full sort of all (logit, index) pairs.  Pure-Python loops: keep shapes tiny.
"""
from __future__ import annotations

import math
import os
import struct
from fractions import Fraction

_HERE = os.path.dirname(os.path.abspath(__file__))


def golden_tables():
    """{'int4': [Fraction]*16, 'fp4': [Fraction]*16, 'fp4_signbit': [bool]*16}"""
    int4, fp4, neg = [], [], []
    with open(os.path.join(_HERE, "golden", "decode_tables.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            n, a, b = line.split()
            assert int(n) == len(int4)
            int4.append(Fraction(a))
            fp4.append(Fraction(b))
            neg.append(b.startswith("-"))
    return {"int4": int4, "fp4": fp4, "fp4_signbit": neg}


_TABLES = golden_tables()


def bf16_fraction(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0])


def e4m3_fraction(code: int) -> Fraction:
    """FP8 E4M3 from its bit fields, exactly (the hand-worked rows of
    golden/e4m3_worked.txt follow the same definition).  NaN codes are rejected."""
    s, ex, m = code >> 7, (code >> 3) & 15, code & 7
    if ex == 15 and m == 7:
        raise ValueError("NaN code")
    mag = Fraction(m, 8) * Fraction(1, 64) if ex == 0 else \
        (1 + Fraction(m, 8)) * (Fraction(2) ** (ex - 7))
    return -mag if s else mag


def fexc_exact(codes, codebooks, scales, group: int):
    """FE-XC: byte row 2g + m of ``codes`` is codebook m's code of group g (8 K indices);
    W[8g + i][n] = (C[0][c0][i] + C[1][c1][i]) * scale[(8g + i) // group][n], exactly."""
    K, N = len(scales) * group, len(scales[0])
    out = []
    for kk in range(K):
        g, i = kk // 8, kk % 8
        row = []
        for n in range(N):
            c0, c1 = int(codes[2 * g][n]), int(codes[2 * g + 1][n])
            v = bf16_fraction(codebooks[0][c0][i]) + bf16_fraction(codebooks[1][c1][i])
            row.append(v * bf16_fraction(scales[kk // group][n]))
        out.append(row)
    return out


def dequant_exact(packed, scales, group: int, fmt: str):
    """packed [K/2][N] bytes (fp8: [K][N]; int2: [K/4][N], or a 4-bit slab whose first
    K/4 rows hold the codes), scales [K/G][N] bf16 bits -> exact W [K][N] (Fractions)."""
    if fmt == "int2":
        K = len(scales) * group
        out = []
        for k in range(K):
            out.append([Fraction(((int(packed[k // 4][n]) >> (2 * (k % 4))) & 3) - 2) *
                        bf16_fraction(scales[k // group][n]) for n in range(len(packed[0]))])
        return out
    if fmt == "fp8":
        return [[e4m3_fraction(int(b)) * bf16_fraction(scales[k // group][n])
                 for n, b in enumerate(row)] for k, row in enumerate(packed)]
    tab = _TABLES[fmt]
    Kp, N = len(packed), len(packed[0])
    W = [[None] * N for _ in range(2 * Kp)]
    for r in range(Kp):
        for n in range(N):
            b = int(packed[r][n])
            for k, code in ((2 * r, b & 0xF), (2 * r + 1, b >> 4)):
                W[k][n] = tab[code] * bf16_fraction(scales[k // group][n])
    return W


def topk_exact(row, k: int):
    pairs = sorted(((Fraction(float(v)), e) for e, v in enumerate(row)),
                   key=lambda p: (-p[0], p[1]))[:k]
    ids = [e for _, e in pairs]
    l0 = float(pairs[0][0])
    ex = [math.exp(float(v) - l0) for v, _ in pairs]
    s = math.fsum(ex)
    return ids, [v / s for v in ex]


def moe_exact(x_bits, logits, k: int, w_gu, s_gu, w_d, s_d, group: int, fmt,
              residual_bits=None, codebooks=None):
    """fmt: one format name, or a list of E names (per-expert formats).
    Returns (out [T][H] float64, ids [T][k], weights [T][k])."""
    T, H = len(x_bits), len(x_bits[0])
    E = len(w_gu)
    I = len(w_gu[0][0]) // 2
    fmts = fmt if isinstance(fmt, list) else [fmt] * E
    def deq(w, s, e, mat):
        if fmts[e] == "fexc":
            return fexc_exact(w, codebooks[e][mat], s, group)
        return dequant_exact(w, s, group, fmts[e])
    Wgu = [deq(w_gu[e], s_gu[e], e, 0) for e in range(E)]
    Wd = [deq(w_d[e], s_d[e], e, 1) for e in range(E)]
    out, all_ids, all_w = [], [], []
    for t in range(T):
        x = [bf16_fraction(v) for v in x_bits[t]]
        ids, wts = topk_exact(logits[t], k)
        ys = []
        for e in ids:
            g = [sum(x[c] * Wgu[e][c][n] for c in range(H)) for n in range(I)]
            u = [sum(x[c] * Wgu[e][c][I + n] for c in range(H)) for n in range(I)]
            h = [float(g[n]) / (1.0 + math.exp(-float(g[n]))) * float(u[n]) for n in range(I)]
            hf = [Fraction(v) for v in h]
            ys.append([float(sum(hf[n] * Wd[e][n][m] for n in range(I))) for m in range(H)])
        row = []
        for m in range(H):
            terms = [wts[j] * ys[j][m] for j in range(len(ids))]
            if residual_bits is not None:
                terms.append(float(bf16_fraction(residual_bits[t][m])))
            row.append(math.fsum(terms))
        out.append(row)
        all_ids.append(ids)
        all_w.append(wts)
    return out, all_ids, all_w


def router_exact(x_bits, wr_bits):
    """logits[t][e] = sum_c x[t][c] W_r[c][e] over bf16 bit patterns, exact, then float."""
    H, E = len(wr_bits), len(wr_bits[0])
    W = [[bf16_fraction(wr_bits[c][e]) for e in range(E)] for c in range(H)]
    out = []
    for xr in x_bits:
        x = [bf16_fraction(v) for v in xr]
        out.append([float(sum(x[c] * W[c][e] for c in range(H))) for e in range(E)])
    return out


def gemv_exact(x_bits, packed, scales, group: int, fmt: str = "int4"):
    W = dequant_exact(packed, scales, group, fmt)
    K, N = len(W), len(W[0])
    out = []
    for xr in x_bits:
        x = [bf16_fraction(v) for v in xr]
        out.append([float(sum(x[k] * W[k][n] for k in range(K))) for n in range(N)])
    return out


def bf16_rne_bits(v: float) -> int:
    """Round a float to the nearest bf16 (ties to even), exactly via Fractions, and return
    its 16-bit pattern.  Normal and subnormal ranges; no overflow handling (tiny tests)."""
    q = Fraction(v)
    if q == 0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                      # now 2^e <= a < 2^(e+1)
    e = max(e, -126)                # subnormals share the smallest normal's step
    step = Fraction(2) ** (e - 7)   # 7 stored mantissa bits
    m = round(a / step)             # Fraction.__round__: nearest, ties to even
    r = m * step
    f = struct.unpack("<I", struct.pack("<f", float(r)))[0]   # r is exactly an fp32 value
    assert f & 0xFFFF == 0
    return sign | (f >> 16)


def moe_stack_exact(x_bits, layers, k: int, group: int, fmt: str):
    """The chained stack x_{l+1} = bf16(x_l + MoE_l(x_l)) through moe_exact, with the exact
    bf16 rounding above between layers.  ``layers``: objects with logits, w_gu, s_gu, w_d,
    s_d.  Returns (bits of the last layer's input, float64 output of the last layer)."""
    x = [[int(v) for v in row] for row in x_bits]
    out, last_in = None, None
    for L in layers:
        out, _, _ = moe_exact(x, L.logits, k, L.w_gu, L.s_gu, L.w_d, L.s_d, group, fmt,
                              residual_bits=x)
        last_in = x
        x = [[bf16_rne_bits(v) for v in row] for row in out]
    return last_in, out
