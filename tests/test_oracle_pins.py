"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: hand-worked decode
tables and bytes (tests/golden), closed forms, special cases that reduce to a library
routine (numpy/scipy/torch), invariants, and exact-rational brute force
(tests/bruteforce.py).  Together they are chosen so that a dropped term, a swapped nibble,
a wrong sign, a transposed operand or a wrong group index fails at least one test.
"""
import math
import os
import struct

import numpy as np
import pytest
import scipy.special
import torch

import bruteforce as BF
from oracle import moe_oracle as O
from workloads import synth as S

HERE = os.path.dirname(os.path.abspath(__file__))


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


# --------------------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------------------
def test_decode_tables_match_hand_worked_golden():
    tabs = BF.golden_tables()
    for fmt, key in ((O.FMT_INT4, "int4"), (O.FMT_FP4, "fp4")):
        t = O.decode_table(fmt)
        for code in range(16):
            assert t[code] == float(tabs[key][code]), (fmt, code)
    # the sign of zero: E2M1 code 8 is -0.0, code 0 is +0.0
    t = O.decode_table(O.FMT_FP4)
    for code in range(16):
        assert bool(np.signbit(t[code])) == tabs["fp4_signbit"][code], code


def _worked_rows():
    rows = []
    with open(os.path.join(HERE, "golden", "worked_bytes.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                b, s, fmt, lo, lob, hi, hib = line.split()
                rows.append((int(b, 16), int(s, 16), fmt, float(lo), int(lob, 16),
                             float(hi), int(hib, 16)))
    return rows


@pytest.mark.parametrize("row", _worked_rows())
def test_worked_bytes(row):
    byte, sbits, fmt, lo, lob, hi, hib = row
    f = O.FMT_INT4 if fmt == "int4" else O.FMT_FP4
    W = O.dequant(np.array([[byte]], np.uint8), np.array([[sbits]], np.uint16), 2, f)
    assert W.shape == (2, 1)
    got_lo, got_hi = np.float32(W[0, 0]), np.float32(W[1, 0])
    # the product is exact in fp32: widening back must not change it
    assert float(got_lo) == W[0, 0] and float(got_hi) == W[1, 0]
    assert f32_bits(float(got_lo)) == lob and f32_bits(float(got_hi)) == hib
    assert float(got_lo) == lo and float(got_hi) == hi


def test_pack_nibbles_hand_worked():
    # K index 0 -> low nibble, K index 1 -> high nibble
    codes = np.array([[1, 15], [2, 0], [7, 8], [9, 3]], np.uint8)
    assert S.pack_nibbles(codes).tolist() == [[0x21, 0x0F], [0x97, 0x38]]


@pytest.mark.parametrize("fmt", [O.FMT_INT4, O.FMT_FP4])
@pytest.mark.parametrize("group", [32, 128])
def test_dequant_orientation_and_group_boundaries(fmt, group):
    K, N = 2 * group + group, 5  # three groups
    codes = np.array([[(k * 7 + n * 3 + k // 5) % 16 for n in range(N)] for k in range(K)],
                     np.uint8)
    # distinct power-of-two scale per (group, column): 2^-(g*N + n)
    sexp = np.array([[-(g * N + n) for n in range(N)] for g in range(K // group)])
    sbits = ((sexp + 127).astype(np.uint32) << 7).astype(np.uint16)
    W = O.dequant(S.pack_nibbles(codes), sbits, group, fmt)
    key = "int4" if fmt == O.FMT_INT4 else "fp4"
    tab = BF.golden_tables()[key]
    for k in range(K):
        for n in range(N):
            want = float(tab[codes[k, n]]) * 2.0 ** float(sexp[k // group, n])
            assert W[k, n] == want, (k, n)
    # column subset selects the same values
    cols = np.array([4, 1])
    assert np.array_equal(O.dequant(S.pack_nibbles(codes), sbits, group, fmt, cols), W[:, cols])


def test_bf16_round_hand_worked_and_vs_torch():
    cases = [(1.0, 0x3F80), (1.0 + 2 ** -8, 0x3F80), (1.0 + 3 * 2 ** -8, 0x3F82),
             (-1.0 - 2 ** -7, 0xBF81), (0.0, 0x0000), (-0.0, 0x8000), (3.0e38, 0x7F62)]
    for v, bits in cases:
        assert int(O.bf16_round_to_bits(np.array([v]))[0]) == bits, v
    rng = np.random.default_rng(5)
    v32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_round_to_bits(v32.astype(np.float64)), ref)


# --------------------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------------------
def test_route_k1_is_argmax_and_kE_is_stable_sort():
    rng = np.random.default_rng(1)
    lg = rng.choice(np.array([-1.0, 0.0, 1.0, -0.0, 0.5], np.float32), size=(40, 9))
    ids1, w1 = O.topk_route(lg, 1)
    assert np.array_equal(ids1[:, 0], np.argmax(lg, axis=1))
    assert np.all(w1 == 1.0)
    idsE, wE = O.topk_route(lg, 9)
    assert np.array_equal(idsE, np.argsort(-lg, axis=1, kind="stable"))
    for t in range(lg.shape[0]):
        ref = scipy.special.softmax(lg[t].astype(np.float64)[idsE[t]])
        np.testing.assert_allclose(wE[t], ref, rtol=1e-14, atol=0)


def test_route_ties_pick_lower_index_and_zero_signs_tie():
    lg = np.array([[0.0, -0.0, 0.0, 2.0, 2.0, -1.0]], np.float32)
    ids, w = O.topk_route(lg, 4)
    assert ids.tolist() == [[3, 4, 0, 1]]
    np.testing.assert_allclose(w.sum(), 1.0, rtol=1e-15)
    assert w[0, 0] == w[0, 1] and w[0, 2] == w[0, 3]


def test_route_rejects_bad_k_and_nonfinite():
    with pytest.raises(ValueError):
        O.topk_route(np.zeros((1, 4), np.float32), 5)
    with pytest.raises(ValueError):
        O.topk_route(np.array([[0.0, np.nan]], np.float32), 1)


@pytest.mark.parametrize("seed", range(6))
def test_route_matches_bruteforce(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(2, 12))
    k = int(rng.integers(1, E + 1))
    lg = rng.choice(np.linspace(-2, 2, 7).astype(np.float32), size=(3, E))
    ids, w = O.topk_route(lg, k)
    for t in range(3):
        bi, bw = BF.topk_exact(lg[t], k)
        assert ids[t].tolist() == bi
        np.testing.assert_allclose(w[t], bw, rtol=1e-14)


# --------------------------------------------------------------------------------------
# SiLU
# --------------------------------------------------------------------------------------
def test_silu_identities_and_library():
    x = np.linspace(-40, 40, 4001)
    s = O.silu(x)
    np.testing.assert_allclose(s - O.silu(-x), x, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s + O.silu(-x), x * np.tanh(x / 2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, x * scipy.special.expit(x), rtol=1e-13, atol=0)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([-1000.0]))[0] == 0.0


# --------------------------------------------------------------------------------------
# expert FFN and combine
# --------------------------------------------------------------------------------------
def _identity_tiny(fmt):
    """Tiny shape (H = 2I = 256): every expert maps gate_n = x_n, up_n = x_{n+I} and
    y_m = h_m (m < I), 0 otherwise; scales 1.0."""
    cfg = S.TINY
    E, H, I, G = cfg.E, cfg.H, cfg.I, cfg.group
    one = 9 if fmt == O.FMT_INT4 else 2   # value 1.0
    zero = 8 if fmt == O.FMT_INT4 else 0  # value 0.0
    cgu = np.full((H, 2 * I), zero, np.uint8)
    for n in range(I):
        cgu[n, n] = one
        cgu[n + I, I + n] = one
    cd = np.full((I, H), zero, np.uint8)
    for n in range(I):
        cd[n, n] = one
    w_gu = np.broadcast_to(S.pack_nibbles(cgu), (E, H // 2, 2 * I)).copy()
    w_d = np.broadcast_to(S.pack_nibbles(cd), (E, I // 2, H)).copy()
    s_gu = np.full((E, H // G, 2 * I), 0x3F80, np.uint16)
    s_d = np.full((E, I // G, H), 0x3F80, np.uint16)
    return w_gu, s_gu, w_d, s_d


@pytest.mark.parametrize("fmt", [O.FMT_INT4, O.FMT_FP4])
def test_identity_expert_closed_form(fmt):
    cfg = S.TINY
    w_gu, s_gu, w_d, s_d = _identity_tiny(fmt)
    rng = np.random.default_rng(3)
    x_bits = S.f32_to_bf16_bits(rng.standard_normal((3, cfg.H)))
    logits = rng.standard_normal((3, cfg.E)).astype(np.float32)
    out, ids, w = O.moe_layer(x_bits, logits, cfg.k, w_gu, s_gu, w_d, s_d, cfg.group, fmt)
    x = S.bf16_bits_view_f32(x_bits).astype(np.float64)
    I = cfg.I
    want = np.zeros_like(out)
    for t in range(3):
        for n in range(I):
            xn = float(x[t, n])
            want[t, n] = xn / (1.0 + math.exp(-xn)) * float(x[t, n + I])
    np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-15)
    assert np.all(out[:, I:] == 0.0)


@pytest.mark.parametrize("fmt", [O.FMT_INT4, O.FMT_FP4])
def test_top1_reduces_to_dense_ffn_torch(fmt):
    cfg = S.replace(S.TINY, k=1, fmt=fmt)
    L = S.make_moe_layer(cfg, seed=4)
    L.x = S.f32_to_bf16_bits(np.random.default_rng(9).standard_normal((4, cfg.H)))
    L.logits = np.random.default_rng(10).standard_normal((4, cfg.E)).astype(np.float32)
    out, ids, w = O.moe_layer(L.x, L.logits, 1, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group, fmt)
    assert np.all(w == 1.0)
    x = torch.from_numpy(S.bf16_bits_view_f32(L.x).astype(np.float64))
    for t in range(4):
        e = int(ids[t, 0])
        Wgu = torch.from_numpy(O.dequant(L.w_gu[e], L.s_gu[e], cfg.group, fmt))
        Wd = torch.from_numpy(O.dequant(L.w_d[e], L.s_d[e], cfg.group, fmt))
        gu = x[t] @ Wgu
        ref = (torch.nn.functional.silu(gu[: cfg.I]) * gu[cfg.I:]) @ Wd
        np.testing.assert_allclose(out[t], ref.numpy(), rtol=1e-12, atol=1e-12)


def _tiny_random(rng, T, E, H, I, G, fmt_key):
    w_gu = rng.integers(0, 256, size=(E, H // 2, 2 * I), dtype=np.uint8)
    w_d = rng.integers(0, 256, size=(E, I // 2, H), dtype=np.uint8)
    # scales: random bf16 in a moderate range, plus some exact powers of two
    s_gu = S.f32_to_bf16_bits(rng.uniform(0.05, 0.5, size=(E, H // G, 2 * I)))
    s_d = S.f32_to_bf16_bits(rng.uniform(0.05, 0.5, size=(E, I // G, H)))
    x = S.f32_to_bf16_bits(rng.standard_normal((T, H)))
    lg = rng.choice(np.array([-1.0, 0.0, 1.0, -0.0, 0.25], np.float32), size=(T, E))
    return x, lg, w_gu, s_gu, w_d, s_d


@pytest.mark.parametrize("seed", range(6))
def test_moe_matches_exact_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 4))
    E = int(rng.integers(1, 5))
    k = int(rng.integers(1, E + 1))
    G = 4
    H = int(rng.choice([8, 12, 16]))
    I = int(rng.choice([4, 8]))
    fmt = O.FMT_INT4 if seed % 2 == 0 else O.FMT_FP4
    key = "int4" if fmt == O.FMT_INT4 else "fp4"
    x, lg, w_gu, s_gu, w_d, s_d = _tiny_random(rng, T, E, H, I, G, key)
    res = S.f32_to_bf16_bits(rng.standard_normal((T, H))) if seed % 3 == 0 else None
    out, ids, w = O.moe_layer(x, lg, k, w_gu, s_gu, w_d, s_d, G, fmt, residual_bits=res)
    bout, bids, bw = BF.moe_exact(x.tolist(), lg.tolist(), k, w_gu.tolist(), s_gu.tolist(),
                                  w_d.tolist(), s_d.tolist(), G, key,
                                  None if res is None else res.tolist())
    assert ids.tolist() == bids
    np.testing.assert_allclose(w, bw, rtol=1e-14)
    scale = max(1e-300, float(np.sqrt(np.mean(np.square(bout)))))
    assert np.max(np.abs(out - np.array(bout))) <= 1e-12 * scale + 1e-300


# --------------------------------------------------------------------------------------
# FP8 E4M3
# --------------------------------------------------------------------------------------
def _e4m3_golden():
    rows = []
    for line in open(os.path.join(HERE, "golden", "e4m3_worked.txt")):
        line = line.split("#")[0].strip()
        if line:
            c, v, b = line.split()
            rows.append((int(c, 16), v, b))
    return rows


def test_e4m3_hand_worked_codes():
    tab = O.decode_table(O.FMT_FP8)
    for code, v, b in _e4m3_golden():
        if v == "nan":
            assert math.isnan(tab[code])
            continue
        assert tab[code] == float(v) and math.copysign(1, tab[code]) == math.copysign(1, float(v))
        W = O.dequant(np.array([[code]], np.uint8), np.array([[0x3C80]], np.uint16), 1, O.FMT_FP8)
        assert struct.unpack("<I", struct.pack("<f", W[0, 0]))[0] == int(b, 16)


def test_e4m3_table_matches_torch_float8():
    tab = O.decode_table(O.FMT_FP8)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(tab), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(tab[ok], ref[ok])
    assert np.array_equal(np.signbit(tab[ok]), np.signbit(ref[ok]))
    assert np.sum(np.isnan(tab)) == 2 and np.nanmax(tab) == 448.0


def test_fp8_dequant_layout_is_one_code_per_byte_row():
    rng = np.random.default_rng(7)
    K, N, G = 64, 16, 32
    codes = S.fp8_codes(rng, (K, N))
    scales = S.f32_to_bf16_bits(rng.uniform(0.1, 1.0, size=(K // G, N)))
    W = O.dequant(codes, scales, G, O.FMT_FP8)
    ex = BF.dequant_exact(codes.tolist(), scales.tolist(), G, "fp8")
    assert W.shape == (K, N)
    assert all(W[kk, n] == float(ex[kk][n]) for kk in range(K) for n in range(N))
    with pytest.raises(ValueError):
        O.dequant(np.full((32, 1), 0x7F, np.uint8), np.ones((1, 1), np.uint16), 32, O.FMT_FP8)


@pytest.mark.parametrize("seed", range(3))
def test_fp8_moe_matches_exact_bruteforce(seed):
    rng = np.random.default_rng(500 + seed)
    T, E, k, G, H, I = int(rng.integers(1, 4)), 3, 2, 4, 8, 4
    x = S.f32_to_bf16_bits(rng.standard_normal((T, H)))
    w_gu = np.stack([S.fp8_codes(rng, (H, 2 * I)) for _ in range(E)])
    w_d = np.stack([S.fp8_codes(rng, (I, H)) for _ in range(E)])
    s_gu = S.f32_to_bf16_bits(rng.uniform(0.05, 0.5, size=(E, H // G, 2 * I)))
    s_d = S.f32_to_bf16_bits(rng.uniform(0.05, 0.5, size=(E, I // G, H)))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    out, ids, w = O.moe_layer(x, lg, k, w_gu, s_gu, w_d, s_d, G, O.FMT_FP8)
    bout, bids, bw = BF.moe_exact(x.tolist(), lg.tolist(), k, w_gu.tolist(), s_gu.tolist(),
                                  w_d.tolist(), s_d.tolist(), G, "fp8")
    assert ids.tolist() == bids
    scale = max(1e-300, float(np.sqrt(np.mean(np.square(bout)))))
    assert np.max(np.abs(out - np.array(bout))) <= 1e-12 * scale + 1e-300


# --------------------------------------------------------------------------------------
# INT2 cold experts and mixed per-expert formats
# --------------------------------------------------------------------------------------
def test_int2_hand_worked_bytes():
    rows = []
    for line in open(os.path.join(HERE, "golden", "int2_worked.txt")):
        line = line.split("#")[0].strip()
        if line:
            b, *v = line.split()
            rows.append((int(b, 16), [float(x) for x in v]))
    packed = np.array([[b] for b, _ in rows], np.uint8)            # [R, 1]
    K = 4 * len(rows)
    W = O.dequant(packed, np.full((K // 4, 1), 0x3F80, np.uint16), 4, O.FMT_INT2)  # scale 1
    assert W[:, 0].tolist() == [x for _, v in rows for x in v]


@pytest.mark.parametrize("seed", range(2))
def test_int2_dequant_matches_exact_bruteforce(seed):
    rng = np.random.default_rng(600 + seed)
    K, N, G = 64, 8, 32
    packed = rng.integers(0, 256, size=(K // 4, N), dtype=np.uint8)
    scales = S.f32_to_bf16_bits(rng.uniform(0.1, 1.0, size=(K // G, N)))
    W = O.dequant(packed, scales, G, O.FMT_INT2)
    ex = BF.dequant_exact(packed.tolist(), scales.tolist(), G, "int2")
    assert all(W[kk, n] == float(ex[kk][n]) for kk in range(K) for n in range(N))


def test_int2_expert_equals_int4_expert_with_shifted_codes():
    """INT2 code n and INT4 nibble n + 6 both mean n - 2: a layer whose experts are INT2 gives
    exactly the output of the same layer stored as INT4 (pins the 2-bit order and offset)."""
    rng = np.random.default_rng(17)
    T, E, k, G, H, I = 3, 4, 2, 32, 64, 32
    x = S.f32_to_bf16_bits(rng.standard_normal((T, H)))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    c_gu = rng.integers(0, 4, size=(E, H, 2 * I))
    c_d = rng.integers(0, 4, size=(E, I, H))
    s_gu = S.f32_to_bf16_bits(rng.uniform(0.05, 0.5, size=(E, H // G, 2 * I)))
    s_d = S.f32_to_bf16_bits(rng.uniform(0.05, 0.5, size=(E, I // G, H)))

    def pack2(c):  # [.., K, N] codes 0..3 -> 4-bit slab [.., K/2, N] with the first K/4 rows
        K = c.shape[-2]
        slab = np.zeros(c.shape[:-2] + (K // 2, c.shape[-1]), np.uint8)
        for i in range(4):
            slab[..., : K // 4, :] |= (c[..., i::4, :] << (2 * i)).astype(np.uint8)
        return slab
    int4 = lambda c: S.pack_nibbles((c + 6).astype(np.uint8))
    o2, i2, _ = O.moe_layer(x, lg, k, pack2(c_gu), s_gu, pack2(c_d), s_d, G, O.FMT_FP4,
                            expert_fmt=np.full(E, O.FMT_INT2))
    o4, i4, _ = O.moe_layer(x, lg, k, np.stack([int4(c) for c in c_gu]), s_gu,
                            np.stack([int4(c) for c in c_d]), s_d, G, O.FMT_INT4)
    assert np.array_equal(i2, i4)
    assert np.array_equal(o2, o4)


@pytest.mark.parametrize("seed", range(3))
def test_mixed_formats_match_exact_bruteforce(seed):
    rng = np.random.default_rng(700 + seed)
    T, E, k, G, H, I = int(rng.integers(1, 4)), 4, 2, 4, 16, 8
    x, lg, w_gu, s_gu, w_d, s_d = _tiny_random(rng, T, E, H, I, G, "fp4")
    efmt = np.array([O.FMT_FP4, O.FMT_INT2, O.FMT_INT2, O.FMT_FP4], np.uint8)
    for e in (1, 2):  # INT2 experts: codes in the first K/4 rows, the rest of the slab zero
        w_gu[e, H // 4:] = 0
        w_d[e, I // 4:] = 0
    out, ids, w = O.moe_layer(x, lg, k, w_gu, s_gu, w_d, s_d, G, O.FMT_FP4, expert_fmt=efmt)
    names = ["fp4", "int2", "int2", "fp4"]
    bout, bids, bw = BF.moe_exact(x.tolist(), lg.tolist(), k, w_gu.tolist(), s_gu.tolist(),
                                  w_d.tolist(), s_d.tolist(), G, names)
    assert ids.tolist() == bids
    scale = max(1e-300, float(np.sqrt(np.mean(np.square(bout)))))
    assert np.max(np.abs(out - np.array(bout))) <= 1e-12 * scale + 1e-300


def test_fexc_closed_form_codebooks():
    """C0[c][i] = c / 16 and C1[c][i] = i / 64 (exact bf16) give W[8g + i, n] =
    c0(g, n) / 16 + i / 64 at scale 1: pins the group axis (K), the plane order and the
    element index."""
    rng = np.random.default_rng(31)
    K, N, G = 64, 8, 32
    codes = rng.integers(0, 256, size=(K // 8, 2, N), dtype=np.uint8)
    c = np.arange(256, dtype=np.float64)
    cb = np.stack([np.repeat((c / 16)[:, None], 8, axis=1),
                   np.repeat((np.arange(8) / 64)[None, :], 256, axis=0)])
    W = O.dequant_fexc(codes.reshape(K // 4, N), S.f32_to_bf16_bits(cb),
                       np.full((K // G, N), 0x3F80, np.uint16), G)
    want = np.array([[codes[kk // 8, 0, n] / 16 + (kk % 8) / 64 for n in range(N)]
                     for kk in range(K)])
    assert np.array_equal(W, want)


@pytest.mark.parametrize("seed", range(2))
def test_mixed_fp4_int2_fexc_match_exact_bruteforce(seed):
    rng = np.random.default_rng(800 + seed)
    T, E, k, G, H, I = 2, 3, 2, 8, 16, 16
    x, lg, w_gu, s_gu, w_d, s_d = _tiny_random(rng, T, E, H, I, G, "fp4")
    efmt = np.array([O.FMT_FP4, O.FMT_INT2, O.FMT_FEXC], np.uint8)
    for e in (1, 2):
        w_gu[e, H // 4:] = 0
        w_d[e, I // 4:] = 0
    cb = S.f32_to_bf16_bits(rng.standard_normal((E, 2, 2, 256, 8)))
    out, ids, w = O.moe_layer(x, lg, k, w_gu, s_gu, w_d, s_d, G, O.FMT_FP4, expert_fmt=efmt,
                              codebooks=cb)
    bout, bids, bw = BF.moe_exact(x.tolist(), lg.tolist(), k, w_gu.tolist(), s_gu.tolist(),
                                  w_d.tolist(), s_d.tolist(), G, ["fp4", "int2", "fexc"],
                                  codebooks=cb.tolist())
    assert ids.tolist() == bids
    scale = max(1e-300, float(np.sqrt(np.mean(np.square(bout)))))
    assert np.max(np.abs(out - np.array(bout))) <= 1e-12 * scale + 1e-300


# --------------------------------------------------------------------------------------
# router logits from the hidden state
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(4))
def test_router_logits_match_exact_bruteforce(seed):
    rng = np.random.default_rng(300 + seed)
    T, H, E = int(rng.integers(1, 4)), int(rng.choice([8, 16, 24])), int(rng.choice([4, 8]))
    x = S.f32_to_bf16_bits(rng.standard_normal((T, H)))
    wr = S.f32_to_bf16_bits(rng.normal(0.0, 0.3, size=(H, E)))
    got = O.router_logits(x, wr)
    want = np.array(BF.router_exact(x.tolist(), wr.tolist()))
    mag = np.abs(S.bf16_bits_view_f32(x).astype(np.float64)) @ \
        np.abs(S.bf16_bits_view_f32(wr).astype(np.float64))
    assert got.shape == (T, E)
    assert np.all(np.abs(got - want) <= 1e-15 * mag + 1e-300)


def test_router_one_hot_hidden_state_picks_a_weight_row():
    H, E = 64, 16
    wr = S.make_router_weights(H, E, seed=3)
    Wr = S.bf16_bits_view_f32(wr).astype(np.float64)
    for c in (0, 1, 31, 63):
        x = np.zeros((1, H), np.float32)
        x[0, c] = 1.0
        got = O.router_logits(S.f32_to_bf16_bits(x), wr)
        assert np.array_equal(got[0], Wr[c])
    # a column sum: x of all ones
    got = O.router_logits(S.f32_to_bf16_bits(np.ones((1, H), np.float32)), wr)
    np.testing.assert_allclose(got[0], Wr.sum(axis=0), rtol=1e-14, atol=1e-15)


def test_route_in_float64_separates_values_tied_in_float32():
    lg = np.array([[1.0, 1.0 + 2.0 ** -30, 0.5]])
    ids32, _ = O.topk_route(lg, 2)
    ids64, w64 = O.topk_route(lg, 2, dtype=np.float64)
    assert ids32.tolist() == [[0, 1]]          # both round to 1.0f: the lower index first
    assert ids64.tolist() == [[1, 0]]
    np.testing.assert_allclose(w64[0], scipy.special.softmax(lg[0, [1, 0]]), rtol=1e-15)


def test_router_weights_recipe_gives_unit_spread_logits():
    H, E = 2048, 128
    wr = S.make_router_weights(H, E, seed=0)
    Wr = S.bf16_bits_view_f32(wr).astype(np.float64)
    assert abs(Wr.std() * np.sqrt(H) - 1.0) < 0.01
    x = S.f32_to_bf16_bits(np.random.default_rng(0).standard_normal((8, H)))
    lg = O.router_logits(x, wr)
    assert 0.9 < lg.std() < 1.1


@pytest.mark.parametrize("seed", range(4))
def test_layer_from_hidden_matches_exact_bruteforce(seed):
    rng = np.random.default_rng(400 + seed)
    T, E, k, G, H, I = int(rng.integers(1, 4)), 4, int(rng.integers(1, 4)), 4, 16, 8
    fmt = O.FMT_INT4 if seed % 2 == 0 else O.FMT_FP4
    key = "int4" if fmt == O.FMT_INT4 else "fp4"
    x, _, w_gu, s_gu, w_d, s_d = _tiny_random(rng, T, E, H, I, G, key)
    wr = S.f32_to_bf16_bits(rng.normal(0.0, 0.5, size=(H, E)))
    out, ids, w, lg = O.moe_layer_from_hidden(x, wr, k, w_gu, s_gu, w_d, s_d, G, fmt)
    blg = BF.router_exact(x.tolist(), wr.tolist())
    bout, bids, bw = BF.moe_exact(x.tolist(), blg, k, w_gu.tolist(), s_gu.tolist(),
                                  w_d.tolist(), s_d.tolist(), G, key)
    assert ids.tolist() == bids
    np.testing.assert_allclose(w, bw, rtol=1e-13)
    scale = max(1e-300, float(np.sqrt(np.mean(np.square(bout)))))
    assert np.max(np.abs(out - np.array(bout))) <= 1e-12 * scale + 1e-300


def test_expert_permutation_invariance():
    cfg = S.TINY
    L = S.make_moe_layer(cfg, seed=7)
    rng = np.random.default_rng(11)
    x = S.f32_to_bf16_bits(rng.standard_normal((3, cfg.H)))
    lg = rng.standard_normal((3, cfg.E)).astype(np.float32)
    out, _, _ = O.moe_layer(x, lg, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group, cfg.fmt)
    p = rng.permutation(cfg.E)
    # expert p[i] moves to slot i (buffers and logit columns together)
    out2, _, _ = O.moe_layer(x, lg[:, p], cfg.k, L.w_gu[p], L.s_gu[p], L.w_d[p], L.s_d[p],
                             cfg.group, cfg.fmt)
    np.testing.assert_allclose(out2, out, rtol=1e-13, atol=1e-15)


def test_power_of_two_down_scale_scales_output_exactly():
    cfg = S.TINY
    L = S.make_moe_layer(cfg, seed=8)
    x, lg = L.x, L.logits
    out, _, _ = O.moe_layer(x, lg, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group, cfg.fmt)
    s_d2 = (L.s_d.astype(np.int32) + (3 << 7)).astype(np.uint16)  # exponent + 3 => x8
    out2, _, _ = O.moe_layer(x, lg, cfg.k, L.w_gu, L.s_gu, L.w_d, s_d2, cfg.group, cfg.fmt)
    assert np.array_equal(out2, 8.0 * out)


def test_k_equals_E_with_equal_logits_is_mean_of_experts():
    cfg = S.replace(S.TINY, E=4, k=4)
    L = S.make_moe_layer(cfg, seed=12)
    lg = np.zeros((1, 4), np.float32)
    out, ids, w = O.moe_layer(L.x, lg, 4, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group, cfg.fmt)
    assert ids.tolist() == [[0, 1, 2, 3]] and np.all(w == 0.25)
    each = [O.moe_layer(L.x, np.eye(4, dtype=np.float32)[e:e + 1] * 50, 1, L.w_gu, L.s_gu,
                        L.w_d, L.s_d, cfg.group, cfg.fmt)[0] for e in range(4)]
    np.testing.assert_allclose(out, np.mean(each, axis=0), rtol=1e-13, atol=1e-15)


def test_duplicated_experts_tied_logits_pick_lower_index():
    cfg = S.replace(S.TINY, E=4, k=1)
    L = S.make_moe_layer(cfg, seed=13)
    for a in (L.w_gu, L.s_gu, L.w_d, L.s_d):
        a[3] = a[1]
    lg = np.array([[0.0, 1.0, -1.0, 1.0]], np.float32)
    out, ids, _ = O.moe_layer(L.x, lg, 1, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group, cfg.fmt)
    assert ids.tolist() == [[1]]


def test_residual_is_added_once():
    cfg = S.TINY
    L = S.make_moe_layer(cfg, seed=14)
    res = S.f32_to_bf16_bits(np.random.default_rng(2).standard_normal((1, cfg.H)))
    a, _, _ = O.moe_layer(L.x, L.logits, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group, cfg.fmt)
    b, _, _ = O.moe_layer(L.x, L.logits, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group,
                          cfg.fmt, residual_bits=res)
    np.testing.assert_allclose(b - a, S.bf16_bits_view_f32(res).astype(np.float64),
                               rtol=0, atol=1e-12)


def test_stack_chains_through_bf16_residual():
    cfg = S.replace(S.W512, E=6, H=64, I=32, k=2, layers=3)
    layers = [S.make_moe_layer(cfg, seed=0, layer=l) for l in range(3)]
    x0 = layers[0].x
    last_in, out = O.moe_stack(x0, layers, cfg.k, cfg.group, cfg.fmt)
    x = x0
    for L in layers:
        o, _, _ = O.moe_layer(x, L.logits, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group,
                              cfg.fmt, residual_bits=x)
        xin, x = x, O.bf16_round_to_bits(o)
    assert np.array_equal(last_in, xin)
    assert np.array_equal(out, o)
    assert not np.array_equal(last_in, x0)


@pytest.mark.parametrize("fmt", [O.FMT_FP4, O.FMT_INT4])
def test_stack_matches_exact_rational_chain(fmt):
    """moe_stack against an exact-rational 3-layer chain: brute-force layers (Fraction gate,
    up and down sums, float64 SiLU and combine) joined by an exact bf16 round-to-nearest-even
    written from the format's definition.  The bf16 inputs of every layer must agree
    bit for bit, the last output to float64 rounding."""
    cfg = S.replace(S.W512, E=4, H=64, I=32, k=2, T=2, layers=3, fmt=fmt)
    layers = [S.make_moe_layer(cfg, seed=0, layer=l) for l in range(3)]
    name = "fp4" if fmt == O.FMT_FP4 else "int4"
    x0 = layers[0].x
    b_in, b_out = BF.moe_stack_exact(x0.tolist(), layers, cfg.k, cfg.group, name)
    o_in, o_out = O.moe_stack(x0, layers, cfg.k, cfg.group, fmt)
    assert np.array_equal(np.asarray(b_in, np.uint16), o_in)
    assert not np.array_equal(o_in, x0)                      # the chain moved
    np.testing.assert_allclose(o_out, np.asarray(b_out), rtol=1e-12, atol=1e-12)


def test_bf16_rne_bits_against_hand_values():
    """The brute-force rounding on values whose bf16 neighbours are known by hand."""
    assert BF.bf16_rne_bits(1.0) == 0x3F80
    assert BF.bf16_rne_bits(1.0 + 2 ** -8) == 0x3F80           # tie -> even (mantissa 0)
    assert BF.bf16_rne_bits(1.0 + 3 * 2 ** -8) == 0x3F82       # tie -> even (mantissa 2)
    assert BF.bf16_rne_bits(1.0 + 2 ** -8 + 2 ** -20) == 0x3F81
    assert BF.bf16_rne_bits(-2.0) == 0xC000
    assert BF.bf16_rne_bits(255.5) == 0x4380                   # 255.5 -> 256 (carry)
    assert BF.bf16_rne_bits(-0.0) == 0x8000
    assert BF.bf16_rne_bits(2.0 ** -130) == 0x0008             # subnormal: 2^-130 = 8 * 2^-133


# --------------------------------------------------------------------------------------
# dense GEMV
# --------------------------------------------------------------------------------------
def test_gemv_one_hot_rows_are_dequantized_rows():
    rng = np.random.default_rng(21)
    K, N, G = 256, 48, 128
    w, s = S.random_packed(rng, K, N, G)
    codes = np.zeros((K, N), np.uint8)
    codes[0::2] = w & 0xF
    codes[1::2] = w >> 4
    tab = BF.golden_tables()["int4"]
    sval = S.bf16_bits_view_f32(s).astype(np.float64)
    for k in (0, 1, 127, 128, 129, 255):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = 0x3F80  # 1.0
        y = O.packed_gemv(x, w, s, G)
        want = np.array([float(tab[codes[k, n]]) * sval[k // G, n] for n in range(N)])
        assert np.array_equal(y[0], want), k


def test_gemv_constant_code_gives_sum_of_x():
    K, N, G = 512, 16, 128
    w = np.full((K // 2, N), 0x99, np.uint8)  # both nibbles 9 -> value 1
    s = np.full((K // G, N), 0x3F80, np.uint16)
    x = S.f32_to_bf16_bits(np.random.default_rng(22).standard_normal((2, K)))
    y = O.packed_gemv(x, w, s, G)
    xs = S.bf16_bits_view_f32(x).astype(np.float64)
    for t in range(2):
        assert np.allclose(y[t], math.fsum(xs[t]), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("seed", range(3))
def test_gemv_matches_exact_bruteforce(seed):
    rng = np.random.default_rng(30 + seed)
    T, K, N, G = 2, 16, 6, 8
    w, s = S.random_packed(rng, K, N, G, 0.1, 1.0)
    x = S.f32_to_bf16_bits(rng.standard_normal((T, K)))
    y = O.packed_gemv(x, w, s, G)
    yb = np.array(BF.gemv_exact(x.tolist(), w.tolist(), s.tolist(), G))
    np.testing.assert_allclose(y, yb, rtol=1e-13, atol=1e-15)


def test_quantizer_roundtrip_within_half_step():
    cfg = S.GemvConfig("q", T=1, K=512, N=64)
    rng = np.random.default_rng(0)
    wf = rng.normal(0, 0.02, size=(cfg.K, cfg.N)).astype(np.float32)
    codes, s = S.quantize_int4_groups(wf, cfg.group)
    W = O.dequant(S.pack_nibbles(codes), s, cfg.group, O.FMT_INT4)
    step = np.repeat(S.bf16_bits_view_f32(s).astype(np.float64), cfg.group, axis=0)
    assert np.all(np.abs(W - wf) <= 0.5 * step * 1.01 + 1e-12)
