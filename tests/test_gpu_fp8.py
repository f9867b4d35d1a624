"""GPU parity: FP8 E4M3 weights (one code per byte) through the single-launch layer and the
multi-launch expert kernels (vector-ALU and matrix-core bodies).

The decode is compared bit for bit (every finite code), the layer per element against the
float64 oracle with the method's tolerance (|gpu - oracle| <= 1e-2 rms + 1 bf16 ulp), the
routing exactly."""
import numpy as np
import pytest
import torch

from gpu_util import bits16, check_bf16, dev, upload_layer
from oracle import moe_oracle as O
from workloads import synth as S

pytestmark = pytest.mark.gpu


def _b():
    from dequant_gemv_amd import binding
    return binding


def test_fp8_dequant_bit_exact_every_finite_code():
    B = _b()
    rng = np.random.default_rng(0)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    K, N, G = 256, 254, 32
    codes = np.stack([np.roll(finite, r) for r in range(K)]).astype(np.uint8)     # [K, N]
    Np = 256  # pad N to a multiple of 16 with zero codes
    w = np.zeros((K, Np), np.uint8)
    w[:, :N] = codes
    s = S.f32_to_bf16_bits(rng.uniform(0.001, 4.0, size=(K // G, Np)))
    got = B.packed_dequant_f32(dev(w), dev(s), G, B.FMT_FP8_E4M3).cpu().numpy()
    want = O.dequant(w, s, G, O.FMT_FP8).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _fp8_layer(T, seed, residual=False):
    cfg = S.Q30_FP8.with_T(T)
    lg = S.moe_layer_logits(cfg, seed)
    ids, _ = O.topk_route(lg, cfg.k)
    L = S.make_moe_layer(cfg, seed, experts=np.unique(ids))
    D = upload_layer(L, np.unique(ids))
    res = S.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal((T, cfg.H))) \
        if residual else None
    return cfg, L, D, res


@pytest.mark.parametrize("T,seed,residual", [(1, 0, False), (1, 1, True), (2, 0, False),
                                             (4, 2, True), (8, 3, False)])
def test_fp8_layer_parity(T, seed, residual):
    B = _b()
    cfg, L, D, res = _fp8_layer(T, seed, residual)
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    out = B.moe_fp4_layer(dev(L.x), dev(L.logits), cfg.k, D["w_gu"], D["s_gu"], D["w_d"],
                          D["s_d"], cfg.group, cfg.fmt,
                          residual=None if res is None else dev(res).view(torch.bfloat16),
                          ids_out=ids, weights_out=w)
    torch.cuda.synchronize()
    want, oids, ow = O.moe_layer(L.x, L.logits, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group,
                                 cfg.fmt, residual_bits=res)
    assert np.array_equal(ids.cpu().numpy(), oids)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=4e-6, atol=1e-7)
    check_bf16(bits16(out), want, what=f"fp8 T={T}")


def test_fp8_layer_from_hidden():
    """The router inside the single launch with FP8 experts."""
    B = _b()
    cfg = S.Q30_FP8
    wr = S.make_router_weights(cfg.H, cfg.E, seed=4)
    L0 = S.make_moe_layer(cfg, 4, experts=[])
    ids, _ = O.topk_route(O.router_logits(L0.x, wr), cfg.k, dtype=np.float64)
    L = S.make_moe_layer(cfg, 4, experts=np.unique(ids))
    D = upload_layer(L, np.unique(ids))
    gids = torch.empty((1, cfg.k), dtype=torch.int32, device="cuda")
    out = B.moe_fp4_layer_from_hidden(dev(L.x), dev(wr), cfg.k, D["w_gu"], D["s_gu"], D["w_d"],
                                      D["s_d"], cfg.group, cfg.fmt, ids_out=gids)
    torch.cuda.synchronize()
    want, oids, _, _ = O.moe_layer_from_hidden(L.x, wr, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d,
                                               cfg.group, cfg.fmt)
    assert np.array_equal(gids.cpu().numpy(), oids)
    check_bf16(bits16(out), want, what="fp8 from hidden")


def test_formats_alternate_on_one_workspace():
    """FP4, FP8 and INT4 single-launch calls at T = 1 and 4 on one workspace (FP8 has its own
    exchange regions): every call reproduces its first result bit for bit."""
    B = _b()
    cases = {}
    for name, base in (("fp4", S.Q30), ("fp8", S.Q30_FP8),
                       ("int4", S.replace(S.Q30, fmt=S.FMT_INT4))):
        for T in (1, 4):
            cfg = base.with_T(T)
            lg = S.moe_layer_logits(cfg, 9)
            ids, _ = O.topk_route(lg, cfg.k)
            L = S.make_moe_layer(cfg, 9, experts=np.unique(ids))
            cases[(name, T)] = (cfg, L, upload_layer(L, np.unique(ids)))
    ws = B.moe_workspace(4, 2048, 768, 128, 8, "cuda")

    def run(key):
        cfg, L, D = cases[key]
        return bits16(B.moe_fp4_layer(dev(L.x), dev(L.logits), cfg.k, D["w_gu"], D["s_gu"],
                                      D["w_d"], D["s_d"], cfg.group, cfg.fmt, workspace=ws))

    order = [("fp4", 1), ("fp8", 1), ("fp8", 4), ("int4", 1), ("fp4", 4), ("fp8", 1),
             ("int4", 4), ("fp4", 1), ("fp8", 4), ("fp8", 1), ("fp4", 4), ("int4", 1)]
    first = {}
    for key in order:
        got = run(key)
        if key in first:
            assert np.array_equal(got, first[key]), key
        else:
            first[key] = got
    assert int(ws[:4].view(torch.int32).item()) == 0
    cfg, L, _ = cases[("fp8", 4)]
    want, _, _ = O.moe_layer(L.x, L.logits, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group,
                             cfg.fmt)
    check_bf16(first[("fp8", 4)], want, what="fp8 T=4 on the shared workspace")


@pytest.mark.parametrize("T", [1, 8])
def test_fp8_layer_w512_shape(T):
    """FP8 weights at the 512-expert shape (k = 10, I = 512, skewed routing), T = 1 and 8."""
    B = _b()
    cfg = S.replace(S.W512, layers=1, fmt=S.FMT_FP8).with_T(T)
    lg = S.moe_layer_logits(cfg, 5)
    ids, _ = O.topk_route(lg, cfg.k)
    L = S.make_moe_layer(cfg, 5, experts=np.unique(ids))
    D = upload_layer(L, np.unique(ids))
    gids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    out = B.moe_fp4_layer(dev(L.x), dev(L.logits), cfg.k, D["w_gu"], D["s_gu"], D["w_d"],
                          D["s_d"], cfg.group, cfg.fmt, ids_out=gids)
    torch.cuda.synchronize()
    want, oids, _ = O.moe_layer(L.x, L.logits, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group,
                                cfg.fmt)
    assert np.array_equal(gids.cpu().numpy(), oids)
    check_bf16(bits16(out), want, what=f"fp8 w512 T={T}")


# ---- the multi-launch expert kernels (T > 8, or DQG_PATH_NO_FUSED) ----------------------------
FP8_BATCH = S.replace(S.Q30_BATCH, fmt=S.FMT_FP8)
FP8_ODD = S.MoEConfig("fp8_odd", T=5, E=8, H=320, I=192, k=2, fmt=S.FMT_FP8, group=32,
                      scale_lo=0.005, scale_hi=0.02)


def _routed(cfg, seed, hot=None):
    """A layer with only its routed experts drawn; `hot` favours one expert for every token."""
    L = S.make_moe_layer(cfg, seed, experts=[])
    lg = L.logits.copy()
    if hot is not None:
        lg[:, hot] += np.float32(12.0)
    ids, _ = O.topk_route(lg, cfg.k)
    L = S.make_moe_layer(cfg, seed, experts=np.unique(ids))
    L.logits = lg
    return L, upload_layer(L, np.unique(ids))


def _flags(B, path):
    return {"auto": 0, "gemv": B.PATH_FORCE_GEMV, "mfma": B.PATH_FORCE_MFMA,
            "unfused": B.PATH_NO_FUSED}[path]


def _layer_out(B, cfg, L, D, flags=0):
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    out = B.moe_fp4_layer(dev(L.x), dev(L.logits), cfg.k, D["w_gu"], D["s_gu"], D["w_d"],
                          D["s_d"], cfg.group, cfg.fmt, ids_out=ids, flags=flags)
    torch.cuda.synchronize()
    return bits16(out), ids.cpu().numpy()


@pytest.mark.parametrize("T", [16, 64])
@pytest.mark.parametrize("path", ["auto", "gemv", "mfma"])
def test_fp8_multi_launch_parity(T, path):
    """T = 16 and 64 on the multi-launch kernels: by token count (auto), every expert on the
    vector-ALU tiles (gemv), every expert on the matrix-core tiles (mfma)."""
    B = _b()
    cfg = FP8_BATCH.with_T(T)
    L, D = _routed(cfg, seed=T)
    want, oids, _ = O.moe_layer(L.x, L.logits, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group,
                                cfg.fmt)
    out, ids = _layer_out(B, cfg, L, D, _flags(B, path))
    assert np.array_equal(ids, oids)
    check_bf16(out, want, what=f"fp8 T={T} {path}")


@pytest.mark.parametrize("T", [40, 64])
def test_fp8_hot_expert_takes_the_mfma_tiles(T):
    """One expert with every token runs the matrix-core body in passes of 16, single-token
    experts the vector-ALU body, in the same launches; then all on the vector-ALU body."""
    B = _b()
    cfg = FP8_BATCH.with_T(T)
    L, D = _routed(cfg, seed=T + 1, hot=5)
    want, oids, _ = O.moe_layer(L.x, L.logits, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group,
                                cfg.fmt)
    assert np.all(oids[:, 0] == 5)
    for path in ("auto", "gemv"):
        out, ids = _layer_out(B, cfg, L, D, _flags(B, path))
        assert np.array_equal(ids, oids)
        check_bf16(out, want, what=f"fp8 hot T={T} {path}")


@pytest.mark.parametrize("T", [1, 4])
def test_fp8_small_batch_off_the_single_launch(T):
    """DQG_PATH_NO_FUSED sends T <= 8 to the multi-launch kernels."""
    B = _b()
    cfg, L, D, _ = _fp8_layer(T, seed=7)
    want, oids, _ = O.moe_layer(L.x, L.logits, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group,
                                cfg.fmt)
    out, ids = _layer_out(B, cfg, L, D, B.PATH_NO_FUSED)
    assert np.array_equal(ids, oids)
    check_bf16(out, want, what=f"fp8 unfused T={T}")


@pytest.mark.parametrize("path", ["auto", "gemv", "mfma"])
def test_fp8_tiles_with_64_column_tails(path):
    """H = 320, I = 192: the last column tile of each projection is half full."""
    B = _b()
    L = S.make_moe_layer(FP8_ODD, 4)
    D = upload_layer(L)
    want, _, _ = O.moe_layer(L.x, L.logits, FP8_ODD.k, L.w_gu, L.s_gu, L.w_d, L.s_d,
                             FP8_ODD.group, FP8_ODD.fmt)
    out, _ = _layer_out(B, FP8_ODD, L, D, _flags(B, path) | B.PATH_NO_FUSED)
    check_bf16(out, want, what=f"fp8 odd {path}")


@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_fp8_group_128(path):
    """Scale groups of 128 K indices (4 blocks share a scale row)."""
    B = _b()
    cfg = S.replace(FP8_BATCH.with_T(16), group=128)
    L, D = _routed(cfg, seed=9)
    want, _, _ = O.moe_layer(L.x, L.logits, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group,
                             cfg.fmt)
    out, _ = _layer_out(B, cfg, L, D, _flags(B, path))
    check_bf16(out, want, what=f"fp8 G=128 {path}")


def test_fp8_ffn_given_routing_with_residual():
    """moe_fp4_ffn with FP8 weights and a given routing (duplicates across tokens)."""
    B = _b()
    cfg = FP8_BATCH.with_T(16)
    rng = np.random.default_rng(6)
    ids, wts = S.make_routing(rng, cfg.T, cfg.E, cfg.k)
    L = S.make_moe_layer(cfg, 5, experts=np.unique(ids))
    D = upload_layer(L, np.unique(ids))
    res = S.f32_to_bf16_bits(rng.standard_normal((cfg.T, cfg.H)))
    out = B.moe_fp4_ffn(dev(L.x), dev(ids), dev(wts), D["w_gu"], D["s_gu"], D["w_d"], D["s_d"],
                        cfg.group, cfg.fmt, residual=dev(res))
    torch.cuda.synchronize()
    want = O.moe_ffn(L.x, ids, wts.astype(np.float64), L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group,
                     cfg.fmt, residual_bits=res)
    check_bf16(bits16(out), want, what="fp8 ffn+residual")


def test_fp8_from_hidden_multi_launch():
    """Router call, then the FP8 layer on the multi-launch kernels (T = 16)."""
    B = _b()
    cfg = FP8_BATCH.with_T(16)
    wr = S.make_router_weights(cfg.H, cfg.E, seed=4)
    L0 = S.make_moe_layer(cfg, 4, experts=[])
    ids, _ = O.topk_route(O.router_logits(L0.x, wr), cfg.k, dtype=np.float64)
    L = S.make_moe_layer(cfg, 4, experts=np.unique(ids))
    D = upload_layer(L, np.unique(ids))
    gids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    out = B.moe_fp4_layer_from_hidden(dev(L.x), dev(wr), cfg.k, D["w_gu"], D["s_gu"], D["w_d"],
                                      D["s_d"], cfg.group, cfg.fmt, ids_out=gids)
    torch.cuda.synchronize()
    want, oids, _, _ = O.moe_layer_from_hidden(L.x, wr, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d,
                                               cfg.group, cfg.fmt)
    check_bf16(bits16(out), want, what="fp8 from hidden T=16")
