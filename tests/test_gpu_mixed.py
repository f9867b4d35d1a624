"""GPU parity: layers whose experts mix FP4 (hot), FE-XC and INT2 (cold) weights, through
moe_fp4_layer_mixed -- the single-launch layer and the multi-launch expert kernels (2-bit
tiles on the vector-ALU and matrix-core bodies) -- against the float64 oracle with the same
per-expert formats (ids exact; output within |diff| <= 1e-2 rms + 1 bf16 ulp)."""
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


def _mixed(cfg, seed):
    lg = S.moe_layer_logits(cfg, seed)
    ids, _ = O.topk_route(lg, cfg.k)
    L = S.make_moe_layer(cfg, seed, experts=np.unique(ids))
    return L, upload_layer(L, np.unique(ids))


def _run(cfg, L, D, efmt, res=None, ws=None, flags=0):
    B = _b()
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    cb = None if L.codebooks is None else dev(L.codebooks)
    out = B.moe_fp4_layer_mixed(dev(L.x), dev(L.logits), cfg.k, D["w_gu"], D["s_gu"], D["w_d"],
                                D["s_d"], dev(efmt), cfg.group, codebooks=cb,
                                residual=None if res is None else dev(res).view(torch.bfloat16),
                                ids_out=ids, weights_out=w, workspace=ws, flags=flags)
    torch.cuda.synchronize()
    return bits16(out), ids.cpu().numpy(), w.cpu().numpy()


CASES = [("q30_half_int2", S.Q30_MIXED, 1, 0), ("q30_half_int2", S.Q30_MIXED, 1, 1),
         ("q30_half_int2", S.Q30_MIXED, 2, 0), ("q30_half_int2", S.Q30_MIXED, 4, 2),
         ("q30_half_int2", S.Q30_MIXED, 8, 3), ("q30_all_int2", S.replace(S.Q30, int2_frac=1.0), 1, 0),
         ("w512_quarter_int2", S.replace(S.W512, layers=1, int2_frac=0.25), 1, 0),
         ("w512_quarter_int2", S.replace(S.W512, layers=1, int2_frac=0.25), 4, 1),
         ("q30_codebook", S.Q30_CODEBOOK, 1, 0), ("q30_codebook", S.Q30_CODEBOOK, 1, 1),
         ("q30_codebook", S.Q30_CODEBOOK, 2, 2), ("q30_codebook", S.Q30_CODEBOOK, 4, 3),
         ("q30_codebook", S.Q30_CODEBOOK, 8, 4), ("q30_all_fexc", S.replace(S.Q30, fexc_frac=1.0), 1, 0),
         ("w512_codebook", S.replace(S.W512, layers=1, int2_frac=0.2, fexc_frac=0.3), 1, 2)]


@pytest.mark.parametrize("name,cfg,T,seed", CASES, ids=[f"{c[0]}-T{c[2]}-s{c[3]}" for c in CASES])
def test_mixed_layer_parity(name, cfg, T, seed):
    cfg = cfg.with_T(T)
    L, D = _mixed(cfg, seed)
    assert L.expert_fmt is not None
    res = S.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal((T, cfg.H))) \
        if seed % 2 else None
    out, ids, w = _run(cfg, L, D, L.expert_fmt, res)
    want, oids, ow = O.moe_layer(L.x, L.logits, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group,
                                 cfg.fmt, residual_bits=res, expert_fmt=L.expert_fmt,
                                 codebooks=L.codebooks)
    assert np.array_equal(ids, oids)
    np.testing.assert_allclose(w, ow, rtol=4e-6, atol=1e-7)
    routed = L.expert_fmt[np.unique(oids)]
    assert cfg.int2_frac == 0 or np.any(routed == O.FMT_INT2), "no INT2 expert routed"
    assert cfg.fexc_frac == 0 or np.any(routed == O.FMT_FEXC), "no FE-XC expert routed"
    check_bf16(out, want, what=f"{name} T={T}")


@pytest.mark.parametrize("name,base,T", [("q30", S.Q30_BATCH, 1), ("q30", S.Q30_BATCH, 4),
                                         ("q30", S.Q30_BATCH, 16), ("q30", S.Q30_BATCH, 64),
                                         ("w512", S.replace(S.W512, layers=1), 1),
                                         ("w512", S.replace(S.W512, layers=1), 8)])
def test_all_fp4_table_equals_the_fp4_layer(name, base, T):
    """With no INT2 entry the mixed call runs exactly the FP4 arithmetic: bitwise equal to
    moe_fp4_layer on the same inputs (ids and weights too).  The two calls run different
    instances of the kernel: the mixed one with the format-table paths, the plain one with
    them compiled out."""
    B = _b()
    cfg = base.with_T(T)
    L, D = _mixed(cfg, 21)
    table = np.full(cfg.E, S.FMT_FP4, np.uint8)
    got, gids, gw = _run(cfg, L, D, table)
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    ref = B.moe_fp4_layer(dev(L.x), dev(L.logits), cfg.k, D["w_gu"], D["s_gu"], D["w_d"],
                          D["s_d"], cfg.group, cfg.fmt, ids_out=ids, weights_out=w)
    torch.cuda.synchronize()
    assert np.array_equal(got, bits16(ref))
    assert np.array_equal(gids, ids.cpu().numpy())
    assert np.array_equal(gw.view(np.uint32), w.cpu().numpy().view(np.uint32))


def test_mixed_and_plain_calls_share_a_workspace():
    """Mixed and plain FP4 calls alternate on one workspace (same exchange regions): each call
    reproduces its first result bit for bit."""
    B = _b()
    cfgm = S.Q30_MIXED
    Lm, Dm = _mixed(cfgm, 5)
    cfgp = S.Q30
    Lp, Dp = _mixed(cfgp, 6)
    ws = B.moe_workspace(1, 2048, 768, 128, 8, "cuda")

    def plain():
        o = B.moe_fp4_layer(dev(Lp.x), dev(Lp.logits), 8, Dp["w_gu"], Dp["s_gu"], Dp["w_d"],
                            Dp["s_d"], 32, cfgp.fmt, workspace=ws)
        return bits16(o)

    first_m = _run(cfgm, Lm, Dm, Lm.expert_fmt, ws=ws)[0]
    first_p = plain()
    for _ in range(3):
        assert np.array_equal(_run(cfgm, Lm, Dm, Lm.expert_fmt, ws=ws)[0], first_m)
        assert np.array_equal(plain(), first_p)
    assert int(ws[:4].view(torch.int32).item()) == 0


# ---- the multi-launch expert kernels: 2-bit tiles ----------------------------------------
def _oracle(cfg, L, res=None):
    return O.moe_layer(L.x, L.logits, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group, cfg.fmt,
                       residual_bits=res, expert_fmt=L.expert_fmt, codebooks=L.codebooks)


def _flags(path):
    B = _b()
    return {"auto": 0, "gemv": B.PATH_FORCE_GEMV, "mfma": B.PATH_FORCE_MFMA,
            "unfused": B.PATH_NO_FUSED}[path]


def _routed_formats(cfg, L, oids):
    routed = L.expert_fmt[np.unique(oids)]
    assert cfg.int2_frac == 0 or np.any(routed == O.FMT_INT2), "no INT2 expert routed"
    assert cfg.fexc_frac == 0 or np.any(routed == O.FMT_FEXC), "no FE-XC expert routed"


BATCH_MIXED = S.replace(S.Q30_MIXED, logits="normal+bias")
BATCH_CODEBOOK = S.replace(S.Q30_CODEBOOK, logits="normal+bias")
MULTI_CASES = [("q30_half_int2", BATCH_MIXED, 16, "auto"), ("q30_half_int2", BATCH_MIXED, 16, "gemv"),
               ("q30_half_int2", BATCH_MIXED, 16, "mfma"), ("q30_half_int2", BATCH_MIXED, 64, "auto"),
               ("q30_codebook", BATCH_CODEBOOK, 16, "auto"), ("q30_codebook", BATCH_CODEBOOK, 16, "gemv"),
               ("q30_codebook", BATCH_CODEBOOK, 16, "mfma"), ("q30_codebook", BATCH_CODEBOOK, 64, "auto"),
               ("q30_codebook", BATCH_CODEBOOK, 64, "mfma"),
               ("q30_codebook", BATCH_CODEBOOK, 1, "unfused"), ("q30_codebook", BATCH_CODEBOOK, 4, "unfused")]


@pytest.mark.parametrize("name,cfg,T,path", MULTI_CASES,
                         ids=[f"{c[0]}-T{c[2]}-{c[3]}" for c in MULTI_CASES])
def test_mixed_multi_launch_parity(name, cfg, T, path):
    """T > 8 (or DQG_PATH_NO_FUSED) on the multi-launch kernels: by token count (auto), every
    expert on the vector-ALU tiles (gemv), every expert on the matrix-core tiles (mfma)."""
    cfg = cfg.with_T(T)
    L, D = _mixed(cfg, T)
    res = S.f32_to_bf16_bits(np.random.default_rng(T).standard_normal((T, cfg.H))) \
        if path == "auto" else None
    out, ids, _ = _run(cfg, L, D, L.expert_fmt, res, flags=_flags(path))
    want, oids, _ = _oracle(cfg, L, res)
    assert np.array_equal(ids, oids)
    _routed_formats(cfg, L, oids)
    check_bf16(out, want, what=f"{name} T={T} {path}")


@pytest.mark.parametrize("T", [16, 40])
def test_hot_2bit_experts_take_the_mfma_tiles(T):
    """An INT2 and an FE-XC expert that every token picks run the matrix-core body in
    passes of 16 by default; then everything on the vector-ALU body."""
    cfg = BATCH_CODEBOOK.with_T(T)
    seed = 3
    efmt = S.expert_formats(cfg, seed)
    hot2 = int(np.flatnonzero(efmt == S.FMT_INT2)[0])
    hotx = int(np.flatnonzero(efmt == S.FMT_FEXC)[0])
    L0 = S.make_moe_layer(cfg, seed, experts=[])
    lg = L0.logits.copy()
    lg[:, hot2] += np.float32(12.0)
    lg[:, hotx] += np.float32(12.0)
    ids, _ = O.topk_route(lg, cfg.k)
    L = S.make_moe_layer(cfg, seed, experts=np.unique(ids))
    L.logits = lg
    D = upload_layer(L, np.unique(ids))
    want, oids, _ = _oracle(cfg, L)
    assert np.all(np.sort(oids[:, :2], axis=1) == sorted((hot2, hotx)))
    for path in ("auto", "gemv"):
        out, gids, _ = _run(cfg, L, D, L.expert_fmt, flags=_flags(path))
        assert np.array_equal(gids, oids)
        check_bf16(out, want, what=f"hot 2-bit T={T} {path}")


SMALL_CODEBOOK = S.MoEConfig("small_codebook", T=6, E=8, H=256, I=192, k=2, fmt=S.FMT_FP4,
                             group=32, scale_lo=0.005, scale_hi=0.02, int2_frac=0.25,
                             fexc_frac=0.25)


@pytest.mark.parametrize("path", ["auto", "gemv", "mfma"])
def test_codebooks_with_small_intermediate(path):
    """FE-XC with I = 192 < 512 (beyond the single launch's codebook staging) on the
    multi-launch kernels, with a half-full last column tile."""
    cfg = SMALL_CODEBOOK
    L = S.make_moe_layer(cfg, 8)
    D = upload_layer(L)
    out, ids, _ = _run(cfg, L, D, L.expert_fmt, flags=_flags(path))
    want, oids, _ = _oracle(cfg, L)
    assert np.array_equal(ids, oids)
    _routed_formats(cfg, L, oids)
    check_bf16(out, want, what=f"small codebook {path}")
