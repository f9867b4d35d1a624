"""GPU parity: the router on the hidden state (router_logits) and the layer that routes from
the hidden state (moe_fp4_layer_from_hidden), through the single launch and the separate
router call.

The GPU computes the logits in fp32 (a fixed order of fma and sums), the oracle in float64.
Per logit the test allows |gpu - oracle| <= 2^-17 * sum_c |x_c W_r[c, e]|, about 40 fp32
roundings of the largest partial (the kernel's chain is 8 fma, then 16 and at most 16
ordered adds).  Expert ids are compared exactly where the oracle's k+1 largest logits are
separated by more than twice that bound (asserted, so a seed that gives a near tie fails
loudly instead of passing on luck)."""
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


def _bound(x_bits, wr_bits):
    mag = np.abs(S.bf16_bits_view_f32(x_bits).astype(np.float64)) @ \
        np.abs(S.bf16_bits_view_f32(wr_bits).astype(np.float64))
    return 2.0 ** -17 * mag


def _check_logits(gpu, want, bound, what):
    err = np.abs(gpu.astype(np.float64) - want)
    assert np.all(err <= bound), f"{what}: worst logit error {err.max()!r}, bound {bound.min()!r}"


def _assert_margin(want, bound, k, what):
    for t in range(want.shape[0]):
        top = np.sort(want[t])[::-1][: k + 1]
        gap = float(np.min(-np.diff(top))) if top.size > 1 else np.inf
        assert gap > 2.0 * bound[t].max(), f"{what}: token {t} has a near tie; pick another seed"


def _layer(cfg, seed):
    """Generator layer, router weight and device buffers (routed experts only for wide E)."""
    cfg = S.replace(cfg, layers=1)
    wr = S.make_router_weights(cfg.H, cfg.E, seed)
    if cfg.E > 128:
        L = S.make_moe_layer(cfg, seed, experts=[])  # x only (the draw order is unchanged)
        lg = O.router_logits(L.x, wr)
        ids, _ = O.topk_route(lg, cfg.k, dtype=np.float64)
        L = S.make_moe_layer(cfg, seed, experts=np.unique(ids))
        return cfg, L, wr, upload_layer(L, np.unique(ids))
    L = S.make_moe_layer(cfg, seed)
    return cfg, L, wr, upload_layer(L)


ROUTER_CASES = [("tiny", S.TINY, 0), ("q30_t1", S.Q30, 0), ("q30_t3", S.Q30.with_T(3), 1),
                ("q30_t16", S.Q30.with_T(16), 2), ("w512_t1", S.replace(S.W512, layers=1), 0),
                ("w512_t5", S.replace(S.W512, layers=1, T=5), 1)]


@pytest.mark.parametrize("name,cfg,seed", ROUTER_CASES, ids=[c[0] for c in ROUTER_CASES])
def test_router_logits_parity(name, cfg, seed):
    B = _b()
    x = S.f32_to_bf16_bits(np.random.default_rng(50 + seed).standard_normal((cfg.T, cfg.H)))
    wr = S.make_router_weights(cfg.H, cfg.E, seed)
    got = B.router_logits(dev(x), dev(wr))
    torch.cuda.synchronize()
    want = O.router_logits(x, wr)
    _check_logits(got.cpu().numpy(), want, _bound(x, wr), name)


def test_router_logits_one_hot_rows_are_exact():
    """x = one-hot rows picks rows of W_r: every product but one is zero, so the fp32 result
    is exact whatever the order."""
    B = _b()
    H, E = 2048, 128
    wr = S.make_router_weights(H, E, seed=5)
    rows = [0, 1, 127, 128, 1000, 2047]
    x = np.zeros((len(rows), H), np.float32)
    for t, c in enumerate(rows):
        x[t, c] = 1.0
    got = B.router_logits(dev(S.f32_to_bf16_bits(x)), dev(wr)).cpu().numpy()
    want = S.bf16_bits_view_f32(wr)[rows]
    assert np.array_equal(got, want)


FUSED_CASES = [("tiny", S.TINY, 0), ("q30_t1_s0", S.Q30, 0), ("q30_t1_s1", S.Q30, 1),
               ("q30_t2", S.Q30.with_T(2), 0), ("q30_t4", S.Q30.with_T(4), 2)]


@pytest.mark.parametrize("name,cfg,seed", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_layer_from_hidden_parity(name, cfg, seed):
    """Single launch with the router units (E <= 128, T <= 4) against the oracle: logits
    within the bound, ids exact, weights and output within the method's tolerance."""
    B = _b()
    cfg, L, wr, D = _layer(cfg, seed)
    T, E, k = cfg.T, cfg.E, cfg.k
    want, oids, ow, olg = O.moe_layer_from_hidden(L.x, wr, k, L.w_gu, L.s_gu, L.w_d, L.s_d,
                                                  cfg.group, cfg.fmt)
    bound = _bound(L.x, wr)
    _assert_margin(olg, bound, k, name)
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = B.moe_fp4_layer_from_hidden(dev(L.x), dev(wr), k, D["w_gu"], D["s_gu"], D["w_d"],
                                      D["s_d"], cfg.group, cfg.fmt, logits_out=lg, ids_out=ids,
                                      weights_out=w)
    torch.cuda.synchronize()
    _check_logits(lg.cpu().numpy(), olg, bound, name)
    assert np.array_equal(ids.cpu().numpy(), oids), "expert selection must match exactly"
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-5, atol=1e-7)
    check_bf16(bits16(out), want, what=name)


@pytest.mark.parametrize("name,cfg,seed", [("q30_t1", S.Q30, 3), ("q30_t4", S.Q30.with_T(4), 0),
                                           ("tiny", S.TINY, 1)])
def test_single_launch_and_router_call_give_identical_logits(name, cfg, seed):
    """The router inside the single launch and the separate router call (forced by
    PATH_NO_FUSED) add the same partials in the same order: bitwise-identical logits and
    routing; both outputs meet the tolerance."""
    B = _b()
    cfg, L, wr, D = _layer(cfg, seed)
    T, E, k = cfg.T, cfg.E, cfg.k
    want, oids, _, olg = O.moe_layer_from_hidden(L.x, wr, k, L.w_gu, L.s_gu, L.w_d, L.s_d,
                                                 cfg.group, cfg.fmt)
    _assert_margin(olg, _bound(L.x, wr), k, name)
    res = {}
    for path, flags in (("fused", 0), ("separate", B.PATH_NO_FUSED)):
        lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        out = B.moe_fp4_layer_from_hidden(dev(L.x), dev(wr), k, D["w_gu"], D["s_gu"], D["w_d"],
                                          D["s_d"], cfg.group, cfg.fmt, logits_out=lg,
                                          ids_out=ids, flags=flags)
        torch.cuda.synchronize()
        res[path] = (lg.cpu().numpy(), ids.cpu().numpy(), bits16(out))
        check_bf16(res[path][2], want, what=f"{name} {path}")
        assert np.array_equal(res[path][1], oids)
    assert np.array_equal(res["fused"][0].view(np.uint32), res["separate"][0].view(np.uint32))
    # the logits-taking layer on the router call's logits takes the same routing
    direct = B.router_logits(dev(L.x), dev(wr))
    assert np.array_equal(direct.cpu().numpy().view(np.uint32), res["fused"][0].view(np.uint32))


@pytest.mark.parametrize("name,cfg,seed", [("q30_t8", S.Q30.with_T(8), 2),
                                           ("q30_t16", S.Q30.with_T(16), 0),
                                           ("w512_t1", S.replace(S.W512, layers=1), 0),
                                           ("w512_t4", S.replace(S.W512, layers=1, T=4), 1)])
def test_layer_from_hidden_other_paths(name, cfg, seed):
    """Shapes outside the single launch with router units (T > 4, or E > 128): the router
    call, then the layer on its logits (the single launch without router units for T <= 8,
    the multi-launch path beyond)."""
    B = _b()
    cfg, L, wr, D = _layer(cfg, seed)
    T, E, k = cfg.T, cfg.E, cfg.k
    want, oids, ow, olg = O.moe_layer_from_hidden(L.x, wr, k, L.w_gu, L.s_gu, L.w_d, L.s_d,
                                                  cfg.group, cfg.fmt)
    bound = _bound(L.x, wr)
    _assert_margin(olg, bound, k, name)
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = B.moe_fp4_layer_from_hidden(dev(L.x), dev(wr), k, D["w_gu"], D["s_gu"], D["w_d"],
                                      D["s_d"], cfg.group, cfg.fmt, logits_out=lg, ids_out=ids,
                                      weights_out=w)
    torch.cuda.synchronize()
    _check_logits(lg.cpu().numpy(), olg, bound, name)
    assert np.array_equal(ids.cpu().numpy(), oids)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-5, atol=1e-7)
    check_bf16(bits16(out), want, what=name)


def test_router_layer_and_logits_layer_share_a_workspace():
    """Calls with and without router units, at T = 1 and T = 4, alternate on one workspace
    (they share each T's call counter and exchange buffers): every call reproduces its first
    result bit for bit, and the router-less call still reads its own logits."""
    B = _b()
    cfg1, L, wr, D = _layer(S.Q30, 1)
    x4 = S.f32_to_bf16_bits(np.random.default_rng(77).standard_normal((4, cfg1.H)))
    ws = B.moe_workspace(4, cfg1.H, cfg1.I, cfg1.E, cfg1.k, "cuda")
    lgt = dev(L.logits)
    args = (D["w_gu"], D["s_gu"], D["w_d"], D["s_d"], cfg1.group, cfg1.fmt)

    def hidden(x):
        return bits16(B.moe_fp4_layer_from_hidden(dev(x), dev(wr), cfg1.k, *args, workspace=ws))

    def given():
        return bits16(B.moe_fp4_layer(dev(L.x), lgt, cfg1.k, *args, workspace=ws))

    first = {"h1": hidden(L.x), "g1": given(), "h4": hidden(x4)}
    for _ in range(3):
        for key, fn in (("g1", given), ("h4", lambda: hidden(x4)), ("h1", lambda: hidden(L.x))):
            got = fn()
            assert np.array_equal(got, first[key]), key
    err = ws[:4].view(torch.int32).item()
    assert err == 0, f"error word {err}"
    want, _, _ = O.moe_layer(L.x, L.logits, cfg1.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg1.group,
                             cfg1.fmt)
    check_bf16(first["g1"], want, what="logits-given call")


def test_router_rows_after_an_interleaved_logits_call():
    """Router calls, then a logits-taking call, then a router call with another hidden state
    on one workspace: the router rows the last call reads are its own (the router's copies
    alternate with router calls only), so its logits equal the separate router call's."""
    B = _b()
    cfg, L, wr, D = _layer(S.Q30, 4)
    xa = dev(L.x)
    xb_bits = S.f32_to_bf16_bits(np.random.default_rng(123).standard_normal((1, cfg.H)))
    xb = dev(xb_bits)
    ws = B.moe_workspace(1, cfg.H, cfg.I, cfg.E, cfg.k, "cuda")
    args = (D["w_gu"], D["s_gu"], D["w_d"], D["s_d"], cfg.group, cfg.fmt)
    lg = torch.empty((1, cfg.E), dtype=torch.float32, device="cuda")
    want_b = B.router_logits(xb, dev(wr)).cpu().numpy()
    for rep in range(3):
        B.moe_fp4_layer_from_hidden(xa, dev(wr), cfg.k, *args, workspace=ws)
        B.moe_fp4_layer_from_hidden(xa, dev(wr), cfg.k, *args, workspace=ws)
        B.moe_fp4_layer(xa, dev(L.logits), cfg.k, *args, workspace=ws)
        out_b = B.moe_fp4_layer_from_hidden(xb, dev(wr), cfg.k, *args, logits_out=lg,
                                            workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(lg.cpu().numpy().view(np.uint32), want_b.view(np.uint32)), rep
    want, _, _, _ = O.moe_layer_from_hidden(xb_bits, wr, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d,
                                            cfg.group, cfg.fmt)
    check_bf16(bits16(out_b), want, what="router call after a logits call")
    assert int(ws[:4].view(torch.int32).item()) == 0
