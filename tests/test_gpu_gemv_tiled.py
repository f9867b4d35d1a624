"""GPU parity: the prepacked dense INT4 GEMV (packed_gemv_int4_prepack + packed_gemv_int4_tiled)
against the oracle, and the prepacked bytes against the layout the header defines."""
import numpy as np
import pytest
import torch

from gpu_util import bits16, check_bf16, dev, guarded, guarded_workspace
from oracle import moe_oracle as O
from workloads import synth as S
from prepack_layout import layout_s, layout_w

pytestmark = pytest.mark.gpu


def _b():
    from dequant_gemv_amd import binding
    return binding


def _prepack(g):
    B = _b()
    return B.packed_gemv_int4_prepack(dev(g.w), dev(g.s), g.cfg.group)


def _run(g, wt=None, st=None, use_ws=True):
    """One prepacked call with y and the workspace inside canary bands; the workspace's error
    word must stay zero."""
    B = _b()
    cfg = g.cfg
    if wt is None:
        wt, st = _prepack(g)
    x = dev(g.x)
    y, chk_y = guarded((cfg.T, cfg.N), torch.bfloat16)
    n = B.packed_gemv_int4_workspace_bytes(cfg.T, cfg.K, cfg.N, cfg.group) if use_ws else 0
    ws, chk_ws = (guarded_workspace(n) if n else (None, None))
    B.packed_gemv_int4_tiled(x, wt, st, cfg.N, cfg.group, y=y, workspace=ws)
    torch.cuda.synchronize()
    chk_y()
    if ws is not None:
        chk_ws()
        assert int(ws[:4].view(torch.int32).item()) == 0
    return bits16(y)


def _oracle_blocks(g, block=4096):
    N = g.cfg.N
    return np.concatenate([O.packed_gemv(g.x, g.w, g.s, g.cfg.group,
                                         cols=np.arange(c, min(c + block, N)))
                           for c in range(0, N, block)], axis=1)


@pytest.mark.parametrize("K,N,group", [(96, 64, 32), (512, 320, 128), (1024, 192, 32),
                                       (1536, 320, 32)])
def test_prepack_bytes(K, N, group):
    """The prepacked bytes and scales are exactly the header's permutation (with zero
    padding of the ragged last tile)."""
    g = S.make_gemv(S.GemvConfig("p", T=1, K=K, N=N, group=group), seed=2)
    wt, st = _prepack(g)
    torch.cuda.synchronize()
    assert np.array_equal(wt.cpu().numpy(), layout_w(g.w))
    assert np.array_equal(bits16(st), layout_s(g.s))


@pytest.mark.parametrize("N", S.GEMV_N)
@pytest.mark.parametrize("T", (1, 2, 4))
def test_tiled_gemv_configs(N, T):
    """Every output column of the GEMV configs (N = 34816 included) within tolerance."""
    g = S.make_gemv(S.gemv_config(N, T), seed=0)
    check_bf16(_run(g), _oracle_blocks(g), what=f"tiled gemv N={N} T={T}")


@pytest.mark.parametrize("T,K,N,group,use_ws", [
    (1, 96, 64, 32, True),        # 3 blocks: a partial round, half a tile
    (2, 96, 64, 32, True),        # matrix-core body: a partial round, half a tile
    (2, 384, 128, 128, False),    # matrix-core body, the last wave's blocks empty, no split
    (1, 384, 128, 128, True),     # 12 blocks: the last wave's blocks are empty
    (3, 5120, 320, 128, True),    # three tokens (four-token instance), half-full last tile
    (2, 1024, 192, 32, True),     # two tokens, a scale per block
    (4, 2048, 64, 32, True),      # four tokens, one half tile, K split
    (4, 1536, 320, 32, False),    # four tokens, no workspace: 3 rounds in one workgroup
    (1, 65536, 64, 128, True),    # the largest K: many splits of one tile
    (1, 2048, 64, 32, False),     # no workspace: 4 rounds in one workgroup
    (2, 7168, 32768, 32, True),   # 14 rounds of 256 tiles, two tokens, a scale per block
])
def test_tiled_gemv_ragged(T, K, N, group, use_ws):
    g = S.make_gemv(S.GemvConfig("r", T=T, K=K, N=N, group=group), seed=3)
    check_bf16(_run(g, use_ws=use_ws), _oracle_blocks(g),
               what=f"tiled gemv T={T} K={K} N={N} G={group}")


@pytest.mark.parametrize("group", [128, 32])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_tiled_one_hot_rows_exact(group, T):
    """x = e_k with power-of-two scales: y must equal row k of W exactly in bf16."""
    rng = np.random.default_rng(7)
    K, N = 5120, 320
    w = rng.integers(0, 256, size=(K // 2, N), dtype=np.uint8)
    s = ((rng.integers(-8, 4, size=(K // group, N)) + 127).astype(np.uint32) << 7).astype(np.uint16)
    B = _b()
    wt, st = B.packed_gemv_int4_prepack(dev(w), dev(s), group)
    ws = B.gemv_workspace(T, K, N, group, "cuda")
    Wd = O.dequant(w, s, group, O.FMT_INT4)
    rows = [0, 1, 2, 3, 31, 32, 127, 128, 129, 2559, 2560, 4095, 5118, 5119]
    for i in range(0, len(rows), T):
        rr = rows[i:i + T]
        x = np.zeros((len(rr), K), np.uint16)
        for j, k in enumerate(rr):
            x[j, k] = 0x3F80
        y = B.packed_gemv_int4_tiled(dev(x), wt, st, N, group, workspace=ws)
        torch.cuda.synchronize()
        want = S.f32_to_bf16_bits(Wd[rr].astype(np.float32))
        assert np.array_equal(bits16(y), want), f"rows {rr}"


def test_tiled_deterministic_and_workspace_reusable():
    """Two calls on one workspace, another shape between them: identical bits."""
    B = _b()
    g = S.make_gemv(S.gemv_config(8192, 4), seed=0)
    wt, st = _prepack(g)
    x = dev(g.x)
    ws = B.gemv_workspace(4, 5120, 8192, 128, x.device)
    y1 = bits16(B.packed_gemv_int4_tiled(x, wt, st, 8192, 128, workspace=ws))
    g2 = S.make_gemv(S.GemvConfig("o", T=1, K=5120, N=8192), seed=9)
    w2, s2 = _prepack(g2)
    B.packed_gemv_int4_tiled(dev(g2.x), w2, s2, 8192, 128, workspace=ws)
    y2 = bits16(B.packed_gemv_int4_tiled(x, wt, st, 8192, 128, workspace=ws))
    torch.cuda.synchronize()
    assert np.array_equal(y1, y2)
    assert int(ws[:4].view(torch.int32).item()) == 0


@pytest.mark.parametrize("T,N,group", [(1, 34816, 128), (1, 320, 32), (1, 8192, 128),
                                       (2, 34816, 128), (3, 320, 32), (4, 8192, 128),
                                       (4, 34816, 128)])
def test_tiled_equals_plain_bitwise(T, N, group):
    """The prepacked call runs the plain call's kernel instance on the same values in the same
    order (only the load addresses differ), so the outputs are identical bit for bit."""
    B = _b()
    g = S.make_gemv(S.GemvConfig("b", T=T, K=5120, N=N, group=group), seed=4)
    x, w, s = dev(g.x), dev(g.w), dev(g.s)
    wt, st = B.packed_gemv_int4_prepack(w, s, group)
    ws = B.gemv_workspace(T, 5120, N, group, "cuda")
    yp = bits16(B.packed_gemv_int4(x, w, s, group, workspace=ws))
    yt = bits16(B.packed_gemv_int4_tiled(x, wt, st, N, group, workspace=ws))
    torch.cuda.synchronize()
    assert np.array_equal(yp, yt)
