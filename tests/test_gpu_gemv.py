"""GPU parity: dense packed INT4 GEMV against the oracle."""
import numpy as np
import pytest
import torch

from gpu_util import bits16, check_bf16, dev, guarded, guarded_workspace
from oracle import moe_oracle as O
from workloads import synth as S

pytestmark = pytest.mark.gpu


def _b():
    from dequant_gemv_amd import binding
    return binding


def _run(g, use_ws=True):
    """One call with y and the workspace inside canary bands; the workspace's error word
    must stay zero."""
    B = _b()
    cfg = g.cfg
    x, w, s = dev(g.x), dev(g.w), dev(g.s)
    y, chk_y = guarded((cfg.T, cfg.N), torch.bfloat16)
    ws, chk_ws = None, None
    if use_ws:
        n = B.packed_gemv_int4_workspace_bytes(cfg.T, cfg.K, cfg.N, cfg.group)
        if n:
            ws, chk_ws = guarded_workspace(n)
    B.packed_gemv_int4(x, w, s, cfg.group, y=y, workspace=ws)
    torch.cuda.synchronize()
    chk_y()
    if ws is not None:
        chk_ws()
        assert int(ws[:4].view(torch.int32).item()) == 0
    return bits16(y)


def _oracle_blocks(g, block=4096):
    """The oracle over every column, computed in column blocks (bounded host memory)."""
    N = g.cfg.N
    return np.concatenate([O.packed_gemv(g.x, g.w, g.s, g.cfg.group,
                                         cols=np.arange(c, min(c + block, N)))
                           for c in range(0, N, block)], axis=1)


@pytest.mark.parametrize("N", S.GEMV_N)
@pytest.mark.parametrize("T", S.GEMV_T)
def test_gemv_configs(N, T):
    """Every output column of every GEMV config (N = 34816 included) within tolerance."""
    g = S.make_gemv(S.gemv_config(N, T), seed=0)
    y = _run(g)
    check_bf16(y, _oracle_blocks(g), what=f"gemv N={N} T={T}")


@pytest.mark.parametrize("T,K,N,group,use_ws", [
    (3, 5120, 320, 128, True),     # matrix-core tile with 13 empty rows; 5 tiles
    (5, 1024, 192, 32, True),      # matrix-core tile, G=32
    (1, 5120, 8192, 128, False),   # no workspace: no K split
    (2, 256, 64, 128, True),       # one tile, short K
    (4, 5120, 64, 128, True),      # many K splits for one tile
    (16, 5120, 320, 128, True),    # one full matrix-core tile, half-full last column tile
    (40, 1024, 192, 32, True),     # matrix-core tiles, two token chunks of 32
    (20, 2048, 256, 128, False),   # matrix-core tiles, no workspace
    (1, 5120, 320, 128, True),     # one token: 3 column tiles, the last half full
    (1, 1024, 192, 32, True),      # one token, G=32 (a scale per block)
    (1, 96, 64, 32, True),         # one token, 3 blocks: a partial chunk, one tile of 64
    (1, 384, 128, 128, True),      # one token, 12 blocks: the last wave's chunk is empty
    (1, 2048, 64, 32, False),      # one token, no workspace: 4 rounds in one workgroup
    (1, 65536, 64, 128, True),     # one token, the largest K
    (2, 96, 64, 32, True),         # two tokens (one vector-ALU pass), a partial chunk
    (2, 2048, 192, 32, False),     # two tokens, no workspace: 4 rounds in one workgroup
    (2, 5120, 320, 128, True),     # two tokens, half-full last column tile
    (3, 2048, 192, 128, True),     # three tokens: the matrix-core tiles
])
def test_gemv_ragged(T, K, N, group, use_ws):
    g = S.make_gemv(S.GemvConfig("r", T=T, K=K, N=N, group=group), seed=3)
    check_bf16(_run(g, use_ws), O.packed_gemv(g.x, g.w, g.s, group), what="gemv ragged")


def test_gemv_seeds_1_2():
    for seed in (1, 2):
        g = S.make_gemv(S.gemv_config(8192, 4), seed=seed)
        check_bf16(_run(g), O.packed_gemv(g.x, g.w, g.s, 128), what=f"seed {seed}")


@pytest.mark.parametrize("rows", [
    [0, 1, 127, 128, 129, 2559, 2560, 5118, 5119],                       # vector-ALU tiles
    [0, 1, 31, 32, 33, 127, 128, 129, 1000, 2559, 2560, 2561, 4095, 4096,
     4097, 5000, 5117, 5118, 5119, 3],                                  # matrix-core tiles
])
def test_gemv_one_hot_rows_exact(rows):
    """x = e_k with power-of-two scales: y must equal row k of W exactly in bf16."""
    rng = np.random.default_rng(5)
    K, N, G = 5120, 256, 128
    w = rng.integers(0, 256, size=(K // 2, N), dtype=np.uint8)
    s = ((rng.integers(-8, 4, size=(K // G, N)) + 127).astype(np.uint32) << 7).astype(np.uint16)
    x = np.zeros((len(rows), K), np.uint16)
    for i, k in enumerate(rows):
        x[i, k] = 0x3F80
    B = _b()
    y = B.packed_gemv_int4(dev(x), dev(w), dev(s), G,
                           workspace=B.gemv_workspace(len(rows), K, N, G, "cuda"))
    torch.cuda.synchronize()
    Wd = O.dequant(w, s, G, O.FMT_INT4)
    want = S.f32_to_bf16_bits(Wd[rows].astype(np.float32))
    assert np.array_equal(bits16(y), want)


@pytest.mark.parametrize("group", [128, 32])
def test_gemv_one_token_one_hot_rows_exact(group):
    """One token, x = e_k with power-of-two scales: y must equal row k of W exactly (the
    paired-row decode and its bias term cancel exactly for a single nonzero activation)."""
    rng = np.random.default_rng(6)
    K, N = 5120, 320
    w = rng.integers(0, 256, size=(K // 2, N), dtype=np.uint8)
    s = ((rng.integers(-8, 4, size=(K // group, N)) + 127).astype(np.uint32) << 7).astype(np.uint16)
    B = _b()
    ws = B.gemv_workspace(1, K, N, group, "cuda")
    Wd = O.dequant(w, s, group, O.FMT_INT4)
    for k in (0, 1, 2, 3, 31, 32, 127, 128, 129, 2559, 2560, 5118, 5119):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = 0x3F80
        y = B.packed_gemv_int4(dev(x), dev(w), dev(s), group, workspace=ws)
        torch.cuda.synchronize()
        want = S.f32_to_bf16_bits(Wd[[k]].astype(np.float32))
        assert np.array_equal(bits16(y), want), f"row {k}"


def test_gemv_deterministic_and_workspace_reusable():
    B = _b()
    g = S.make_gemv(S.gemv_config(8192, 4), seed=0)
    x, w, s = dev(g.x), dev(g.w), dev(g.s)
    ws = B.gemv_workspace(4, 5120, 8192, 128, x.device)
    y1 = bits16(B.packed_gemv_int4(x, w, s, 128, workspace=ws))
    g2 = S.make_gemv(S.GemvConfig("o", T=1, K=5120, N=8192), seed=9)
    B.packed_gemv_int4(dev(g2.x), dev(g2.w), dev(g2.s), 128, workspace=ws)  # other shape
    y2 = bits16(B.packed_gemv_int4(x, w, s, 128, workspace=ws))
    torch.cuda.synchronize()
    assert np.array_equal(y1, y2)
