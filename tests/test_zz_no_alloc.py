"""GPU: the allocation-free GEMV entry point (library-owned scratch) against the workspace
entry point and the oracle, on two calls in a row, the second with a smaller input."""
import numpy as np
import pytest
import torch

from gpu_util import bits16, check_bf16, dev
from oracle import moe_oracle as O
from workloads import synth as S

pytestmark = pytest.mark.gpu


def _pair(T, N, seed):
    from dequant_gemv_amd import binding as B
    g = S.make_gemv(S.GemvConfig("na", T=T, K=5120, N=N, group=128), seed=seed)
    x, w, s = dev(g.x), dev(g.w), dev(g.s)
    status = torch.zeros(1, dtype=torch.int32, device=x.device)
    y_na = B.packed_gemv_int4_noalloc(x, w, s, 128, status=status)
    ws = B.gemv_workspace(T, 5120, N, 128, x.device)
    y_ws = B.packed_gemv_int4(x, w, s, 128, workspace=ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert int(ws.view(torch.int32)[0].item()) == 0
    return g, bits16(y_na), bits16(y_ws)


def test_noalloc_gemv_matches_workspace_entry_point_twice():
    # first call: 34816 columns, 4 tokens (10 K splits in the scratch); second: smaller
    for T, N, seed in ((4, 34816, 11), (1, 8192, 12)):
        g, y_na, y_ws = _pair(T, N, seed)
        assert np.array_equal(y_na, y_ws), f"T={T} N={N}: outputs differ"
        cols = np.arange(0, N, 7)
        check_bf16(y_na[:, cols], O.packed_gemv(g.x, g.w, g.s, 128, cols=cols),
                   what=f"noalloc T={T} N={N}")
