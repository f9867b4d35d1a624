"""GPU parity: in-register decode (bit-exact) and top-k routing (ids bit-exact)."""
import numpy as np
import pytest
import torch

from gpu_util import dev
from oracle import moe_oracle as O
from workloads import synth as S

pytestmark = pytest.mark.gpu


def _b():
    from dequant_gemv_amd import binding
    return binding


@pytest.mark.parametrize("fmt", [O.FMT_INT4, O.FMT_FP4])
@pytest.mark.parametrize("group", [32, 128])
def test_dequant_bit_exact(fmt, group):
    B = _b()
    rng = np.random.default_rng(40 + fmt + group)
    K, N = 4 * group, 112
    w = rng.integers(0, 256, size=(K // 2, N), dtype=np.uint8)
    # every byte value appears, including 0x08 / 0x80 (signed zeros of E2M1)
    w.flat[:256] = np.arange(256, dtype=np.uint8)
    s = S.f32_to_bf16_bits(rng.uniform(0.001, 4.0, size=(K // group, N)))
    s[0, :4] = [0x3C80, 0x3C23, 0x3F80, 0x4000]
    out = B.packed_dequant_f32(dev(w), dev(s), group, fmt)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = O.dequant(w, s, group, fmt).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("T,E,k,dist", [
    (1, 8, 2, "normal"), (1, 128, 8, "normal"), (64, 128, 8, "normal"),
    (8, 512, 10, "normal"), (3, 1000, 5, "normal"), (5, 4096, 32, "normal"),
    (33, 16, 16, "ties"), (17, 64, 7, "ties"), (9, 70, 1, "ties"), (4, 4, 4, "ties"),
])
def test_topk_route_ids_bit_exact(T, E, k, dist):
    B = _b()
    rng = np.random.default_rng(T * 7 + E + k)
    if dist == "ties":
        lg = rng.choice(np.array([-1.0, 0.0, -0.0, 1.0, 0.5], np.float32), size=(T, E))
    else:
        lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = B.topk_route(dev(lg), k)
    torch.cuda.synchronize()
    oi, ow = O.topk_route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), oi)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=4e-6, atol=1e-7)
