"""CPU pins of the prepacked GEMV layout's reference definition (tests/prepack_layout.py, which
the GPU test compares the prepack kernel's bytes with): it must be a permutation of the
[K/2, N] bytes plus zero padding of the ragged last tile, and every byte must sit where the
block / unit / byte formulas of include/dqg.h put it."""
import numpy as np

from prepack_layout import layout_s, layout_w

KP, N = 320, 192          # 20 blocks of 16 byte rows: a full round of 16 and a partial one of 4
TILES, NB = 2, 20         # the second tile has 64 real columns and 64 padded ones


def _sources():
    """For every prepacked byte, the (row, column) of [K/2, N] it was taken from, or -1 for
    padding: the layout applied to matrices of row and column tags (the layout only moves
    bytes, so tagged inputs reveal the permutation)."""
    r = np.arange(KP)[:, None].repeat(N, 1)
    c = np.arange(N)[None, :].repeat(KP, 0)
    tags = {}
    for name, a in (("rlo", r % 256), ("rhi", r // 256), ("c", c)):
        tags[name] = layout_w((a + (1 if name != "rhi" else 0)).astype(np.uint8)).astype(np.int64)
    valid = tags["c"] > 0
    # the low row byte was tagged + 1 (mod 256): tag 0 is row % 256 == 255, padding is told
    # apart by the column tag, which is never 0 for a real byte
    rows = np.where(valid, ((tags["rlo"] - 1) % 256) + 256 * tags["rhi"], -1)
    cols = np.where(valid, tags["c"] - 1, -1)
    return rows, cols


def test_layout_is_a_permutation_with_zero_padding():
    rows, cols = _sources()
    assert rows.size == TILES * NB * 2048
    real = rows >= 0
    assert int(real.sum()) == KP * N
    seen = set(zip(rows[real].tolist(), cols[real].tolist()))
    assert len(seen) == KP * N  # every byte of the matrix exactly once
    assert int((~real).sum()) == KP * (TILES * 128 - N)
    w = np.random.default_rng(0).integers(1, 256, size=(KP, N), dtype=np.uint8)
    assert np.all(layout_w(w)[~real] == 0)


def test_layout_matches_the_header_formulas():
    rows, cols = _sources()
    for t in range(TILES):
        for b in range(NB):
            i = b // 16
            n_i = min(16, NB - 16 * i)
            base = 2048 * (16 * i * TILES + t * n_i + b - 16 * i)
            for u in range(128):
                h, l = divmod(u, 64)
                q, kq = l % 16, l // 16
                r = 16 * b + 4 * kq + 2 * h
                c = 128 * t + 8 * q
                for m in range(4):
                    want = [(r, c + 2 * m), (r, c + 2 * m + 1), (r + 1, c + 2 * m),
                            (r + 1, c + 2 * m + 1)]
                    for j, (wr, wc) in enumerate(want):
                        p = base + 16 * u + 4 * m + j
                        if wc < N:
                            assert (rows[p], cols[p]) == (wr, wc), (t, b, u, m, j)
                        else:
                            assert rows[p] == -1


def test_scale_layout_pads_columns():
    s = np.arange(1, 3 * 64 + 1, dtype=np.uint16).reshape(3, 64)
    out = layout_s(s).reshape(3, 128)
    assert np.array_equal(out[:, :64], s) and np.all(out[:, 64:] == 0)
