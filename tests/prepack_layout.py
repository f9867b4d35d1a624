"""Reference definition of the prepacked GEMV layout (include/dqg.h, packed_gemv_int4_prepack),
written out from the header's description in numpy; used by the GPU byte-exact test and pinned
on the CPU by tests/test_prepack_layout.py."""
import numpy as np


def layout_w(w: np.ndarray) -> np.ndarray:
    """The prepacked weight bytes, written out from the header's definition: blocks of 16
    byte rows of a 128-column tile, units (h, l) = rows r = 16 b + 4 (l // 16) + 2 h and
    r + 1 of the 8 columns c from 128 t + 8 (l % 16), as (r, c + 2m), (r, c + 2m + 1),
    (r + 1, c + 2m), (r + 1, c + 2m + 1) for m = 0..3; zero bytes past N; blocks ordered by
    step of 16 blocks, then tile, then block."""
    Kp, N = w.shape
    tiles, nb = (N + 127) // 128, Kp // 16
    wp = np.zeros((Kp, tiles * 128), np.uint8)
    wp[:, :N] = w
    blocks = {}
    for t in range(tiles):
        for b in range(nb):
            out = np.zeros((2, 64, 4, 4), np.uint8)
            for h in range(2):
                for l in range(64):
                    r = 16 * b + 4 * (l // 16) + 2 * h
                    c = 128 * t + 8 * (l % 16)
                    for m in range(4):
                        out[h, l, m] = [wp[r, c + 2 * m], wp[r, c + 2 * m + 1],
                                        wp[r + 1, c + 2 * m], wp[r + 1, c + 2 * m + 1]]
            blocks[(t, b)] = out.reshape(-1)
    order = [(t, b) for i in range((nb + 15) // 16) for t in range(tiles)
             for b in range(16 * i, min(16 * i + 16, nb))]
    return np.concatenate([blocks[o] for o in order])


def layout_s(s: np.ndarray) -> np.ndarray:
    ng, N = s.shape
    tiles = (N + 127) // 128
    sp = np.zeros((ng, tiles * 128), np.uint16)
    sp[:, :N] = s
    return sp.reshape(-1)
