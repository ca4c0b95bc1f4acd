"""The NumPy form of the packed weight order (used by the GPU tests) against
the element formula of include/nvfp4moe.h, evaluated entry by entry."""
import numpy as np

from _cases import pack_weights_np


def test_pack_np_matches_the_formula():
    rng = np.random.default_rng(5)
    B, N, K = 2, 64, 256
    q = rng.integers(0, 256, (B, N, K // 2), dtype=np.uint8)
    sf = rng.integers(0, 256, (B, N, K // 16), dtype=np.uint8)
    got = pack_weights_np(q, sf)
    assert got.shape == (B, N // 32, K // 128, 2304)
    for b in range(B):
        for t in range(N // 32):
            for c in range(K // 128):
                ch = got[b, t, c]
                for l in range(64):
                    row = 32 * t + l % 32
                    for h in range(2):
                        for i in range(16):
                            assert ch[h * 1024 + 16 * l + i] == q[b, row, 64 * c + 32 * (l // 32) + 16 * h + i]
                    for i in range(4):
                        assert ch[2048 + 4 * l + i] == sf[b, row, 8 * c + 4 * (l // 32) + i]


def test_pack_np_is_a_permutation():
    rng = np.random.default_rng(6)
    q = rng.integers(0, 256, (1, 96, 192), dtype=np.uint8)
    sf = rng.integers(0, 256, (1, 96, 24), dtype=np.uint8)
    got = pack_weights_np(q, sf).reshape(-1)
    assert np.array_equal(np.sort(got), np.sort(np.concatenate([q.reshape(-1), sf.reshape(-1)])))
