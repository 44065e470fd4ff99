"""CPU check of the numpy key code that the GPU key tests compare against."""
import numpy as np

from key_codes import key_code16


def test_key_code16_is_monotone():
    # ordered by their order keys (which put -0 below +0), floats never get a
    # smaller code than a lower key: across both signs, zeros, the window's
    # edges and infinities
    vals = np.concatenate([np.float32([-np.inf, -3e38, -1e3, -512.0, -511.9, -2.0 ** -7,
                                       -1e-3, -0.0, 0.0, 1e-30, 2.0 ** -7, 3.49, 3.5, 511.9,
                                       512.0, 1e30, np.inf]),
                           np.linspace(-600, 600, 100001, dtype=np.float32),
                           np.float32(np.random.default_rng(3).standard_normal(10000) * 50)])
    x = vals.view(np.uint32)
    u = np.sort(np.where(x & 0x80000000, ~x, x | 0x80000000).astype(np.uint32))
    c = key_code16(u)
    assert np.all(np.diff(c) >= 0) and c.min() >= 1 and c.max() <= 0xFFFF
    # inside the window a binade has 2048 codes: the values k/2048 of [1, 2)
    # and of [-2, -1) each get a code of their own
    grid = np.float32(1.0 + np.arange(2048) / 2048.0)
    for g_ in (grid, -grid):
        y = g_.view(np.uint32)
        cu = key_code16(np.where(y & 0x80000000, ~y, y | 0x80000000).astype(np.uint32))
        assert np.unique(cu).size == 2048
