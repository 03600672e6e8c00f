"""The split-operand layout decoder used by the GPU tests, against the
layout's index formula written out element by element (include/encscore.h,
last-token refinement kernels)."""
import numpy as np

from helpers import split_decode


def test_split_decode_inverts_the_index_formula():
    rng = np.random.default_rng(0)
    for M, K in ((1, 16), (33, 48), (70, 64)):
        M32 = -(-M // 32) * 32
        hi = rng.integers(0, 1 << 16, (M32, K), dtype=np.uint32).astype(np.uint16)
        lo = rng.integers(0, 1 << 16, (M32, K), dtype=np.uint32).astype(np.uint16)
        buf = np.zeros(2 * M32 * K, dtype=np.uint16)
        for m in range(M32):
            for k in range(K):
                for h, src in ((0, hi), (1, lo)):
                    i = ((((m // 32) * (K // 16) + k // 16) * 2 + h) * 64 + ((k // 8) % 2) * 32 + m % 32) * 8 + k % 8
                    buf[i] = src[m, k]
        dh, dl = split_decode(buf, M, K)
        assert np.array_equal(dh, hi) and np.array_equal(dl, lo)
