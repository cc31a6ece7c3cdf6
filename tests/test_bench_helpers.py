"""bench.py's FLOP counts against brute-force loops over the lists (CPU).

kept_flop is the numerator of the reported TFLOP/s (4 * rows * keys * d per
kept pair, partial blocks counted exactly); pipe_mfma_flop is what the d = 128,
128-token kernel must issue, checked against the MFMA counter on the GPU.
"""

import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _lists(rng, BH, nb, width):
    idx = np.full((1, BH, nb, width), -1, dtype=np.int32)
    cnt = np.zeros((1, BH, nb), dtype=np.int32)
    for h in range(BH):
        for i in range(nb):
            c = int(rng.integers(0, width + 1))
            idx[0, h, i, :c] = np.sort(rng.choice(nb, size=c, replace=False))
            cnt[0, h, i] = c
    return idx, cnt


def _brute(idx, cnt, N, block, d):
    kept = mfma = 0
    for h in range(idx.shape[1]):
        for i in range(idx.shape[2]):
            rows = min(block, N - i * block)
            for t in range(cnt[0, h, i]):
                j = int(idx[0, h, i, t])
                keys = min(block, N - j * block)
                kept += 4 * rows * keys * d
                halves = 1 + (j * 128 + 64 < N)
                mfma += halves * 4 * 32 * 32768
    return kept, mfma


def test_flop_counts_match_brute_force():
    rng = np.random.default_rng(4)
    for N, width in ((1000, 3), (1100, 8), (1024, 5), (1090, 2)):
        nb = -(-N // 128)
        idx, cnt = _lists(rng, 3, nb, width)
        kept, mfma = _brute(idx, cnt, N, 128, 128)
        ti, tc = torch.from_numpy(idx), torch.from_numpy(cnt)
        assert bench.kept_flop(ti, tc, N, 128, 128) == kept
        assert bench.pipe_mfma_flop(ti, tc, N) == mfma


def test_full_tiles_mfma_equals_attention_flop():
    # every block full: the kernel issues exactly the attention FLOP
    N, nb = 1024, 8
    idx = torch.arange(nb, dtype=torch.int32).expand(1, 2, nb, nb).contiguous()
    cnt = torch.full((1, 2, nb), nb, dtype=torch.int32)
    assert bench.pipe_mfma_flop(idx, cnt, N) == 4.0 * 2 * N * N * 128
    assert bench.kept_flop(idx, cnt, N, 128, 128) == 4.0 * 2 * N * N * 128
