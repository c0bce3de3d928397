"""Host-side arithmetic of bench.py: algorithmic work counts against brute force."""
import numpy as np

import bench
from oracle import attention as OA


def test_visible_pairs_matches_mask_count():
    rng = np.random.default_rng(0)
    for _ in range(20):
        L = int(rng.integers(1, 300))
        n = int(rng.integers(1, L + 1))
        for causal in (True, False):
            mask = OA.visible_mask(np.arange(L - n, L), L, causal)
            assert bench.visible_pairs([L], [n], causal) == int(mask.sum())


def test_causal_full_prefill_pairs_closed_form():
    N = 4096
    assert bench.visible_pairs([N], [N], True) == N * (N + 1) // 2
    # 4*d*H*pairs for the causal N=4096, 32-head, d=128 prefill: 137.5 GFLOP
    assert abs(4 * 128 * 32 * bench.visible_pairs([N], [N], True) - 137.5e9) < 0.1e9
