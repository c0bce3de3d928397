"""The seeded input generator: determinism and the structure of every workload
(lengths, block tables, pool sizing), checked on layouts without drawing pools."""
import math

import numpy as np
import torch

from exact_tiled_attention_pa_amd import workloads as W


def test_small_workload_is_deterministic():
    a = W.build("x", 3, heads=2, head_dim=64, page_size=16, lens=[37, 5], q_lens=[37, 5],
                pool_slack=1.5, poison=True)
    b = W.build("x", 3, heads=2, head_dim=64, page_size=16, lens=[37, 5], q_lens=[37, 5],
                pool_slack=1.5, poison=True)
    c = W.build("x", 4, heads=2, head_dim=64, page_size=16, lens=[37, 5], q_lens=[37, 5],
                pool_slack=1.5, poison=True)
    assert a.digest() == b.digest() != c.digest()


def _check_tables(call, page_size, num_pages, unique=True):
    used = []
    for b in range(call.batch):
        L = int(call.seq_lens_host[b])
        n = -(-L // page_size)
        row = call.block_table_host[b]
        assert np.all(row[:n] >= 0) and np.all(row[:n] < num_pages)
        assert np.all(row[n:] == -1)
        used.extend(row[:n].tolist())
    if unique:
        assert len(set(used)) == len(used)
    return used


def test_prefill_600_layout():
    wl = W.prefill_600(tensors=False)
    call = wl.calls[0]
    assert call.block_table_host.tolist() == [[5, 1, 9]]
    assert wl.num_pages == 12 and wl.page_size == 256 and wl.head_dim == 64
    assert call.seq_lens_host.tolist() == [600] and call.q_start_host.tolist() == [0, 600]
    assert wl.scale == 0.125


def test_decode_64_layout():
    wl = W.decode_64(tensors=False)
    call = wl.calls[0]
    lens = call.seq_lens_host
    assert len(lens) == 64 and lens.min() >= 512 and lens.max() <= 8192
    used = _check_tables(call, 16, wl.num_pages)
    assert sorted(used) == list(range(wl.num_pages))  # pool sized exactly, a permutation
    assert wl.scale == np.float32(1 / math.sqrt(128))


def test_prefill_4096_layout():
    wl = W.prefill_4096(tensors=False)
    assert wl.calls[0].block_table_host.tolist() == [list(range(16))]


def test_prefill_32k_layout():
    wl = W.prefill_32k(tensors=False)
    used = _check_tables(wl.calls[0], 256, wl.num_pages)
    assert sorted(used) == list(range(128)) and used != list(range(128))
    assert wl.sigma == 0.5


def test_mixed_layout():
    wl = W.mixed_128x4(tensors=False)
    dec, pre = wl.calls
    lens = dec.seq_lens_host
    assert len(lens) == 128 and lens.min() >= 1024 and lens.max() <= 32768
    assert 2048 < np.median(lens) < 8192
    assert pre.seq_lens_host.tolist() == [10240] * 4
    assert pre.q_start_host.tolist() == [0, 2048, 4096, 6144, 8192]
    used = _check_tables(dec, 16, wl.num_pages) + _check_tables(pre, 16, wl.num_pages)
    assert len(set(used)) == len(used)
    assert wl.num_pages == math.ceil(1.25 * len(used))


def test_poison_marks_exactly_the_unread_slots():
    wl = W.build("p", 8, heads=1, head_dim=64, page_size=16, lens=[20, 16, 1], q_lens=[1, 1, 1],
                 pool_slack=2.0, poison=True)
    call = wl.calls[0]
    nan = torch.isnan(wl.k_pool.float())[:, :, 0, 0].numpy()
    expect = np.ones_like(nan)
    for b, L in enumerate(call.seq_lens_host):
        for j in range(-(-int(L) // 16)):
            p = call.block_table_host[b, j]
            expect[p, :min(16, L - 16 * j)] = False
    assert np.array_equal(nan, expect)
