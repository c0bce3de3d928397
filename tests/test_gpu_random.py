"""Seeded random configurations of decode and prefill against the fp64 oracle.

Each case draws head_dim, page size, K/V heads, query heads per K/V head, sequence
lengths (edge lengths around page, chunk and split boundaries mixed with random ones),
query chunk lengths, the causal flag and a sliding window, builds NaN-poisoned pools
with a shuffled page assignment, and compares the library's output element by
element with the oracle on the same bytes.  The draws are fixed by the seed, so a
failure names a reproducible case."""
import numpy as np
import pytest
import torch

from exact_tiled_attention_pa_amd import binding as B
from exact_tiled_attention_pa_amd import workloads as W
from oracle import attention as OA
from tests import gpu_helpers as G
from tests.gpu_helpers import prefill_path  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 2, 15, 16, 17, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025]


@pytest.fixture(autouse=True)
def _gpu():
    G.gpu_or_skip()


def _lens(rng, batch, cap):
    out = []
    for _ in range(batch):
        if rng.random() < 0.5:
            out.append(int(rng.choice([x for x in EDGE_LENS if x <= cap])))
        else:
            out.append(int(rng.integers(1, cap + 1)))
    return out


def decode_case(seed):
    rng = np.random.default_rng(1000 + seed)
    d = int(rng.choice([64, 128]))
    ps = int(rng.choice([16, 32, 64, 128, 256]))
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 8]))
    batch = int(rng.integers(1, 6))
    lens = _lens(rng, batch, 4000)
    window = int(rng.choice([0, 0, 1, 17, 300, 1500]))
    return d, ps, hkv, hkv * g, lens, window


def prefill_case(seed):
    rng = np.random.default_rng(2000 + seed)
    d = int(rng.choice([64, 128]))
    ps = int(rng.choice([16, 32, 64, 128, 256]))
    hkv = int(rng.choice([1, 2, 3]))
    g = int(rng.choice([1, 2, 4]))
    batch = int(rng.integers(1, 4))
    lens = _lens(rng, batch, 700)
    q_lens = [int(rng.integers(0, L + 1)) if rng.random() < 0.3 else
              int(rng.choice([L, min(L, 1), min(L, 129)])) for L in lens]
    causal = bool(rng.random() < 0.75)
    window = int(rng.choice([0, 0, 5, 64, 200])) if causal else 0
    return d, ps, hkv, hkv * g, lens, q_lens, causal, window


@pytest.mark.parametrize("seed", range(16))
def test_random_decode(seed):
    d, ps, hkv, hq, lens, window = decode_case(seed)
    G.banner(f"random decode seed={seed} d={d} ps={ps} Hkv={hkv} Hq={hq} lens={lens} "
             f"window={window}")
    wl = W.build("rdec", 3000 + seed, heads=hkv, head_dim=d, page_size=ps, lens=lens,
                 kind="decode", pool_slack=1.3, device="cuda", poison=True, q_heads=hq)
    call = wl.calls[0]
    out = torch.empty_like(call.q)
    ws = B.decode_workspace(call.q, wl.k_pool, call.block_table)
    B.pa_decode(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, wl.scale, out,
                ws, window=window)
    torch.cuda.synchronize()
    q, k, v, table = G.host_inputs(wl, call, list(range(call.batch)))
    ref, _ = OA.paged_decode(q, k, v, table, call.seq_lens_host, wl.scale, window=window)
    G.compare(G.bf16_out_to_f64(out), ref, f"random decode seed={seed}")


@pytest.mark.parametrize("seed", range(12))
def test_random_prefill(seed, prefill_path):
    d, ps, hkv, hq, lens, q_lens, causal, window = prefill_case(seed)
    G.banner(f"random prefill seed={seed} d={d} ps={ps} Hkv={hkv} Hq={hq} lens={lens} "
             f"q_lens={q_lens} causal={causal} window={window}")
    wl = W.build("rpre", 4000 + seed, heads=hkv, head_dim=d, page_size=ps, lens=lens,
                 q_lens=q_lens, causal=causal, pool_slack=1.3, device="cuda", poison=True,
                 q_heads=hq)
    call = wl.calls[0]
    out = torch.full_like(call.q, float("nan"))
    if call.q.shape[0] > 0:
        B.pa_prefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, causal,
                     wl.scale, out, call.q_start, call.max_q_len, window=window)
    torch.cuda.synchronize()
    q, k, v, table = G.host_inputs(wl, call, list(range(call.batch)))
    ref, _ = OA.paged_prefill(q, k, v, table, call.seq_lens_host, call.q_start_host, causal,
                              wl.scale, window=window)
    G.compare(G.bf16_out_to_f64(out), ref, f"random prefill seed={seed}")


def short_chunk_case(seed):
    """Chunks of a few rows on caches of up to 6,000 keys: the split-key prefill's
    regime (each wave of a 32-row workgroup walks a quarter of a long key range)."""
    rng = np.random.default_rng(5000 + seed)
    d = int(rng.choice([64, 128]))
    ps = int(rng.choice([16, 32, 64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4]))
    batch = int(rng.integers(1, 4))
    lens = _lens(rng, batch, 6000)
    q_lens = [int(rng.choice([min(L, x) for x in (1, 2, 7, 31, 32, 33, 64)])) for L in lens]
    causal = bool(rng.random() < 0.75)
    window = int(rng.choice([0, 0, 1, 40, 700, 5000])) if causal else 0
    return d, ps, hkv, hkv * g, lens, q_lens, causal, window


@pytest.mark.parametrize("seed", range(10))
def test_random_short_chunks(seed, prefill_path):
    d, ps, hkv, hq, lens, q_lens, causal, window = short_chunk_case(seed)
    G.banner(f"random short chunks seed={seed} d={d} ps={ps} Hkv={hkv} Hq={hq} lens={lens} "
             f"q_lens={q_lens} causal={causal} window={window}")
    wl = W.build("rshort", 6000 + seed, heads=hkv, head_dim=d, page_size=ps, lens=lens,
                 q_lens=q_lens, causal=causal, pool_slack=1.2, device="cuda", poison=True,
                 q_heads=hq)
    call = wl.calls[0]
    out = torch.full_like(call.q, float("nan"))
    B.pa_prefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, causal,
                 wl.scale, out, call.q_start, call.max_q_len, window=window)
    torch.cuda.synchronize()
    G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call, window=window),
              f"random short chunks seed={seed}")


def test_many_short_sequences_decode_and_prefill(prefill_path):
    """Thousands of short decode sequences (grid z in the thousands, one chunk per
    split) and hundreds of short prefill chunks in one call."""
    rng = np.random.default_rng(77)
    lens = [int(x) for x in rng.integers(1, 80, size=3000)]
    G.banner(f"many sequences: decode batch={len(lens)}")
    wl = W.build("many_dec", 78, heads=2, head_dim=64, page_size=16, lens=lens, kind="decode",
                 pool_slack=1.1, device="cuda", poison=True, q_heads=4)
    call = wl.calls[0]
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    q, k, v, table = G.host_inputs(wl, call, list(range(call.batch)))
    ref, _ = OA.paged_decode(q, k, v, table, call.seq_lens_host, wl.scale)
    G.compare(G.bf16_out_to_f64(out), ref, "many short decode sequences")

    lens = [int(x) for x in rng.integers(1, 300, size=300)]
    q_lens = [int(rng.integers(0, min(L, 40) + 1)) for L in lens]
    G.banner(f"many sequences: prefill batch={len(lens)} rows={sum(q_lens)}")
    wl = W.build("many_pre", 79, heads=2, head_dim=128, page_size=32, lens=lens, q_lens=q_lens,
                 causal=True, pool_slack=1.1, device="cuda", poison=True)
    call = wl.calls[0]
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call), "many short prefill chunks")
