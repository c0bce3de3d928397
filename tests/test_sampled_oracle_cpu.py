"""The sampled evaluation behind every full-size parity verdict, pinned on the CPU.

At full sizes the GPU tests hand the oracle only the pages that the sampled
sequences read (tests/gpu_helpers.host_inputs: the pages are compacted and the
block table rewritten onto them) and ask it for some rows or sequences only.
Here that compaction is checked to change no output bit against the whole pool
and original table, and two plausible slips in it are planted and caught.  The
rows= / seqs= sampling of the oracle itself is pinned in tests/oracle_pins.py
(pin_sampled_rows_match_full, pin_sampled_seqs_match_full).
"""
import numpy as np
import pytest

from exact_tiled_attention_pa_amd import workloads as W
from oracle import attention as OA
from tests import gpu_helpers as G


def _small(kind, q_heads):
    lens = [40, 7, 300, 129, 16]
    q_lens = [40, 3, 100, 1, 16] if kind == "prefill" else None
    return W.build("sample", 21, heads=2, head_dim=8, page_size=16, lens=lens, q_lens=q_lens,
                   kind=kind, causal=True, pool_slack=1.6, device="cpu", poison=True,
                   q_heads=q_heads)


def _whole_pool_reference(wl, call, seqs, rows=None):
    """The oracle on the uncompacted pool and the original block table."""
    q = W.to_host_bits(call.q)
    k = W.to_host_bits(wl.k_pool)
    v = W.to_host_bits(wl.v_pool)
    if call.kind == "prefill":
        if rows is None:
            rows = {b: np.arange(call.q_start_host[b + 1] - call.q_start_host[b]) for b in seqs}
        ref, _ = OA.paged_prefill(q, k, v, call.block_table_host, call.seq_lens_host,
                                  call.q_start_host, call.causal, wl.scale, rows=rows)
    else:
        ref, _ = OA.paged_decode(q, k, v, call.block_table_host, call.seq_lens_host, wl.scale,
                                 seqs=seqs)
    return ref


def compaction_is_exact(wl, call, seqs, rows=None) -> bool:
    """host_inputs' compacted pool and table give the same output bits as the whole
    pool; an exception (a page the compacted table cannot reach) counts as a failure."""
    try:
        got = G.oracle_for(wl, call, seqs=seqs, rows=rows)
    except (IndexError, ValueError, KeyError):
        return False
    want = _whole_pool_reference(wl, call, seqs, rows)
    return bool(np.array_equal(np.isnan(got), np.isnan(want)) and
                np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)]))


CASES = [("decode", 2, [4, 0, 2], None), ("decode", 6, [1, 3], None),
         ("prefill", 2, [0, 2, 4], None), ("prefill", 4, [2, 3], {2: np.array([99, 0, 50]),
                                                                  3: np.array([0])})]


@pytest.mark.parametrize("kind,q_heads,seqs,rows", CASES)
def test_compaction_changes_no_output_bit(kind, q_heads, seqs, rows):
    wl = _small(kind, q_heads)
    assert compaction_is_exact(wl, wl.calls[0], seqs, rows)


def _reversed_page_list(block_table_host, seq_lens_host, seqs, page_size):
    # takes the pages in the sorted order but numbers them from the other end
    uniq, table = _ORIG_COMPACT(block_table_host, seq_lens_host, seqs, page_size)
    n = len(uniq)
    return uniq, np.where(table >= 0, n - 1 - table, table)


def _first_sequence_pages_only(block_table_host, seq_lens_host, seqs, page_size):
    # keeps the page list of the first sampled sequence only
    return _ORIG_COMPACT(block_table_host, seq_lens_host, seqs[:1], page_size)


_ORIG_COMPACT = G.compact_pages


@pytest.mark.parametrize("slip", [_reversed_page_list, _first_sequence_pages_only],
                         ids=lambda f: f.__name__)
def test_planted_compaction_slips_are_caught(monkeypatch, slip):
    monkeypatch.setattr(G, "compact_pages", slip)
    caught = []
    for kind, q_heads, seqs, rows in CASES:
        wl = _small(kind, q_heads)
        caught.append(not compaction_is_exact(wl, wl.calls[0], seqs, rows))
    assert any(caught), "no case caught the planted compaction slip"
