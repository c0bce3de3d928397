"""Parity at the sizes bench.py times for the rows beyond the core path: the windowed
decode over decode_64 (w = 1024), the windowed prefill over prefill_32k (w = 4096), the
4096-token KV append and the 2048-pair page copy, each built and launched as the bench
builds and launches it.  Attention outputs are compared with the oracle on sampled
sequences or rows; the movers' whole pools are compared bit for bit."""
import numpy as np
import pytest
import torch

from exact_tiled_attention_pa_amd import binding as B
from exact_tiled_attention_pa_amd import workloads as W
from oracle import attention as OA
from oracle import logical_cache as LC
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    G.gpu_or_skip()


def test_window_decode_at_bench_size():
    """decode_64 (64 sequences of 512-8192 tokens, 32 heads) with a 1024-token window;
    the shortest and longest sequences and four others against the oracle."""
    G.banner("decode_64 with a 1024-token window, 6 sequences")
    wl = W.decode_64(device="cuda")
    call = wl.calls[0]
    w = 1024
    out = torch.empty_like(call.q)
    ws = B.decode_workspace(call.q, wl.k_pool, call.block_table)
    B.pa_decode(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, wl.scale, out,
                ws, window=w)
    torch.cuda.synchronize()
    lens = call.seq_lens_host
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 17, 40, 63})
    G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call, seqs=seqs, window=w),
              "decode_64 window 1024")


def test_window_prefill_at_bench_size():
    """prefill_32k (N = 32768, 8 heads, shuffled pages of 256) with a 4096-token window:
    rows before the window is full, at its edge, across query-tile and page boundaries
    and at the end, all heads, against the oracle."""
    G.banner("prefill_32k with a 4096-token window, sampled rows")
    wl = W.prefill_32k(device="cuda")
    call = wl.calls[0]
    w = 4096
    out = torch.empty_like(call.q)
    B.pa_prefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, True,
                 wl.scale, out, call.q_start, call.max_q_len, window=w)
    torch.cuda.synchronize()
    rng = np.random.default_rng(41)
    rows = np.unique(np.concatenate([
        [0, 1, 127, 128, 255, 256, w - 2, w - 1, w, w + 1, w + 127, 2 * w + 63, 32767],
        rng.integers(0, 32768, 24)]))
    ref = G.oracle_for(wl, call, rows={0: rows}, window=w)
    G.compare(G.bf16_out_to_f64(out), ref, "prefill_32k window 4096")


def test_kv_append_at_bench_size():
    """4096 tokens of one sequence (32 K/V heads, d = 128, shuffled pages of 16) appended
    as the bench appends them; both pools compared bit for bit with the oracle's."""
    G.banner("kv_append, 4096 tokens x 32 heads")
    n_tok, heads, d, ps = 4096, 32, 128, 16
    a = W.build("append_4096", 11, heads=heads, head_dim=d, page_size=ps, lens=[n_tok],
                kind="decode", pool_slack=1.25, device="cuda")
    ac = a.calls[0]
    k_new = W.normal_bf16((n_tok, heads, d), 1.0, 12, "cuda")
    v_new = W.normal_bf16((n_tok, heads, d), 1.0, 13, "cuda")
    ids = torch.zeros(n_tok, dtype=torch.int32, device="cuda")
    pos = torch.arange(n_tok, dtype=torch.int32, device="cuda")
    ref_k, ref_v = OA.kv_append(W.to_host_bits(a.k_pool), W.to_host_bits(a.v_pool),
                                ac.block_table_host, [0] * n_tok, list(range(n_tok)),
                                W.to_host_bits(k_new), W.to_host_bits(v_new))
    B.pa_kv_append(k_new, v_new, ids, pos, a.k_pool, a.v_pool, ac.block_table)
    torch.cuda.synchronize()
    assert np.array_equal(W.to_host_bits(a.k_pool), ref_k)
    assert np.array_equal(W.to_host_bits(a.v_pool), ref_v)


def test_copy_pages_at_bench_size():
    """2048 disjoint page pairs in a 4096-page pool (pages of 16 tokens x 32 heads x
    d = 128, 537 MB per pool) as the bench copies them; both pools bit for bit."""
    G.banner("copy_pages, 2048 pairs over 4096 pages")
    n_pages, n_pairs, ps, heads, d = 4096, 2048, 16, 32, 128
    kp = W.normal_bf16((n_pages, ps, heads, d), 1.0, 14, "cuda")
    vp = W.normal_bf16((n_pages, ps, heads, d), 1.0, 15, "cuda")
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(16))
    src = perm[:n_pairs].to(torch.int32)
    dst = perm[n_pairs:2 * n_pairs].to(torch.int32)
    ref_k, ref_v = LC.copy_pages(W.to_host_bits(kp), W.to_host_bits(vp), src.tolist(),
                                 dst.tolist())
    B.pa_copy_pages(kp, vp, src.cuda(), dst.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(W.to_host_bits(kp), ref_k)
    assert np.array_equal(W.to_host_bits(vp), ref_v)
