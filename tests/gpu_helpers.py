"""Helpers for the GPU parity tests: run the HIP library on a workload, hand the
same inputs (copied to the host) to the oracle, and compare.

The oracle is called only here and in the CPU tests; it never sees anything the
HIP library produced except the output being checked.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_tiled_attention_pa_amd import binding as B
from exact_tiled_attention_pa_amd import workloads as W
from oracle import attention as OA

# Tolerances against the fp64 oracle: bf16 inputs and outputs, fp32 accumulation.
MAX_ABS_TOL = 1e-2
MEAN_ABS_TOL = 1e-3


def gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    # on a GPU machine the library must be there: fail loudly if it is not
    B.load_library()


def banner(msg: str):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(params=["tiles", "split"])
def prefill_path(request, monkeypatch):
    """Runs a prefill test once with each prefill kernel forced through PA_PREFILL_PATH:
    the 128-row tiled kernel and the split-key kernel (which small launches take by
    default)."""
    monkeypatch.setenv("PA_PREFILL_PATH", request.param)
    print(f"[case] prefill path {request.param}", flush=True)
    return request.param


def run_call(wl: W.Workload, call: W.AttnCall, out=None, workspace=None):
    """Runs one library call of a workload on the current stream; returns out (bf16)."""
    if out is None:
        out = torch.empty_like(call.q)
    if call.kind == "prefill":
        B.pa_prefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens,
                     call.causal, wl.scale, out, call.q_start, call.max_q_len)
    else:
        if workspace is None:
            workspace = B.decode_workspace(call.q, wl.k_pool, call.block_table)
        B.pa_decode(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, wl.scale,
                    out, workspace)
    return out


def bf16_out_to_f64(out: torch.Tensor) -> np.ndarray:
    return OA.bf16_to_f64(W.to_host_bits(out))


def compact_pages(block_table_host, seq_lens_host, seqs, page_size):
    """The pages the given sequences read, sorted and without repeats, and the block
    table rewritten onto positions in that list (-1 for everything else)."""
    pages = []
    for b in seqs:
        n = OA.pages_needed(int(seq_lens_host[b]), page_size)
        pages.extend(int(p) for p in block_table_host[b, :n])
    uniq = sorted(set(pages))
    index = {p: i for i, p in enumerate(uniq)}
    table = np.full_like(block_table_host, -1)
    for b in seqs:
        n = OA.pages_needed(int(seq_lens_host[b]), page_size)
        table[b, :n] = [index[int(p)] for p in block_table_host[b, :n]]
    return uniq, table


def host_inputs(wl: W.Workload, call: W.AttnCall, seqs):
    """Host copies (uint16 bit patterns) of the pages the given sequences read, with
    the block table rewritten onto the compacted page list; the oracle then gathers
    the very same bytes the kernel reads.  (The compaction changes no output bit:
    tests/test_sampled_oracle_cpu.py.)"""
    uniq, table = compact_pages(call.block_table_host, call.seq_lens_host, seqs,
                                wl.page_size)
    sel = torch.tensor(uniq, dtype=torch.long, device=wl.k_pool.device)
    k = W.to_host_bits(wl.k_pool.index_select(0, sel))
    v = W.to_host_bits(wl.v_pool.index_select(0, sel))
    q = W.to_host_bits(call.q)
    return q, k, v, table


def oracle_for(wl: W.Workload, call: W.AttnCall, seqs=None, rows=None, window=0):
    """fp64 reference of (some of) a call's outputs.  rows: {b: local row indices}.
    Grouped heads need nothing here: the oracle reads the K/V head count from the
    pools and maps query heads onto K/V heads itself."""
    if seqs is None:
        seqs = list(range(call.batch)) if rows is None else sorted(rows)
    q, k, v, table = host_inputs(wl, call, seqs)
    if call.kind == "prefill":
        sel_rows = rows if rows is not None else {b: np.arange(
            call.q_start_host[b + 1] - call.q_start_host[b]) for b in seqs}
        ref, _ = OA.paged_prefill(q, k, v, table, call.seq_lens_host, call.q_start_host,
                                  call.causal, wl.scale, rows=sel_rows, window=window)
    else:
        ref, _ = OA.paged_decode(q, k, v, table, call.seq_lens_host, wl.scale, seqs=seqs,
                                 window=window)
    return ref


def compare(got: np.ndarray, ref: np.ndarray, what: str, max_tol=MAX_ABS_TOL,
            mean_tol=MEAN_ABS_TOL):
    """Element-wise comparison over the entries the oracle evaluated (non-NaN)."""
    sel = ~np.isnan(ref)
    assert sel.any(), "nothing to compare"
    g, r = got[sel], ref[sel]
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    rms = float(np.sqrt(np.mean(r * r)))
    # the worst element against half a bf16 ulp of its reference value: the rounding
    # of the output itself, which no kernel can avoid
    w = int(np.argmax(err))
    half_ulp = 2.0 ** (np.floor(np.log2(max(abs(float(r[w])), 2.0 ** -126))) - 8)
    print(f"[parity] {what}: n={err.size} max_abs={err.max():.3e} mean_abs={err.mean():.3e} "
          f"rms_ref={rms:.3e} worst_ref={float(r[w]):.4f} half_ulp={half_ulp:.2e}", flush=True)
    assert err.max() <= max_tol, f"{what}: max abs error {err.max():.3e} > {max_tol}"
    assert err.mean() <= mean_tol, f"{what}: mean abs error {err.mean():.3e} > {mean_tol}"
    return float(err.max()), float(err.mean())


def spread_rows(q_len: int, n: int, seed: int, tile: int = 128):
    """Row sample: first/last rows, both sides of every few tile boundaries, random."""
    rng = np.random.default_rng(seed)
    picks = {0, q_len - 1}
    for t in range(tile, q_len, max(tile, q_len // 8 // tile * tile or tile)):
        picks.update({t - 1, t})
    picks.update(int(x) for x in rng.integers(0, q_len, size=n))
    return np.array(sorted(p for p in picks if 0 <= p < q_len))
