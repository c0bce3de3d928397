"""Benchmark of the paged-attention hot path on one MI355X.

Every workload of the set runs in the default invocation, each on seeded synthetic
inputs already resident in device memory, each kernel launch bracketed by HIP events
on the stream the library launches on (torch's current stream):

  decode_64               64 sequences x 1 query token, 32 heads, d=128, lengths
                          uniform on {512..8192}, 16-token pages in a shuffled pool.
                          One step = pa_decode_partial + pa_decode_combine.  `value`
                          is its KV bytes per second over whole steps (the headline);
                          `roofline` rates the split kernel alone against 8 TB/s.
  prefill_4096_causal     N=4096, 32 heads, d=128, identity table     -> `prefill`
  prefill_4096_noncausal  the same, non-causal                         -> `prefill_noncausal`
  prefill_32k             causal N=32768, 8 heads, shuffled pages of 256 -> `prefill_long`
  mixed_128x4             128 lognormal decode sequences + 4 causal 2048-row chunks
                          on 8192 cached tokens, one pool -> `mixed` (decode GB/s,
                          chunk TFLOP/s, combined T_roof / T_meas)
  prefill_600             the worked example's layout (600 tokens, table [5, 1, 9],
                          d=64): launch-latency bound, reported in microseconds
  next                    the rows beyond the core path (grouped heads, KV append,
                          page copy, sliding windows)             -> `next_rows`

Each kernel's rate uses its average event-timed launch (the figure rocprofv3's
average duration is compared with); median and minimum are reported beside it.
`input_sha256` holds a digest of every input buffer of every workload.
`cpu_baseline` times the CPU oracle over a pool of host processes on every workload
(whole decode sequences; all or every 2nd / 8th query row of the prefills and chunks)
and compares the oracle's outputs with the GPU outputs of the timed runs (`parity`).

Usage: python bench.py [--steps K] [--warmup W] [--legs a,b,...] [--no-cpu-baseline]
       [--no-digest]
Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-attn prefill TFLOP/s and decode KV GB/s on 1 MI355X (% of roofline)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "exact_tiled_attention_pa_amd", "csrc")
KERNEL_SOURCES = {
    "decode": ["decode.hip", "device_util.h", "lds_tile.h", "kernels.h"],
    "decode_gqa": ["decode_gqa.hip", "device_util.h", "lds_tile.h", "kernels.h"],
    "prefill": ["prefill.hip", "device_util.h", "lds_tile.h", "kernels.h"],
}
# file-name stem of each kernel's committed counter summary
KERNEL_FILES = {"decode": "decode_partial_kernel", "decode_gqa": "decode_gqa_kernel",
                "prefill": "prefill_kernel"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ algorithmic work

def visible_pairs(seq_lens, q_lens, causal: bool) -> int:
    """Visible (query, key) pairs per head; causal is bottom-right aligned."""
    total = 0
    for L, n in zip(seq_lens, q_lens):
        L, n = int(L), int(n)
        if causal:
            total += n * (L - n + 1) + n * (n - 1) // 2
        else:
            total += n * L
    return total


def prefill_work(wl, call):
    """(FLOPs, bytes): 4*d*Hq per visible pair; Q + O + valid K/V read or written once."""
    q_lens = call.q_start_host[1:] - call.q_start_host[:-1]
    hq = call.q.shape[1]
    d = wl.head_dim
    flops = 4 * d * hq * visible_pairs(call.seq_lens_host, q_lens, call.causal)
    nbytes = 2 * (2 * int(q_lens.sum()) * hq * d + 2 * int(call.seq_lens_host.sum()) * wl.heads * d)
    return flops, nbytes


def naive_attention_bytes(n: int, d: int, heads: int = 1) -> int:
    """HBM bytes of the unfused three-step kernel for n x n attention in 16-bit floats,
    8n^2 + 8nd per head: S and P each written and read once (8n^2), Q, K, V read and O
    written once (8nd) ("What do FlashAttention and PagedAttention actually optimize?",
    "Count the reads and writes FlashAttention removes")."""
    return heads * (8 * n * n + 8 * n * d)


def decode_kv_bytes(wl, call) -> int:
    """K and V bytes of every valid cached token (the decode metric)."""
    return int(call.seq_lens_host.astype("int64").sum()) * 2 * wl.heads * wl.head_dim * 2


# ------------------------------------------------------------------ traffic record

def source_digest(kind: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kind: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None if absent or
    if the kernel sources changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{KERNEL_FILES[kind]}.{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != source_digest(kind):
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_CYCLES")


def mfma_busy_fraction(mfma_busy_cycles, sq_cycles, simd_count, shader_engines):
    """Share of the kernel's duration the matrix cores were busy: SQ_VALU_MFMA_BUSY_CYCLES
    is summed over every SIMD and SQ_CYCLES over every shader engine's sequencer, so the
    kernel's duration in shader cycles is SQ_CYCLES / shader_engines."""
    return mfma_busy_cycles / (simd_count * sq_cycles / shader_engines)


def recorded_mfma(kind: str, workload: str):
    """Matrix-core busy fraction from the committed counter summary, or None if absent
    or if the kernel sources changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{KERNEL_FILES[kind]}.{workload}.mfma.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != source_digest(kind):
        return None
    try:
        return float(vals["mfma_busy_fraction"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ GPU legs

GQA_MIN_GROUP = 4  # query heads per K/V head from which the library runs decode_gqa_kernel


def decode_kind(wl) -> str:
    """Which pass-1 decode kernel the library runs for this head layout."""
    return "decode_gqa" if wl.num_q_heads // wl.heads >= GQA_MIN_GROUP else "decode"


# the library's choice between its two prefill kernels (prefill_split.h): the split-key
# kernel when its grid of 32-row workgroups fits one per CU and a sequence may span more
# than one 64-key tile, unless PA_PREFILL_PATH forces one
PREFILL_SPLIT_BLOCK_M = 32
PREFILL_SPLIT_MAX_WORKGROUPS = 512


def prefill_takes_split(wl, call) -> bool:
    path = os.environ.get("PA_PREFILL_PATH", "") or "auto"
    if path != "auto":
        return path == "split"
    wgs = wl.num_q_heads * call.batch * (-(-call.max_q_len // PREFILL_SPLIT_BLOCK_M))
    return (wgs <= PREFILL_SPLIT_MAX_WORKGROUPS and
            int(call.block_table.shape[1]) * wl.page_size > 64)


def prefill_kernel_name(wl, call) -> str:
    """The prefill instantiation a call runs: which kernel, head dim, causal and, for the
    tiled kernel, whether a key tile of 64 lies in one page (pages of 64 tokens or more)."""
    causal = str(bool(call.causal)).lower()
    if prefill_takes_split(wl, call):
        return f"prefill_split_kernel<{wl.head_dim}, {causal}>"
    return f"prefill_kernel<{wl.head_dim}, {causal}, {str(wl.page_size >= 64).lower()}>"


def decode_kernel_name(wl, call) -> str:
    """The pass-1 instantiation a decode call runs: the grouped-head kernel, or the
    one-head-per-row kernel with the split length the library picks for this batch
    (in steps of 32 keys)."""
    if decode_kind(wl) == "decode_gqa":
        return f"decode_gqa_kernel<{wl.head_dim}>"
    from exact_tiled_attention_pa_amd import binding as B
    split = B.pa_decode_split_tokens(call.batch, wl.num_q_heads,
                                     B.layout_of(wl.k_pool, call.block_table))
    return f"decode_partial_kernel<{wl.head_dim}, {split // 32}>"


def timing_stats(ms):
    """avg / median / min of a list of HIP-event durations (ms)."""
    s = sorted(ms)
    n = len(s)
    med = s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])
    return {"avg": sum(s) / n, "median": med, "min": s[0]}


def _ms(st, key):
    return round(st[key], 4)


def region_ms(fn, steps):
    """(wall s, ms per call) of `steps` back-to-back calls of fn, timed by one pair of
    HIP events around them on torch's current stream (the stream the library launches
    on) and by the host clock."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return time.perf_counter() - t0, e0.elapsed_time(e1) / steps


def paired_ms(fn, steps):
    """HIP-event duration (ms) of each of `steps` calls of fn, one event pair per call."""
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        fn()
        ev[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


class Timing:
    """A kernel's timed launches: `avg` (ms) from one event pair around `steps`
    back-to-back launches, the kernel's average launch duration; `pairs`, each launch of a
    second run of `steps` timed by its own event pair, for the median and minimum (the
    event commands between launches add 1-2 us to each of these)."""

    def __init__(self, avg, pairs):
        self.avg = avg
        self.pairs = pairs


def timed_decode(wl, call, out, steps, warmup):
    """K decode steps (pass 1 + combine); returns (wall s per K whole steps, pass-1
    Timing, combine Timing)."""
    import torch
    from exact_tiled_attention_pa_amd import binding as B
    ws = B.decode_workspace(call.q, wl.k_pool, call.block_table)
    lay = B.layout_of(wl.k_pool, call.block_table)

    def partial():
        B.pa_decode_partial(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens,
                            wl.scale, ws)

    def combine():
        B.pa_decode_combine(call.seq_lens, out, ws, lay)

    def step():
        partial()
        combine()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    wall, _ = region_ms(step, steps)
    _, p_avg = region_ms(partial, steps)
    _, c_avg = region_ms(combine, steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        partial()
        ev[i][1].record()
        combine()
        ev[i][2].record()
    torch.cuda.synchronize()
    step()  # the output of one whole step, for the digests and the baseline
    torch.cuda.synchronize()
    return (wall, Timing(p_avg, [e[0].elapsed_time(e[1]) for e in ev]),
            Timing(c_avg, [e[1].elapsed_time(e[2]) for e in ev]))


def timed_launches(fn, steps, warmup, warm_s=0.0):
    """(wall s, Timing) of `steps` launches of fn on torch's current stream, after
    `warmup` untimed ones and, with warm_s > 0, after untimed launches for at least
    warm_s seconds (the chip's clock settles under sustained load)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + warm_s
    while time.perf_counter() < t_end:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
    wall, avg = region_ms(fn, steps)
    return wall, Timing(avg, paired_ms(fn, steps))


def _rate(work, timing, peak, unit, **extra):
    """Rate of one kernel against its peak from its average launch duration, with the
    median and minimum of the per-launch timings beside it."""
    st = timing_stats(timing.pairs)
    scale = 1e9 if unit == "GB/s" else 1e12
    achieved = work / (timing.avg * 1e-3) / scale
    return dict(extra, achieved=round(achieved, 2), unit=unit, peak=peak,
                frac=round(achieved / peak, 4), kernel_ms_avg=round(timing.avg, 4),
                kernel_ms_median=_ms(st, "median"), kernel_ms_min=_ms(st, "min"),
                kernel_ms_avg_paired=_ms(st, "avg"))


def decode_leg(wl, call, steps, warmup):
    """decode: KV bytes per second over whole steps, and pass 1 against 8 TB/s."""
    import torch
    nbytes = decode_kv_bytes(wl, call)
    out = torch.empty_like(call.q)
    wall, split_t, comb_t = timed_decode(wl, call, out, steps, warmup)
    ms_step = wall / steps * 1e3
    roof = _rate(nbytes, split_t, HBM_PEAK_GBS, "GB/s", bound="hbm",
                 kernel=decode_kernel_name(wl, call))
    cst = timing_stats(comb_t.pairs)
    roof.update(traffic=recorded_traffic(decode_kind(wl), wl.name),
                combine_ms_avg=round(comb_t.avg, 4), combine_ms_median=_ms(cst, "median"))
    res = {"workload": wl.name, "gbs": round(nbytes / (ms_step * 1e-3) / 1e9, 2),
           "ms_per_step": round(ms_step, 4), "kv_bytes_per_step": nbytes,
           "total_tokens": int(call.seq_lens_host.sum()), "roofline": roof}
    return res, out


# untimed prefill launches before each prefill leg's timed region: the shader clock
# takes tens of milliseconds of sustained MFMA load to settle after the chip has idled
# (input generation between legs); half a second reaches the steady state a serving
# loop runs at
PREFILL_WARM_S = 0.5


def prefill_leg(wl, call, steps, warmup):
    """prefill: FLOPs of the visible pairs against 2.5 PFLOP/s, per launch."""
    import torch
    from exact_tiled_attention_pa_amd import binding as B
    flops, nbytes = prefill_work(wl, call)
    out = torch.empty_like(call.q)
    # validated and marshalled once: each timed launch is one C call, so short launches
    # (the 600-token example) are not paced by the binding's per-call checks
    run = B.PreparedPrefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens,
                            call.causal, wl.scale, out, call.q_start, call.max_q_len).launch

    wall, tm = timed_launches(run, steps, warmup, warm_s=PREFILL_WARM_S)
    roof = _rate(flops, tm, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", bound="mfma",
                 kernel=prefill_kernel_name(wl, call))
    wl_key = wl.name if len(wl.calls) == 1 else f"{wl.name}_chunks"
    roof.update(traffic=recorded_traffic("prefill", wl_key),
                mfma_busy=recorded_mfma("prefill", wl_key))
    res = {"workload": wl.name, "causal": call.causal, "tflops": roof["achieved"],
           "kernel_ms_avg": roof["kernel_ms_avg"], "kernel_ms_median": roof["kernel_ms_median"],
           "kernel_ms_min": roof["kernel_ms_min"],
           "us_per_call_wall": round(wall / steps * 1e6, 2), "flops_per_launch": flops,
           "alg_bytes_per_launch": nbytes, "roofline": roof}
    n = int(call.seq_lens_host[0])
    if call.batch == 1 and int(call.q_start_host[1]) == n:
        # one square n x n attention per head: what the unfused kernel would move
        naive = naive_attention_bytes(n, wl.head_dim, wl.num_q_heads)
        res["naive_traffic"] = {
            "bytes": naive, "formula": "heads * (8 N^2 + 8 N d)",
            "measured_over_naive": (round(roof["traffic"] / naive, 4)
                                    if roof.get("traffic") else None)}
    return res, out


def mixed_leg(wl, steps, warmup):
    """mixed batch: the decode call and the chunk prefill over one pool, each timed, and
    the combined fraction T_roof / T_meas with T_roof = bytes / 8 TB/s + FLOPs / 2.5 PF."""
    dec, dec_out = decode_leg(wl, wl.calls[0], steps, warmup)
    chunks, pre_out = prefill_leg(wl, wl.calls[1], steps, warmup)
    t_roof = dec["kv_bytes_per_step"] / (HBM_PEAK_GBS * 1e9) + chunks["flops_per_launch"] / (
        MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_meas = (dec["roofline"]["kernel_ms_avg"] + dec["roofline"]["combine_ms_avg"] +
              chunks["kernel_ms_avg"]) * 1e-3
    res = {"workload": wl.name, "decode": dec, "chunks": chunks,
           "combined_roofline_fraction": round(t_roof / t_meas, 4),
           "combined_ms": round(t_meas * 1e3, 4)}
    return res, (dec_out, pre_out)


def next_rows_summary(decode_wl, steps, warmup):
    """Throughput of the rows beyond the core path, each against its own roofline:
    grouped-head decode, KV append, page copy, sliding-window prefill and decode."""
    import numpy as np
    import torch
    from exact_tiled_attention_pa_amd import binding as B
    from exact_tiled_attention_pa_amd import workloads as W

    res = {}
    # f4, decode: the decode_64 batch with a 1024-token window
    call = decode_wl.calls[0]
    ws = B.decode_workspace(call.q, decode_wl.k_pool, call.block_table)
    out = torch.empty_like(call.q)
    w = 1024
    _, tm = timed_launches(lambda: B.pa_decode(call.q, decode_wl.k_pool, decode_wl.v_pool,
                                               call.block_table, call.seq_lens,
                                               decode_wl.scale, out, ws, window=w),
                           steps, warmup)
    seen = np.minimum(call.seq_lens_host.astype(np.int64), w).sum()
    nbytes = int(seen) * 2 * decode_wl.heads * decode_wl.head_dim * 2
    res["window_decode"] = _rate(nbytes, tm, HBM_PEAK_GBS, "GB/s", bound="hbm",
                                 workload=f"decode_64, window {w}",
                                 kernel=decode_kernel_name(decode_wl, call) + " + combine")
    del ws, out

    # f1: grouped heads
    g = W.decode_64_gqa8(device="cuda")
    gc = g.calls[0]
    ws = B.decode_workspace(gc.q, g.k_pool, gc.block_table)
    _, tm = timed_launches(lambda: B.pa_decode_partial(gc.q, g.k_pool, g.v_pool,
                                                       gc.block_table, gc.seq_lens, g.scale,
                                                       ws), steps, warmup)
    res["gqa_decode"] = _rate(decode_kv_bytes(g, gc), tm, HBM_PEAK_GBS, "GB/s", bound="hbm",
                              workload=g.name, kernel=decode_kernel_name(g, gc),
                              traffic=recorded_traffic("decode_gqa", g.name))
    del g, gc, ws

    # f2: appending a 4096-token chunk of one sequence (32 K/V heads, d=128, pages of 16)
    n_tok, heads, d, ps = 4096, 32, 128, 16
    a = W.build("append_4096", 11, heads=heads, head_dim=d, page_size=ps, lens=[n_tok],
                kind="decode", pool_slack=1.25, device="cuda")
    ac = a.calls[0]
    k_new = W.normal_bf16((n_tok, heads, d), 1.0, 12, "cuda")
    v_new = W.normal_bf16((n_tok, heads, d), 1.0, 13, "cuda")
    ids = torch.zeros(n_tok, dtype=torch.int32, device="cuda")
    pos = torch.arange(n_tok, dtype=torch.int32, device="cuda")
    _, tm = timed_launches(lambda: B.pa_kv_append(k_new, v_new, ids, pos, a.k_pool, a.v_pool,
                                                  ac.block_table), steps, warmup)
    nbytes = n_tok * heads * d * 2 * 2 * 2  # K and V rows, read once and written once
    res["kv_append"] = _rate(nbytes, tm, HBM_PEAK_GBS, "GB/s", bound="hbm",
                             workload="append_4096: 4096 tokens, 32 K/V heads, d=128, "
                                      "pages of 16, shuffled", kernel="kv_append_kernel")
    del a, ac, k_new, v_new, ids, pos

    # f3: copy-on-write page copies: 2048 disjoint page pairs in a 4096-page pool
    n_pages, n_pairs = 4096, 2048
    kp = W.normal_bf16((n_pages, ps, heads, d), 1.0, 14, "cuda")
    vp = W.normal_bf16((n_pages, ps, heads, d), 1.0, 15, "cuda")
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(16))
    src = perm[:n_pairs].to(torch.int32).cuda()
    dst = perm[n_pairs:2 * n_pairs].to(torch.int32).cuda()
    _, tm = timed_launches(lambda: B.pa_copy_pages(kp, vp, src, dst), steps, warmup)
    page_bytes = ps * heads * d * 2
    nbytes = n_pairs * page_bytes * 2 * 2  # both pools, read and write
    res["copy_pages"] = _rate(nbytes, tm, HBM_PEAK_GBS, "GB/s", bound="hbm",
                              workload=f"copy_2048: {n_pairs} page pairs of 16 tokens x 32 "
                                       "heads x d=128", kernel="copy_pages_kernel")
    del kp, vp, src, dst

    # f4, prefill: prefill_32k with a 4096-token window
    p = W.prefill_32k(device="cuda")
    pc = p.calls[0]
    out = torch.empty_like(pc.q)
    w = 4096
    _, tm = timed_launches(lambda: B.pa_prefill(pc.q, p.k_pool, p.v_pool, pc.block_table,
                                                pc.seq_lens, True, p.scale, out, pc.q_start,
                                                pc.max_q_len, window=w), steps, warmup,
                           warm_s=PREFILL_WARM_S)
    n = int(pc.seq_lens_host[0])
    pairs = w * (w + 1) // 2 + (n - w) * w
    flops = 4 * p.head_dim * pc.q.shape[1] * pairs
    res["window_prefill"] = _rate(flops, tm, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", bound="mfma",
                                  workload=f"prefill_32k, window {w}",
                                  kernel=prefill_kernel_name(p, pc))
    del p, pc, out
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ CPU baseline (oracle)
#
# The oracle as it stands (NumPy fp64, oracle/attention.py), never tuned for speed, run
# over a process pool of the host's cores (one BLAS thread per process) on whole decode
# sequences or on query rows of a prefill.  Inputs are the same host bit patterns the GPU
# legs ran on, written once to files the workers memory-map.  The oracle's outputs for the
# evaluated rows are also compared with the GPU outputs of the timed runs.

_WORKER_CACHE = {}
_BLAS_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def _worker_init(_=None):
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def _worker_arrays(paths):
    import numpy as np
    key = tuple(paths)
    if key not in _WORKER_CACHE:
        _WORKER_CACHE.clear()
        _WORKER_CACHE[key] = [np.load(p, mmap_mode="r") for p in paths]
    return _WORKER_CACHE[key]


def _oracle_task(task):
    """One unit of oracle work in a pool worker: decode of some sequences, or some query
    rows of one prefill sequence.  Returns (outputs of those rows, seconds spent)."""
    from oracle import attention as OA
    kind, paths, meta, sel = task
    q, k, v, table, lens = _worker_arrays(paths)[:5]
    t0 = time.perf_counter()
    if kind == "decode":
        out, _ = OA.paged_decode(q, k, v, table, lens, meta["scale"], seqs=sel)
        res = out[sel]
    else:
        q_start = _worker_arrays(paths)[5]
        b, rows = sel
        out, _ = OA.paged_prefill(q, k, v, table, lens, q_start, meta["causal"], meta["scale"],
                                  rows={b: rows})
        res = out[int(q_start[b]) + rows]
    return res, time.perf_counter() - t0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_workers() -> int:
    """Processes for the oracle pool: the host cores this process may run on, at most 16
    (the host share of one GPU on the measurement machines)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _parity(got_bits, ref):
    """max / mean |O_gpu - O_ref| and the largest per-(row, head) max error divided by
    that row's RMS(O_ref), over the rows the oracle evaluated."""
    import numpy as np
    from oracle import attention as OA
    got = OA.bf16_to_f64(got_bits)
    err = np.abs(got - ref)
    rms = np.sqrt(np.mean(ref * ref, axis=-1))
    ratio = err.max(axis=-1) / np.maximum(rms, 1e-300)
    return {"elements": int(err.size), "max_abs": float(f"{err.max():.4e}"),
            "mean_abs": float(f"{err.mean():.4e}"),
            "max_err_over_rms_ref": float(f"{ratio.max():.4e}"),
            "within_tolerance": bool(err.max() <= 1e-2 and err.mean() <= 1e-3)}


def cpu_baseline(legs, scratch_dir):
    """Times the oracle over a process pool on each leg's sample; returns the baseline
    record (headline: decode GB/s) with one entry per leg, each with parity figures."""
    import multiprocessing as mp

    import numpy as np

    from exact_tiled_attention_pa_amd import workloads as W

    n = cpu_workers()
    ctx = mp.get_context("spawn")
    entries = {}
    total = 0.0
    # one BLAS thread per worker process, fixed before the workers import NumPy
    saved = {k: os.environ.get(k) for k in _BLAS_THREAD_VARS}
    os.environ.update({k: "1" for k in _BLAS_THREAD_VARS})
    try:
        pool = ctx.Pool(n, initializer=_worker_init)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    with pool:
        pool.map(_worker_init, range(n))  # workers up and imported before any timing
        for name, (wl, call, out, sample) in legs.items():
            base = os.path.join(scratch_dir, name)
            arrays = [W.to_host_bits(call.q), W.to_host_bits(wl.k_pool),
                      W.to_host_bits(wl.v_pool), call.block_table_host.astype(np.int64),
                      call.seq_lens_host.astype(np.int64)]
            if call.kind == "prefill":
                arrays.append(call.q_start_host.astype(np.int64))
            paths = []
            for i, a in enumerate(arrays):
                p = f"{base}_{i}.npy"
                np.save(p, a)
                paths.append(p)
            del arrays
            meta = {"scale": wl.scale, "causal": call.causal}
            if call.kind == "decode":
                tasks = [("decode", paths, meta, [int(b)]) for b in sample]
            else:
                tasks = [("prefill", paths, meta, piece) for piece in sample]
            t0 = time.perf_counter()
            results = pool.map(_oracle_task, tasks, chunksize=1)
            wall = time.perf_counter() - t0
            total += wall
            got = W.to_host_bits(out)
            if call.kind == "decode":
                ref = np.concatenate([r for r, _ in results])
                rows_bits = got[np.asarray(sample)]
                work = sum(int(call.seq_lens_host[b]) for b in sample) * 2 * wl.heads * \
                    wl.head_dim * 2
                rate, unit = work / wall / 1e9, "GB/s"
                what = (f"{len(sample)} whole decode sequences ({sum(int(call.seq_lens_host[b]) for b in sample)} "
                        f"tokens, all {wl.num_q_heads} query heads)")
            else:
                ref = np.concatenate([r for r, _ in results])
                qs = call.q_start_host
                rows_bits = got[np.concatenate([int(qs[b]) + rows for b, rows in sample])]
                pairs = n_rows = 0
                for b, rows in sample:
                    L, q_len = int(call.seq_lens_host[b]), int(qs[b + 1] - qs[b])
                    pos = L - q_len + rows
                    pairs += int(np.minimum(pos + 1, L).sum()) if call.causal else L * len(rows)
                    n_rows += len(rows)
                work = 4 * wl.head_dim * wl.num_q_heads * pairs
                rate, unit = work / wall / 1e12, "TFLOP/s"
                n_seqs = len({b for b, _ in sample})
                what = (f"{n_rows} of {int(qs[-1])} query rows spread over "
                        f"{n_seqs} sequence{'s' if n_seqs > 1 else ''}, all "
                        f"{wl.num_q_heads} heads ({pairs} visible pairs per head)")
            entries[name] = {"value": round(rate, 6), "unit": unit, "wall_s": round(wall, 2),
                             "cpu_s": round(sum(t for _, t in results), 2), "sample": what,
                             "parity": _parity(rows_bits, ref)}
            for p in paths:
                os.remove(p)
            _WORKER_CACHE.clear()
            log(f"cpu baseline {name}: {rate:.4g} {unit} in {wall:.1f} s, "
                f"parity {entries[name]['parity']}")
    head = entries.get("decode_64") or next(iter(entries.values()))
    return {"value": head["value"], "unit": head["unit"], "cores": n, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"oracle (NumPy fp64, one BLAS thread per process, {n} processes) on "
                      f"{head['sample']}; {total:.1f} s wall over all legs",
            "legs": entries}


# every how-many-th query row of each sequence the oracle evaluates (1: all of them)
BASELINE_ROW_STRIDE = {"prefill_32k": 8, "mixed_128x4_chunks": 8, "prefill_4096_noncausal": 2}


def baseline_samples(name, wl, call):
    """What the oracle evaluates for each leg: whole decode sequences, or (sequence,
    query rows) tasks of up to 32 rows, every row-stride-th row of each sequence from an
    offset."""
    import numpy as np
    if call.kind == "decode":
        return list(range(call.batch))
    stride = BASELINE_ROW_STRIDE.get(name, 1)
    per_task = 32
    tasks = []
    for b in range(call.batch):
        q_len = int(call.q_start_host[b + 1] - call.q_start_host[b])
        rows = np.arange(stride // 2, q_len, stride, dtype=np.int64)
        tasks += [(b, rows[i:i + per_task]) for i in range(0, len(rows), per_task)]
    return tasks


# ------------------------------------------------------------------ rocprofv3 summaries

KERNEL_TAGS = {"decode": "decode_partial_kernel", "decode_gqa": "decode_gqa_kernel",
               "prefill": "prefill_kernel<128, true",
               "prefill_noncausal": "prefill_kernel<128, false"}


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_trace(trace_dir, out_path, command):
    """Writes the kernel-trace statistics of a rocprofv3 --kernel-trace --stats run."""
    rows = _read_csv(os.path.join(trace_dir, "run_kernel_stats.csv"))
    lines = ["# rocprofv3 kernel statistics (durations in microseconds)",
             f"# command: {command}",
             f"# {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}  kernel"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "")
        short = name.split("(")[0].replace("void ", "")
        lines.append(f"  {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                     f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f}  {short}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_traffic(fetch_dir, write_dir, kind, workload, out_path, command):
    """HBM bytes per launch of one kernel from FETCH_SIZE and WRITE_SIZE runs, each
    scaled by what the same counter reads for a plain 1 GiB device copy."""
    tag = KERNEL_TAGS[kind]
    gib_kib = float(1 << 20)
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _read_csv(os.path.join(d, "run_counter_collection.csv"))
                if r["Counter_Name"] == counter]
        copies = [float(r["Counter_Value"]) for r in rows
                  if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) >= 131072
                  and float(r["Counter_Value"]) > gib_kib / 4]
        kern = [float(r["Counter_Value"]) for r in rows if tag in r["Kernel_Name"]]
        if not copies or not kern:
            raise SystemExit(f"{counter}: no calibration copy or no {tag} dispatch in {d}")
        factor = gib_kib / (sum(copies) / len(copies))
        res[counter] = (sum(kern) / len(kern), factor, len(kern))
    fetch_kib, f_fac, n = res["FETCH_SIZE"]
    write_kib, w_fac, _ = res["WRITE_SIZE"]
    hbm = (fetch_kib * f_fac + write_kib * w_fac) * 1024
    src = kind if kind in KERNEL_SOURCES else "prefill"
    lines = [f"# HBM traffic per launch of {tag} on workload {workload}",
             f"# command (run twice, once per counter): {command}",
             "# each counter is scaled by (1 GiB / its reading for a plain 1 GiB device copy);",
             "# bench.py reports this figure only while source_sha256 matches the kernel sources",
             f"kernel={tag}",
             f"workload={workload}",
             f"dispatches={n}",
             f"fetch_kib_raw={fetch_kib:.1f}",
             f"fetch_copy_factor={f_fac:.4f}",
             f"write_kib_raw={write_kib:.1f}",
             f"write_copy_factor={w_fac:.4f}",
             f"hbm_bytes_per_launch={hbm:.0f}",
             f"source_sha256={source_digest(src)}"]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_mfma(pmc_dir, kind, workload, out_path, command):
    """Matrix-core busy fraction of one kernel from a --pmc run of MFMA_COUNTERS,
    averaged over its dispatches, with the GPU's SIMD and shader-engine counts taken
    from the same run's agent table."""
    tag = KERNEL_TAGS[kind]
    per = {}
    for r in _read_csv(os.path.join(pmc_dir, "run_counter_collection.csv")):
        if tag in r["Kernel_Name"] and r["Counter_Name"] in MFMA_COUNTERS:
            per.setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
    per = {k: v for k, v in per.items() if len(v) == len(MFMA_COUNTERS)}
    gpus = [a for a in _read_csv(os.path.join(pmc_dir, "run_agent_info.csv"))
            if a.get("Agent_Type", "").strip('"') == "GPU"]
    if not per or not gpus:
        raise SystemExit(f"no {tag} dispatch with {MFMA_COUNTERS} or no GPU agent in {pmc_dir}")
    simds, engines = int(gpus[0]["Simd_Count"]), int(gpus[0]["Num_Shader_Banks"])
    fr = [mfma_busy_fraction(v["SQ_VALU_MFMA_BUSY_CYCLES"], v["SQ_CYCLES"], simds, engines)
          for v in per.values()]
    cyc = [v["SQ_CYCLES"] / engines for v in per.values()]
    src = kind if kind in KERNEL_SOURCES else "prefill"
    lines = [f"# matrix-core busy fraction of {tag} on workload {workload}",
             f"# command: {command}",
             "# fraction = SQ_VALU_MFMA_BUSY_CYCLES / (simd_count * SQ_CYCLES / shader_engines),",
             "# averaged over dispatches; bench.py reports it only while source_sha256 matches",
             f"kernel={tag}",
             f"workload={workload}",
             f"dispatches={len(fr)}",
             f"simd_count={simds}",
             f"shader_engines={engines}",
             f"shader_cycles_per_launch={sum(cyc) / len(cyc):.0f}",
             f"mfma_busy_fraction={sum(fr) / len(fr):.4f}",
             f"source_sha256={source_digest(src)}"]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ------------------------------------------------------------------ main

LEGS = ("decode_64", "prefill_4096_causal", "prefill_4096_noncausal", "prefill_32k",
        "mixed_128x4", "prefill_600", "next")
# the oracle's legs, in the order they run; the mixed batch gives two (its decode call
# and its chunk prefill)
BASELINE_LEGS = ("decode_64", "prefill_4096_causal", "prefill_4096_noncausal", "prefill_32k",
                 "mixed_128x4_decode", "mixed_128x4_chunks", "prefill_600")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma-separated legs to run (default: all): " + ", ".join(LEGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-digest", action="store_true",
                    help="skip the SHA-256 of every input buffer")
    ap.add_argument("--prefill-warm-s", type=float, default=0.5,
                    help="seconds of untimed launches before each prefill leg (profiling "
                         "runs shorten it)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "OUT"),
                    help="write a kernel-statistics summary of a rocprofv3 run and exit")
    ap.add_argument("--summarize-traffic", nargs=5,
                    metavar=("FETCH_DIR", "WRITE_DIR", "KIND", "WORKLOAD", "OUT"),
                    help="write the calibrated HBM traffic of one kernel and exit")
    ap.add_argument("--summarize-mfma", nargs=4, metavar=("PMC_DIR", "KIND", "WORKLOAD", "OUT"),
                    help="write the matrix-core busy fraction of one kernel and exit")
    ap.add_argument("--profile-command", default="",
                    help="the command recorded in a summary")
    args = ap.parse_args()
    globals()["PREFILL_WARM_S"] = args.prefill_warm_s
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.profile_command)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.profile_command)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma, args.profile_command)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)
    legs = [x for x in args.legs.split(",") if x]
    unknown = [x for x in legs if x not in LEGS]
    if unknown:
        raise SystemExit(f"unknown legs {unknown}; choose from {LEGS}")

    import torch
    from exact_tiled_attention_pa_amd import binding as B
    from exact_tiled_attention_pa_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.load_library()
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "bf16", "data": "synthetic"}
    kept = {}      # leg -> (workload, call, GPU output) for the digests and the baseline
    workloads = {}
    # the headline legs run first: the clock the chip holds depends on how long it has
    # been loaded, and the prefill legs warm up for at least 10 launches
    for leg in legs:
        if leg == "next":
            continue
        log(f"leg {leg}: generating inputs")
        wl = W.FULL_WORKLOADS[leg](device="cuda")
        torch.cuda.synchronize()
        workloads[leg] = wl
        if leg == "decode_64":
            res, out = decode_leg(wl, wl.calls[0], args.steps, args.warmup)
            kept[leg] = (wl, wl.calls[0], out)
            result.update({
                "value": res["gbs"], "unit": "GB/s", "ms_per_step": res["ms_per_step"],
                "config": {"workload": wl.name, "batch": wl.calls[0].batch,
                           "heads": wl.num_q_heads, "kv_heads": wl.heads,
                           "head_dim": wl.head_dim, "page_size": wl.page_size,
                           "total_tokens": res["total_tokens"],
                           "kv_bytes_per_step": res["kv_bytes_per_step"],
                           "description": wl.description},
                "roofline": res["roofline"],
            })
        elif leg == "mixed_128x4":
            res, (dout, pout) = mixed_leg(wl, args.steps, max(args.warmup, 10))
            kept["mixed_128x4_decode"] = (wl, wl.calls[0], dout)
            kept["mixed_128x4_chunks"] = (wl, wl.calls[1], pout)
            result["mixed"] = res
        else:
            res, out = prefill_leg(wl, wl.calls[0], args.steps,
                                   max(args.warmup, 3 if leg == "prefill_32k" else 10))
            kept[leg] = (wl, wl.calls[0], out)
            key = {"prefill_4096_causal": "prefill", "prefill_4096_noncausal": "prefill_noncausal",
                   "prefill_32k": "prefill_long", "prefill_600": "prefill_600"}[leg]
            result[key] = res
        log(f"leg {leg}: done")
    if "value" not in result and "mixed" in result:  # the mixed batch's decode heads it
        d = result["mixed"]["decode"]
        result.update({"value": d["gbs"], "unit": "GB/s", "ms_per_step": d["ms_per_step"],
                       "config": {"workload": d["workload"]}, "roofline": d["roofline"]})
    prefills = [k for k in ("prefill", "prefill_noncausal", "prefill_long", "prefill_600")
                if k in result]
    if "value" not in result and prefills:  # no decode leg: the first prefill leg heads it
        s = result[prefills[0]]
        result.update({"value": s["tflops"], "unit": "TFLOP/s",
                       "ms_per_step": round(s["us_per_call_wall"] / 1e3, 4),
                       "config": {"workload": s["workload"], "causal": s["causal"]},
                       "roofline": s["roofline"]})

    if "next" in legs:
        log("rows beyond the core path: grouped heads, append, page copy, windows")
        dwl = workloads.get("decode_64") or W.decode_64(device="cuda")
        result["next_rows"] = next_rows_summary(dwl, args.steps, args.warmup)
        if "value" not in result:  # only these rows ran: the grouped-head decode heads it
            g = result["next_rows"]["gqa_decode"]
            result.update({"value": g["achieved"], "unit": g["unit"],
                           "ms_per_step": g["kernel_ms_avg"],
                           "config": {"workload": g["workload"]}, "roofline": g})

    if not args.no_digest:
        log("SHA-256 of every input buffer")
        result["input_sha256"] = {name: wl.digest() for name, wl in workloads.items()}
        if "config" in result and result["config"].get("workload") in result["input_sha256"]:
            result["config"]["input_sha256"] = result["input_sha256"][result["config"]["workload"]]

    # the oracle runs last, after every GPU leg, so its host time cannot idle the GPU
    # between a warm-up and a timed region
    if not args.no_cpu_baseline:
        todo = {k: kept[k] for k in BASELINE_LEGS if k in kept}
        if todo:
            import shutil
            import tempfile
            log(f"cpu baseline (oracle) on {cpu_workers()} processes: {sorted(todo)}")
            scratch = tempfile.mkdtemp(prefix="pa_oracle_",
                                       dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
            try:
                samples = {k: (wl, call, out, baseline_samples(k, wl, call))
                           for k, (wl, call, out) in todo.items()}
                result["cpu_baseline"] = cpu_baseline(samples, scratch)
            finally:
                shutil.rmtree(scratch, ignore_errors=True)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
