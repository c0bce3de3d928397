"""Benchmark of the paged-attention hot path on one MI355X.

Default workload: decode_64 (64 sequences x 1 query token, 32 heads, d=128,
lengths uniform on {512..8192}, 16-token pages in a shuffled pool).  One step is
one pa_decode over the batch (the split pass and the combine pass, issued as
pa_decode_partial + pa_decode_combine so each kernel can be timed with HIP events
on the stream it runs on).  `value` is algorithmic KV bytes per second over whole
steps; `roofline` rates the split kernel alone against 8 TB/s.  A `prefill` object
times the causal N=4096 prefill (32 heads, d=128) against the 2.5 PFLOP/s dense
bf16 MFMA peak.  `cpu_baseline` times the CPU oracle on a bounded sample.

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
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


def decode_kernel_name(wl) -> str:
    return f"{KERNEL_FILES[decode_kind(wl)]}<{wl.head_dim}>"


def timed_decode(wl, call, steps, warmup):
    import torch
    from exact_tiled_attention_pa_amd import binding as B
    ws = B.decode_workspace(call.q, wl.k_pool, call.block_table)
    out = torch.empty_like(call.q)
    lay = B.layout_of(wl.k_pool, call.block_table)

    def step():
        B.pa_decode_partial(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens,
                            wl.scale, ws)
        B.pa_decode_combine(call.seq_lens, out, ws, lay)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        B.pa_decode_partial(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens,
                            wl.scale, ws)
        ev[i][1].record()
        B.pa_decode_combine(call.seq_lens, out, ws, lay)
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    split_ms = [e[0].elapsed_time(e[1]) for e in ev]
    comb_ms = [e[1].elapsed_time(e[2]) for e in ev]
    return wall, split_ms, comb_ms


def timed_prefill(wl, call, steps, warmup):
    import torch
    from exact_tiled_attention_pa_amd import binding as B
    out = torch.empty_like(call.q)

    def run():
        B.pa_prefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens,
                     call.causal, wl.scale, out, call.q_start, call.max_q_len)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        run()
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [e[0].elapsed_time(e[1]) for e in ev]


def timed_launches(fn, steps, warmup):
    """HIP-event durations (ms) of `steps` launches of fn on torch's current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        fn()
        ev[i][1].record()
    torch.cuda.synchronize()
    return [e[0].elapsed_time(e[1]) for e in ev]


def _rate(nbytes_or_flops, ms, peak, unit, **extra):
    avg = sum(ms) / len(ms)
    scale = 1e9 if unit == "GB/s" else 1e12
    achieved = nbytes_or_flops / (avg * 1e-3) / scale
    return dict(extra, achieved=round(achieved, 2), unit=unit, peak=peak,
                frac=round(achieved / peak, 4), kernel_ms_avg=round(avg, 4))


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
    ms = timed_launches(lambda: B.pa_decode(call.q, decode_wl.k_pool, decode_wl.v_pool,
                                            call.block_table, call.seq_lens, decode_wl.scale,
                                            out, ws, window=w), steps, warmup)
    seen = np.minimum(call.seq_lens_host.astype(np.int64), w).sum()
    nbytes = int(seen) * 2 * decode_wl.heads * decode_wl.head_dim * 2
    res["window_decode"] = _rate(nbytes, ms, HBM_PEAK_GBS, "GB/s", bound="hbm",
                                 workload=f"decode_64, window {w}",
                                 kernel="decode_partial_kernel<128> + decode_combine_kernel<128>")
    del ws, out

    # f1: grouped heads
    g = W.decode_64_gqa8(device="cuda")
    gc = g.calls[0]
    ws = B.decode_workspace(gc.q, g.k_pool, gc.block_table)
    out = torch.empty_like(gc.q)
    ms = timed_launches(lambda: B.pa_decode_partial(gc.q, g.k_pool, g.v_pool, gc.block_table,
                                                    gc.seq_lens, g.scale, ws), steps, warmup)
    res["gqa_decode"] = _rate(decode_kv_bytes(g, gc), ms, HBM_PEAK_GBS, "GB/s", bound="hbm",
                              workload=g.name, kernel=decode_kernel_name(g))
    del g, gc, ws, out

    # f2: appending a 4096-token chunk of one sequence (32 K/V heads, d=128, pages of 16)
    n_tok, heads, d, ps = 4096, 32, 128, 16
    a = W.build("append_4096", 11, heads=heads, head_dim=d, page_size=ps, lens=[n_tok],
                kind="decode", pool_slack=1.25, device="cuda")
    ac = a.calls[0]
    k_new = W.normal_bf16((n_tok, heads, d), 1.0, 12, "cuda")
    v_new = W.normal_bf16((n_tok, heads, d), 1.0, 13, "cuda")
    ids = torch.zeros(n_tok, dtype=torch.int32, device="cuda")
    pos = torch.arange(n_tok, dtype=torch.int32, device="cuda")
    ms = timed_launches(lambda: B.pa_kv_append(k_new, v_new, ids, pos, a.k_pool, a.v_pool,
                                               ac.block_table), steps, warmup)
    nbytes = n_tok * heads * d * 2 * 2 * 2  # K and V rows, read once and written once
    res["kv_append"] = _rate(nbytes, ms, HBM_PEAK_GBS, "GB/s", bound="hbm",
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
    ms = timed_launches(lambda: B.pa_copy_pages(kp, vp, src, dst), steps, warmup)
    page_bytes = ps * heads * d * 2
    nbytes = n_pairs * page_bytes * 2 * 2  # both pools, read and write
    res["copy_pages"] = _rate(nbytes, ms, HBM_PEAK_GBS, "GB/s", bound="hbm",
                              workload=f"copy_2048: {n_pairs} page pairs of 16 tokens x 32 "
                                       "heads x d=128", kernel="copy_pages_kernel")
    del kp, vp, src, dst

    # f4, prefill: prefill_32k with a 4096-token window
    p = W.prefill_32k(device="cuda")
    pc = p.calls[0]
    out = torch.empty_like(pc.q)
    w = 4096
    ms = timed_launches(lambda: B.pa_prefill(pc.q, p.k_pool, p.v_pool, pc.block_table,
                                             pc.seq_lens, True, p.scale, out, pc.q_start,
                                             pc.max_q_len, window=w), steps, warmup)
    n = int(pc.seq_lens_host[0])
    pairs = w * (w + 1) // 2 + (n - w) * w
    flops = 4 * p.head_dim * pc.q.shape[1] * pairs
    res["window_prefill"] = _rate(flops, ms, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", bound="mfma",
                                  workload=f"prefill_32k, window {w}", kernel="prefill_kernel")
    del p, pc, out
    torch.cuda.empty_cache()
    return res


def prefill_summary(wl, call, steps, warmup):
    flops, nbytes = prefill_work(wl, call)
    wall, ms = timed_prefill(wl, call, steps, warmup)
    avg = sum(ms) / len(ms)
    tflops = flops / (avg * 1e-3) / 1e12
    traffic = recorded_traffic("prefill", wl.name)
    mfma_busy = recorded_mfma("prefill", wl.name) if call.causal else None
    return {
        "workload": wl.name,
        "tflops": round(tflops, 2),
        "kernel_ms_avg": round(avg, 4),
        "kernel_ms_min": round(min(ms), 4),
        "ms_per_call_wall": round(wall / steps * 1e3, 4),
        "flops_per_launch": flops,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "mfma_busy": mfma_busy},
        "alg_bytes_per_launch": nbytes,
    }


# ------------------------------------------------------------------ CPU baseline

def cpu_baseline_decode(wl, call, budget_s=10.0):
    """The oracle as it stands, single BLAS thread, on whole sequences of the same
    batch, in order and wrapping around, until about budget_s seconds of CPU work;
    reported in GB/s of KV read.  Host copies of the pages are not timed."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from exact_tiled_attention_pa_amd import workloads as W
    from oracle import attention as OA

    q = W.to_host_bits(call.q)
    done_bytes = 0
    done_tokens = 0
    spent = 0.0
    count = 0
    with threadpool_limits(limits=1):
        while spent < budget_s:
            b = count % call.batch
            L = int(call.seq_lens_host[b])
            n = -(-L // wl.page_size)
            pages = call.block_table_host[b, :n]
            sel = torch.as_tensor(pages.astype("int64"), device=wl.k_pool.device)
            k = W.to_host_bits(wl.k_pool.index_select(0, sel))
            v = W.to_host_bits(wl.v_pool.index_select(0, sel))
            table = np.arange(n, dtype=np.int64)[None, :]
            t0 = time.perf_counter()
            OA.paged_decode(q[b:b + 1], k, v, table, call.seq_lens_host[b:b + 1], wl.scale)
            spent += time.perf_counter() - t0
            done_bytes += L * 2 * wl.heads * wl.head_dim * 2
            done_tokens += L
            count += 1
    return {
        "value": round(done_bytes / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"oracle (NumPy fp64, 1 BLAS thread) on {count} decode sequences of the "
                  f"{call.batch}-sequence batch taken in order ({done_tokens} tokens, all "
                  f"{wl.num_q_heads} query heads) in {spent:.1f} s",
    }


def cpu_baseline_prefill(wl, call, budget_s=15.0):
    """Oracle on query rows of the first sequence, spread over the whole range."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from exact_tiled_attention_pa_amd import workloads as W
    from oracle import attention as OA

    q = W.to_host_bits(call.q)
    k = W.to_host_bits(wl.k_pool)
    v = W.to_host_bits(wl.v_pool)
    q_len = int(call.q_start_host[1] - call.q_start_host[0])
    L = int(call.seq_lens_host[0])
    n_rows, spent, pairs = 16, 0.0, 0
    with threadpool_limits(limits=1):
        while spent < budget_s and n_rows <= q_len:
            rows = np.linspace(0, q_len - 1, n_rows).astype(np.int64)
            t0 = time.perf_counter()
            OA.paged_prefill(q, k, v, call.block_table_host, call.seq_lens_host,
                             call.q_start_host, call.causal, wl.scale, rows={0: rows})
            spent = time.perf_counter() - t0
            pos = L - q_len + rows
            pairs = int((pos + 1).sum()) if call.causal else L * len(rows)
            n_rows *= 2
    hq = call.q.shape[1]
    flops = 4 * wl.head_dim * hq * pairs
    return {
        "value": round(flops / spent / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"oracle (NumPy fp64, 1 BLAS thread) on {n_rows // 2} query rows of "
                  f"{q_len}, all {hq} heads, in {spent:.1f} s",
    }


# ------------------------------------------------------------------ rocprofv3 summaries

KERNEL_TAGS = {"decode": "decode_partial_kernel", "decode_gqa": "decode_gqa_kernel",
               "prefill": "prefill_kernel<128, true>",
               "prefill_noncausal": "prefill_kernel<128, false>"}


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

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode_64")
    ap.add_argument("--prefill-workload", default="prefill_4096_causal")
    ap.add_argument("--prefill-long-workload", default="prefill_32k",
                    help="second prefill leg: the long causal context")
    ap.add_argument("--no-prefill-long", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the grouped-head / append / copy / window legs")
    ap.add_argument("--only-next", action="store_true",
                    help="run only those legs (on the decode_64 batch) and print them")
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

    if args.only_next:
        wl = W.decode_64(device="cuda")
        print(json.dumps({"next_rows": next_rows_summary(wl, args.steps, args.warmup)}),
              flush=True)
        return

    if args.workload not in W.FULL_WORKLOADS:
        raise SystemExit(f"unknown workload {args.workload}")
    log(f"generating {args.workload}")
    wl = W.FULL_WORKLOADS[args.workload](device="cuda")
    torch.cuda.synchronize()

    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "bf16", "data": "synthetic"}
    call = wl.calls[0]
    if call.kind == "decode":
        nbytes = decode_kv_bytes(wl, call)
        log(f"decode: {call.batch} seqs, {int(call.seq_lens_host.sum())} tokens, "
            f"{nbytes / 1e9:.3f} GB of K/V per step")
        wall, split_ms, comb_ms = timed_decode(wl, call, args.steps, args.warmup)
        ms_step = wall / args.steps * 1e3
        split_avg = sum(split_ms) / len(split_ms)
        achieved = nbytes / (split_avg * 1e-3) / 1e9
        traffic = recorded_traffic(decode_kind(wl), wl.name)
        result.update({
            "value": round(nbytes / (ms_step * 1e-3) / 1e9, 2),
            "unit": "GB/s",
            "ms_per_step": round(ms_step, 4),
            "config": {"workload": wl.name, "batch": call.batch, "heads": wl.num_q_heads,
                       "kv_heads": wl.heads, "head_dim": wl.head_dim,
                       "page_size": wl.page_size,
                       "total_tokens": int(call.seq_lens_host.sum()),
                       "kv_bytes_per_step": nbytes, "description": wl.description},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                         "kernel": decode_kernel_name(wl),
                         "kernel_ms_avg": round(split_avg, 4),
                         "combine_ms_avg": round(sum(comb_ms) / len(comb_ms), 4)},
        })
        if len(wl.calls) > 1:  # mixed batch: the prefill chunks on the same pools
            chunks = wl.calls[1]
            cs = prefill_summary(wl, chunks, args.steps, args.warmup)
            t_roof = nbytes / (HBM_PEAK_GBS * 1e9) + cs["flops_per_launch"] / (
                MFMA_BF16_PEAK_TFLOPS * 1e12)
            t_meas = (split_avg + sum(comb_ms) / len(comb_ms) + cs["kernel_ms_avg"]) * 1e-3
            result["chunks"] = cs
            result["combined_roofline_fraction"] = round(t_roof / t_meas, 4)
    else:
        s = prefill_summary(wl, call, args.steps, args.warmup)
        result.update({
            "value": s["tflops"], "unit": "TFLOP/s", "ms_per_step": s["ms_per_call_wall"],
            "config": {"workload": wl.name, "heads": wl.heads, "head_dim": wl.head_dim,
                       "page_size": wl.page_size, "causal": call.causal,
                       "description": wl.description},
            "roofline": dict(s["roofline"], kernel="prefill_kernel",
                             kernel_ms_avg=s["kernel_ms_avg"]),
        })

    if not args.no_prefill and call.kind == "decode":
        log(f"prefill leg: {args.prefill_workload}")
        pw = W.FULL_WORKLOADS[args.prefill_workload](device="cuda")
        # a longer warm-up: the leg follows the decode loop and must not time clock ramps
        result["prefill"] = prefill_summary(pw, pw.calls[0], args.steps, max(args.warmup, 10))
        del pw
        if not args.no_prefill_long:
            log(f"prefill leg: {args.prefill_long_workload}")
            pw = W.FULL_WORKLOADS[args.prefill_long_workload](device="cuda")
            result["prefill_long"] = prefill_summary(pw, pw.calls[0], min(args.steps, 10),
                                                     max(args.warmup, 3))
            del pw
            torch.cuda.empty_cache()

    # the rows beyond the core path run after the headline legs
    if (not args.no_next and call.kind == "decode" and len(wl.calls) == 1
            and wl.name == "decode_64"):
        log("rows beyond the core path: grouped heads, append, page copy, windows")
        result["next_rows"] = next_rows_summary(wl, args.steps, args.warmup)

    # the oracle runs last, after every GPU leg, so its host time cannot idle the GPU
    # between a warm-up and a timed region
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on a bounded sample")
        if call.kind == "decode":
            result["cpu_baseline"] = cpu_baseline_decode(wl, call)
        else:
            result["cpu_baseline"] = cpu_baseline_prefill(wl, call)
    del wl

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
