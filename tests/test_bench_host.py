"""Host-side arithmetic of bench.py: algorithmic work counts against brute force."""
import os

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


def test_mfma_busy_fraction_from_a_counter_run(tmp_path):
    """Two dispatches of the causal prefill kernel plus an unrelated kernel: the summary
    averages the per-dispatch fractions of the prefill kernel only."""
    import csv

    head = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    # shader cycles per launch = SQ_CYCLES / 32 engines; busy cycles summed over 1024 SIMDs
    for disp, (busy, sq) in {"7": (0.5 * 1024 * 300000, 32 * 300000),
                             "9": (0.25 * 1024 * 200000, 32 * 200000)}.items():
        rows.append([disp, "pa::prefill_kernel<128, true, true>", "SQ_VALU_MFMA_BUSY_CYCLES", busy])
        rows.append([disp, "pa::prefill_kernel<128, true, true>", "SQ_CYCLES", sq])
    rows.append(["8", "pa::decode_partial_kernel<128>", "SQ_VALU_MFMA_BUSY_CYCLES", 1.0])
    rows.append(["8", "pa::decode_partial_kernel<128>", "SQ_CYCLES", 1.0])
    with open(tmp_path / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(head)
        w.writerows(rows)
    with open(tmp_path / "run_agent_info.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Agent_Type", "Simd_Count", "Num_Shader_Banks"])
        w.writerow(["CPU", "0", "0"])
        w.writerow(["GPU", "1024", "32"])
    out = tmp_path / "summary.txt"
    bench.summarize_mfma(str(tmp_path), "prefill", "prefill_4096_causal", str(out), "cmd")
    vals = dict(l.split("=", 1) for l in out.read_text().splitlines() if "=" in l
                and not l.startswith("#"))
    assert vals["dispatches"] == "2"
    assert abs(float(vals["mfma_busy_fraction"]) - 0.375) < 1e-9
    assert vals["source_sha256"] == bench.source_digest("prefill")


def test_decode_kind_follows_the_library_dispatch():
    class Wl:
        def __init__(self, hq, hkv):
            self.num_q_heads, self.heads = hq, hkv
    assert bench.decode_kind(Wl(32, 32)) == "decode"
    assert bench.decode_kind(Wl(32, 16)) == "decode"    # g = 2: one-head-per-row kernel
    assert bench.decode_kind(Wl(24, 8)) == "decode"     # g = 3
    assert bench.decode_kind(Wl(32, 8)) == "decode_gqa"


def test_gqa_threshold_matches_the_library():
    import re
    text = open(bench.os.path.join(bench.CSRC, "kernels.h")).read()
    assert int(re.search(r"kGqaMinGroup\s*=\s*(\d+)", text).group(1)) == bench.GQA_MIN_GROUP
    # the host layer's split rule counts the grouped kernel's head blocks with the
    # kernel's own block size
    api = open(bench.os.path.join(bench.CSRC, "api.cpp")).read()
    gqa = open(bench.os.path.join(bench.CSRC, "decode_gqa.hip")).read()
    assert int(re.search(r"kGqaHeadBlock\s*=\s*(\d+)", api).group(1)) == \
        int(re.search(r"kHeadBlock\s*=\s*(\d+)", gqa).group(1))


def test_prefill_kernel_choice_matches_the_library():
    """bench.py names the prefill kernel a call runs by the library's own rule: its
    constants are the header's, and the worked example takes the split-key kernel
    while the N=4096 workload takes the tiled one."""
    import re
    text = open(bench.os.path.join(bench.CSRC, "prefill_split.h")).read()
    assert int(re.search(r"kPrefillSplitBlockM\s*=\s*(\d+)", text).group(1)) == \
        bench.PREFILL_SPLIT_BLOCK_M
    assert int(re.search(r"kPrefillSplitMaxWorkgroups\s*=\s*(\d+)", text).group(1)) == \
        bench.PREFILL_SPLIT_MAX_WORKGROUPS
    from exact_tiled_attention_pa_amd import workloads as W
    small = W.prefill_600(tensors=False)
    large = W.prefill_4096(causal=True, tensors=False)
    assert bench.prefill_kernel_name(small, small.calls[0]) == "prefill_split_kernel<64, true>"
    assert bench.prefill_kernel_name(large, large.calls[0]) == "prefill_kernel<128, true, true>"


def test_kernel_source_lists_cover_local_includes():
    """The source hash that guards each counter summary covers every local header the
    kernel's file includes."""
    import re
    for kind, files in bench.KERNEL_SOURCES.items():
        text = open(bench.os.path.join(bench.CSRC, files[0])).read()
        for inc in re.findall(r'#include "([^"]+)"', text):
            assert inc in files, (kind, inc)


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    """FETCH_SIZE and WRITE_SIZE runs, each with a 1 GiB calibration copy: the kernel's
    readings are scaled by 1 GiB / the copy's reading; bench reads the figure back only
    while the recorded source hash matches."""
    import csv

    def run_dir(name, counter, copy_kib, kernel_kib):
        d = tmp_path / name
        d.mkdir()
        with open(d / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                        "Counter_Value"])
            w.writerow(["1", "__amd_rocclr_copyBuffer", "1048576", counter, copy_kib])
            w.writerow(["2", "__amd_rocclr_copyBuffer", "64", counter, 1.0])  # small copy
            for i, v in enumerate(kernel_kib):
                w.writerow([str(3 + i), "pa::prefill_kernel<128, true, true>", "262144", counter, v])
            w.writerow(["9", "pa::decode_partial_kernel<128>", "262144", counter, 1e9])
        return str(d)

    gib_kib = float(1 << 20)
    fetch = run_dir("fetch", "FETCH_SIZE", gib_kib / 2, [1000.0, 3000.0])  # factor 2
    write = run_dir("write", "WRITE_SIZE", gib_kib, [500.0, 500.0])        # factor 1
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    out = tmp_path / f"{bench.KERNEL_FILES['prefill']}.wl.traffic.txt"
    bench.summarize_traffic(fetch, write, "prefill", "wl", str(out), "cmd")
    expect = (2000.0 * 2 + 500.0 * 1) * 1024
    assert bench.recorded_traffic("prefill", "wl") == int(expect)
    # a summary taken from other kernel sources is not reported
    text = out.read_text().replace(bench.source_digest("prefill"), "0" * 64)
    out.write_text(text)
    assert bench.recorded_traffic("prefill", "wl") is None


def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=bench.os.path.dirname(
        bench.os.path.abspath(bench.__file__)), capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_pool_on_small_workloads(tmp_path, monkeypatch):
    """The bench's oracle pool on two small workloads: per-leg rates, the process count,
    the CPU model, and parity figures against stand-in outputs (the oracle's own values
    rounded to bf16, well inside the tolerance)."""
    import torch
    from exact_tiled_attention_pa_amd import workloads as W
    from tests.oracle_pins import to_bf16_bits

    monkeypatch.setattr(bench, "cpu_workers", lambda: 2)
    dec = W.build("decode_64", 5, heads=2, head_dim=64, page_size=16, lens=[40, 300, 17],
                  kind="decode", pool_slack=1.3, device="cpu", q_heads=4)
    pre = W.build("prefill_32k", 6, heads=2, head_dim=64, page_size=16, lens=[200],
                  q_lens=[200], causal=True, device="cpu")
    # chunks on cached context, as in the mixed batch: 3 sequences, rows not starting at 0
    chunks = W.build("mixed_128x4", 7, heads=2, head_dim=64, page_size=16,
                     lens=[150, 90, 260], q_lens=[40, 90, 33], causal=True, device="cpu")
    legs = {}
    for name, wl in (("decode_64", dec), ("prefill_32k", pre), ("mixed_128x4_chunks", chunks)):
        call = wl.calls[0]
        q = W.to_host_bits(call.q)
        k, v = W.to_host_bits(wl.k_pool), W.to_host_bits(wl.v_pool)
        if call.kind == "decode":
            ref, _ = OA.paged_decode(q, k, v, call.block_table_host, call.seq_lens_host, wl.scale)
        else:
            ref, _ = OA.paged_prefill(q, k, v, call.block_table_host, call.seq_lens_host,
                                      call.q_start_host, True, wl.scale)
        out = torch.from_numpy(to_bf16_bits(ref).view(np.int16)).view(torch.bfloat16)
        legs[name] = (wl, call, out, bench.baseline_samples(name, wl, call))
    res = bench.cpu_baseline(legs, str(tmp_path))
    assert res["cores"] == 2 and res["kind"] == "oracle" and res["cpu_model"]
    assert res["unit"] == "GB/s" and res["value"] > 0
    d, p = res["legs"]["decode_64"], res["legs"]["prefill_32k"]
    assert d["unit"] == "GB/s" and p["unit"] == "TFLOP/s" and p["value"] > 0
    for leg in (d, p):
        assert leg["parity"]["within_tolerance"], leg
        assert leg["parity"]["max_abs"] <= 1e-2
    # the prefill sample: every 8th row from row 4, all heads
    assert p["parity"]["elements"] == len(range(4, 200, 8)) * 2 * 64
    # the chunk sample: every 8th row of each sequence from its row 4; its visible pairs
    # counted by brute force over the sampled rows' absolute positions
    c = res["legs"]["mixed_128x4_chunks"]
    assert c["parity"]["within_tolerance"], c
    lens, q_lens = [150, 90, 260], [40, 90, 33]
    rows = [range(4, n, 8) for n in q_lens]
    assert c["parity"]["elements"] == sum(len(r) for r in rows) * 2 * 64
    pairs = sum(1 for L, n, rr in zip(lens, q_lens, rows) for i in rr for t in range(L)
                if t <= L - n + i)
    assert f"({pairs} visible pairs per head)" in c["sample"]
    assert "over 3 sequences" in c["sample"]
    assert os.listdir(tmp_path) == []


def test_rate_takes_the_average_from_the_whole_timed_region():
    """`achieved` and `frac` come from the average over one event pair around all timed
    launches; median, minimum and the per-launch-pair average come from the second run."""
    import bench

    t = bench.Timing(2.0, [2.5, 2.1, 2.2, 3.0])
    r = bench._rate(8e12, t, 2500.0, "TFLOP/s", bound="mfma")
    assert r["kernel_ms_avg"] == 2.0 and r["achieved"] == 4000.0
    assert r["frac"] == round(4000.0 / 2500.0, 4)
    assert r["kernel_ms_median"] == 2.35 and r["kernel_ms_min"] == 2.1
    assert r["kernel_ms_avg_paired"] == 2.45 and r["bound"] == "mfma"


def test_naive_traffic_count_matches_the_pages_worked_figures():
    """The unfused kernel's byte count the bench sets beside each prefill's measured
    traffic reproduces the figures the page states for N = 4096, d = 128 (one head):
    the S/P term about 134 MB, the Q/K/V/O term about 4 MB, S and P about 32 MiB each,
    about 97 % of the traffic in S and P, and about 62 operations per byte against
    4N^2 d + 3N^2 operations."""
    import json
    g = json.load(open(bench.os.path.join(bench.ROOT, "tests", "golden",
                                          "naive_attention_traffic.json")))
    n, d = g["N"], g["d"]
    total = bench.naive_attention_bytes(n, d)
    sp, nd = bench.naive_attention_bytes(n, 0), total - bench.naive_attention_bytes(n, 0)
    assert round(sp / 1e6) == g["s_p_term_mb_about"]
    assert round(nd / 1e6) == g["nd_term_mb_about"]
    assert round(2 * n * n / 2 ** 20) == g["s_or_p_mib_about"]  # one 16-bit n x n matrix
    assert round(sp / total, 2) == g["s_p_share_about"]
    ops = 4 * n * n * d + 3 * n * n
    assert round(ops / total) == g["ops_per_byte_about"]
    assert bench.naive_attention_bytes(n, d, heads=32) == 32 * total
