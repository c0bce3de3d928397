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


def test_mfma_busy_fraction_from_a_counter_run(tmp_path):
    """Two dispatches of the causal prefill kernel plus an unrelated kernel: the summary
    averages the per-dispatch fractions of the prefill kernel only."""
    import csv

    head = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    # shader cycles per launch = SQ_CYCLES / 32 engines; busy cycles summed over 1024 SIMDs
    for disp, (busy, sq) in {"7": (0.5 * 1024 * 300000, 32 * 300000),
                             "9": (0.25 * 1024 * 200000, 32 * 200000)}.items():
        rows.append([disp, "pa::prefill_kernel<128, true>", "SQ_VALU_MFMA_BUSY_CYCLES", busy])
        rows.append([disp, "pa::prefill_kernel<128, true>", "SQ_CYCLES", sq])
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
                w.writerow([str(3 + i), "pa::prefill_kernel<128, true>", "262144", counter, v])
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
