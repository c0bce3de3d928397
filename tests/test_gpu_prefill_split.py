"""The split-key prefill kernel (32 query rows per workgroup, the key tiles dealt over
its waves, eight at d = 64 and five at d = 128, the waves' softmax states merged at the end) against the fp64 oracle,
the automatic choice between it and the 128-row tiled kernel, and the binding's
prepared calls (PreparedPrefill, PreparedDecode) against the direct ones.

The shared small-shape parity tests already run under both kernels (the
`prefill_path` fixture); these cases add what only the split kernel has: a key loop
divided over waves (waves with no tile at all, long contexts under few rows, windows
that leave some waves only masked keys) and the merge."""
import pytest
import torch

from exact_tiled_attention_pa_amd import binding as B
from exact_tiled_attention_pa_amd import workloads as W
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    G.gpu_or_skip()


def _prefill(wl, call, window=0):
    out = torch.full_like(call.q, float("nan"))
    B.pa_prefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, call.causal,
                 wl.scale, out, call.q_start, call.max_q_len, window=window)
    torch.cuda.synchronize()
    return out


SPLIT_CASES = [
    # (head_dim, page_size, causal, Hq, Hkv, lens, q_lens, window)
    (128, 16, True, 4, 4, [20000, 3000], [5, 40], 0),      # long contexts, few rows
    (64, 256, True, 2, 2, [9000], [33], 0),                # one row past a 32-row tile
    (128, 32, False, 8, 2, [5000, 64, 65], [7, 64, 65], 0),  # grouped heads, non-causal
    (64, 16, True, 4, 1, [1, 64, 65, 128, 129], [1, 64, 1, 2, 129], 0),  # waves with no tile
    (128, 64, True, 4, 4, [6000, 2000], [40, 300], 100),   # window: most waves masked only
    (128, 16, True, 2, 2, [4097], [64], 1),                # window 1: own V row
    (64, 128, True, 3, 3, [7777], [31], 3000),
]


@pytest.mark.parametrize("d,ps,causal,hq,hkv,lens,q_lens,window", SPLIT_CASES)
def test_split_kernel_element_wise(d, ps, causal, hq, hkv, lens, q_lens, window, monkeypatch):
    monkeypatch.setenv("PA_PREFILL_PATH", "split")
    G.banner(f"split prefill d={d} ps={ps} causal={causal} Hq={hq} Hkv={hkv} lens={lens} "
             f"q_lens={q_lens} window={window}")
    wl = W.build("split", 900 + d + ps + window, heads=hkv, head_dim=d, page_size=ps,
                 lens=lens, q_lens=q_lens, causal=causal, pool_slack=1.2, device="cuda",
                 poison=True, q_heads=hq)
    call = wl.calls[0]
    out = _prefill(wl, call, window)
    G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call, window=window),
              f"split d={d} ps={ps} window={window}")


def test_split_kernel_window_one_returns_own_value_row(monkeypatch):
    """w = 1 through the split kernel: each row's one visible key lies in one wave's tile;
    the other three waves hold m = -inf and must contribute exactly nothing."""
    monkeypatch.setenv("PA_PREFILL_PATH", "split")
    G.banner("split prefill window=1 exactness")
    wl = W.build("sw1", 78, heads=2, head_dim=128, page_size=16, lens=[2000], q_lens=[100],
                 causal=True, device="cuda", poison=True)
    call = wl.calls[0]
    out = _prefill(wl, call, window=1)
    bt = call.block_table_host[0]
    for i in range(100):
        t = 2000 - 100 + i
        assert torch.equal(out[i], wl.v_pool[int(bt[t // 16]), t % 16]), i


@pytest.mark.parametrize("which", ["prefill_600", "tiny_heads", "mid", "large"])
def test_automatic_choice_follows_the_launch_size(which, monkeypatch):
    """With PA_PREFILL_PATH unset, a launch whose 32-row grid is at most 512 workgroups
    (the worked example: 19; 4 heads x 600 rows: 76; 16 heads x 1024 rows: 512) runs the
    split-key kernel and a larger one (32 heads x 1024 rows: 1024) the tiled kernel.  The two
    kernels round differently, so the automatic output equals exactly one forced path's
    output bit for bit (and matches the oracle)."""
    G.banner(f"automatic prefill kernel choice: {which}")
    if which == "prefill_600":
        wl = W.prefill_600(device="cuda", poison=True)
        want = "split"
    elif which == "tiny_heads":
        wl = W.build("auto4", 55, heads=4, head_dim=128, page_size=256, lens=[600],
                     q_lens=[600], causal=True, device="cuda", poison=True)
        want = "split"
    elif which == "mid":
        wl = W.build("auto16", 57, heads=16, head_dim=128, page_size=256, lens=[1024],
                     q_lens=[1024], causal=True, device="cuda", poison=True)
        want = "split"
    else:
        wl = W.build("auto32", 56, heads=32, head_dim=128, page_size=256, lens=[1024],
                     q_lens=[1024], causal=True, device="cuda", poison=True)
        want = "tiles"
    call = wl.calls[0]
    outs = {}
    for path in ("", "tiles", "split"):
        monkeypatch.setenv("PA_PREFILL_PATH", path)
        outs[path or "auto"] = _prefill(wl, call)
    other = "tiles" if want == "split" else "split"
    assert torch.equal(outs["auto"], outs[want])
    assert not torch.equal(outs[want], outs[other]), "the two kernels agreed bit for bit"
    if which not in ("large", "mid"):
        G.compare(G.bf16_out_to_f64(outs["auto"]), G.oracle_for(wl, call), which)
    else:
        rows = {0: G.spread_rows(1024, 256, seed=3)}
        ref = G.oracle_for(wl, call, rows=rows)
        G.compare(G.bf16_out_to_f64(outs["auto"]), ref, which)


@pytest.mark.parametrize("window", [0, 50])
def test_prepared_prefill_matches_direct_calls(window):
    """A PreparedPrefill launched twice, with new query values written into its q between
    the launches, returns exactly what pa_prefill returns for each."""
    G.banner(f"prepared prefill window={window}")
    wl = W.build("prep", 91, heads=2, head_dim=128, page_size=16, lens=[700, 90],
                 q_lens=[300, 90], causal=True, pool_slack=1.2, device="cuda", poison=True,
                 q_heads=4)
    call = wl.calls[0]
    out = torch.empty_like(call.q)
    prep = B.PreparedPrefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens,
                             True, wl.scale, out, call.q_start, call.max_q_len, window=window)
    ref = torch.empty_like(call.q)
    for rnd in range(2):
        if rnd:
            call.q.mul_(-0.5)  # new contents, same buffer
        got = prep.launch().clone()
        B.pa_prefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, True,
                     wl.scale, ref, call.q_start, call.max_q_len, window=window)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), rnd
    G.compare(G.bf16_out_to_f64(ref), G.oracle_for(wl, call, window=window), "prepared")


@pytest.mark.parametrize("window,hq", [(0, 4), (0, 16), (300, 4)])
def test_prepared_decode_matches_direct_calls(window, hq):
    """A PreparedDecode launched twice (new query values between the launches) returns
    exactly what pa_decode returns, for both decode kernels and with a window."""
    G.banner(f"prepared decode window={window} Hq={hq}")
    wl = W.build("prepd", 92, heads=4, head_dim=128, page_size=16, lens=[1, 700, 3000],
                 kind="decode", pool_slack=1.2, device="cuda", poison=True, q_heads=hq)
    call = wl.calls[0]
    out = torch.empty_like(call.q)
    ws = B.decode_workspace(call.q, wl.k_pool, call.block_table)
    prep = B.PreparedDecode(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens,
                            wl.scale, out, ws, window=window)
    ref = torch.empty_like(call.q)
    ws2 = torch.empty_like(ws)
    for rnd in range(2):
        if rnd:
            call.q.mul_(-0.5)
        got = prep.launch().clone()
        B.pa_decode(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, wl.scale,
                    ref, ws2, window=window)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), rnd
    G.compare(G.bf16_out_to_f64(ref), G.oracle_for(wl, call, window=window), "prepared decode")


@pytest.mark.parametrize("causal", [True, False])
def test_split_and_tiled_kernels_agree_on_every_element_at_4096(causal, monkeypatch):
    """The two prefill kernels over the N=4096, 32-head workload (the split-key one forced:
    4096 workgroups), compared on every output element, plus sampled rows of each against
    the oracle.  Two independent decompositions of the same exact result."""
    G.banner(f"split vs tiled prefill, N=4096 causal={causal}")
    wl = W.prefill_4096(causal=causal, device="cuda")
    call = wl.calls[0]
    outs = {}
    for path in ("tiles", "split"):
        monkeypatch.setenv("PA_PREFILL_PATH", path)
        outs[path] = _prefill(wl, call)
    G.compare(G.bf16_out_to_f64(outs["split"]), G.bf16_out_to_f64(outs["tiles"]),
              "split vs tiled", max_tol=8e-3, mean_tol=5e-4)
    rows = {0: G.spread_rows(4096, 128, seed=11)}
    ref = G.oracle_for(wl, call, rows=rows)
    for path, out in outs.items():
        G.compare(G.bf16_out_to_f64(out), ref, f"N=4096 {path}")
