"""GPU parity: the HIP library (called through the C ABI) against the fp64 oracle on
identical seeded inputs.  Bar: max |O_gpu - O_ref| <= 1e-2 and mean <= 1e-3; the
block-table address math bit-exact (address probe, permutation invariance)."""
import numpy as np
import pytest
import torch

from exact_tiled_attention_pa_amd import binding as B
from exact_tiled_attention_pa_amd import workloads as W
from tests import gpu_helpers as G
from tests.gpu_helpers import prefill_path  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    G.gpu_or_skip()


# ----------------------------------------------------------------- small, element-wise

def test_prefill_600_worked_example_full(prefill_path):
    """Paged causal prefill on the worked example's layout (600 tokens, pages of 256,
    table [5, 1, 9]); unread slots hold NaN.  Every output element is compared."""
    G.banner("prefill_600 full, poisoned pool")
    wl = W.prefill_600(device="cuda", poison=True)
    call = wl.calls[0]
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call), "prefill_600")


PREFILL_CASES = [
    # (head_dim, page_size, causal, Hq, Hkv, lens, q_lens)
    (128, 16, True, 4, 4, [1, 200, 777], [1, 200, 300]),
    (128, 16, False, 4, 4, [1, 200, 777], [1, 200, 300]),
    (128, 256, True, 2, 2, [64, 1000], [64, 129]),
    (128, 32, True, 8, 2, [300, 513], [300, 17]),
    (128, 64, False, 4, 1, [129, 65], [129, 65]),
    (64, 16, True, 3, 3, [259, 31], [259, 31]),
    (64, 128, False, 2, 2, [1000, 1], [999, 1]),
    (64, 256, True, 4, 2, [700], [700]),
]


@pytest.mark.parametrize("d,ps,causal,hq,hkv,lens,q_lens", PREFILL_CASES)
def test_prefill_small_element_wise(d, ps, causal, hq, hkv, lens, q_lens, prefill_path):
    G.banner(f"prefill small d={d} ps={ps} causal={causal} Hq={hq} Hkv={hkv} lens={lens} "
             f"q_lens={q_lens}")
    wl = W.build("small", 100 + d + ps, heads=hkv, head_dim=d, page_size=ps, lens=lens,
                 q_lens=q_lens, causal=causal, kind="prefill", pool_slack=1.3, device="cuda",
                 poison=True)
    call = wl.calls[0]
    if hq != hkv:  # grouped heads: more query heads than K/V heads
        gen = torch.Generator(device="cuda").manual_seed(7)
        call.q = (torch.randn(call.q.shape[0], hq, d, generator=gen, device="cuda")
                  .to(torch.bfloat16))
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    ref = G.oracle_for(wl, call)
    G.compare(G.bf16_out_to_f64(out), ref, f"prefill d={d} ps={ps} causal={causal}")


DECODE_CASES = [
    # (head_dim, page_size, Hq, Hkv, lens)
    (128, 16, 4, 4, [1, 15, 16, 17, 511, 512, 513, 3000]),
    (128, 256, 2, 2, [1, 255, 256, 257, 1500]),
    (64, 16, 3, 3, [7, 1024, 2049]),
    # grouped K/V heads (one page read serves the whole group)
    (128, 32, 8, 2, [100, 700]),
    (64, 64, 4, 1, [65, 1]),
    (128, 16, 16, 2, [1, 15, 16, 17, 31, 32, 33, 255, 256, 257, 3000]),
    (128, 16, 64, 8, [1, 100, 2049]),
    (128, 256, 4, 2, [1, 255, 256, 257, 1500]),
    (64, 16, 12, 3, [7, 1024, 2049]),
    (128, 16, 32, 1, [5, 600]),
    (128, 32, 40, 1, [100, 700]),         # 40 heads per K/V head: blocks of 32 + 8
    (64, 64, 71, 1, [65, 1, 2000]),       # 71 heads: blocks of 32 + 32 + 7
    (128, 256, 16, 2, [1, 255, 256, 257, 1023, 1024, 1025, 5000]),
    (64, 128, 8, 1, [127, 128, 129, 2049]),
    # one-head-per-row kernel: a last head group with absent heads, splits shorter than
    # its load ring, and 3 query heads per K/V head
    (128, 16, 5, 5, [1, 16, 63, 64, 65, 300]),
    (128, 16, 6, 2, [17, 1000]),
    (64, 32, 9, 3, [33, 2049]),
]


@pytest.mark.parametrize("d,ps,hq,hkv,lens", DECODE_CASES)
def test_decode_small_element_wise(d, ps, hq, hkv, lens):
    G.banner(f"decode small d={d} ps={ps} Hq={hq} Hkv={hkv} lens={lens}")
    wl = W.build("small", 200 + d + ps + hq, heads=hkv, head_dim=d, page_size=ps, lens=lens,
                 kind="decode", pool_slack=1.2, device="cuda", poison=True, q_heads=hq)
    call = wl.calls[0]
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call), f"decode d={d} ps={ps}")


@pytest.mark.parametrize("hq", [4, 16])
def test_decode_two_passes_equal_one_call(hq):
    G.banner(f"decode partial+combine vs pa_decode, Hq={hq}")
    wl = W.build("small", 5, heads=4, head_dim=128, page_size=16, lens=[40, 1300, 900],
                 kind="decode", device="cuda", poison=True, q_heads=hq)
    call = wl.calls[0]
    ws = B.decode_workspace(call.q, wl.k_pool, call.block_table)
    one = G.run_call(wl, call, workspace=ws)
    two = torch.empty_like(one)
    B.pa_decode_partial(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens,
                        wl.scale, ws)
    B.pa_decode_combine(call.seq_lens, two, ws, B.layout_of(wl.k_pool, call.block_table))
    torch.cuda.synchronize()
    assert torch.equal(one, two)


# ----------------------------------------------------------------- full-size, sampled

def test_decode_64_gqa8_sampled():
    G.banner("decode_64_gqa8 full size (64 query heads over 8 K/V heads), 6 sequences")
    wl = W.decode_64_gqa8(device="cuda", poison=True)
    call = wl.calls[0]
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    lens = call.seq_lens_host
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 63, 21, 40})
    ref = G.oracle_for(wl, call, seqs=seqs)
    G.compare(G.bf16_out_to_f64(out), ref, "decode_64_gqa8")


def test_decode_64_sampled():
    G.banner("decode_64 full size, 8 sequences sampled (all heads)")
    wl = W.decode_64(device="cuda", poison=True)
    call = wl.calls[0]
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    lens = call.seq_lens_host
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 63, 17, 31, 42, 50})
    ref = G.oracle_for(wl, call, seqs=seqs)
    G.compare(G.bf16_out_to_f64(out), ref, "decode_64")


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_4096_sampled(causal):
    G.banner(f"prefill_4096 causal={causal} full size, rows sampled (all heads)")
    wl = W.prefill_4096(device="cuda", poison=True, causal=causal)
    call = wl.calls[0]
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    rows = {0: G.spread_rows(4096, 48, seed=1)}
    G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call, rows=rows),
              f"prefill_4096 causal={causal}")


def test_prefill_4096_grouped_heads_sampled():
    """64 query heads over 8 K/V heads at N=4096, causal, shuffled pages of 256: the
    grouped-head prefill at full size, rows sampled, all query heads checked."""
    G.banner("prefill N=4096, 64 query heads over 8 K/V heads, rows sampled")
    wl = W.build("pf_gqa", 5, heads=8, head_dim=128, page_size=256, lens=[4096],
                 q_lens=[4096], causal=True, shuffle=True, device="cuda", poison=True,
                 q_heads=64)
    call = wl.calls[0]
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    rows = {0: G.spread_rows(4096, 24, seed=6)}
    ref = G.oracle_for(wl, call, rows=rows)
    G.compare(G.bf16_out_to_f64(out), ref, "prefill_4096 grouped 64/8")


def test_prefill_32k_sampled():
    G.banner("prefill_32k full size, rows sampled (all heads)")
    wl = W.prefill_32k(device="cuda", poison=True)
    call = wl.calls[0]
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    rows = {0: G.spread_rows(32768, 40, seed=2, tile=4096)}
    G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call, rows=rows), "prefill_32k")


def test_mixed_128x4_sampled():
    G.banner("mixed_128x4 full size: decode then chunked prefill on one stream, sampled")
    wl = W.mixed_128x4(device="cuda", poison=True)
    dec, pre = wl.calls
    out_d = G.run_call(wl, dec)
    out_p = G.run_call(wl, pre)
    torch.cuda.synchronize()
    lens = dec.seq_lens_host
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 127, 64})
    G.compare(G.bf16_out_to_f64(out_d), G.oracle_for(wl, dec, seqs=seqs), "mixed decode")
    rows = {b: G.spread_rows(2048, 12, seed=10 + b) for b in range(4)}
    G.compare(G.bf16_out_to_f64(out_p), G.oracle_for(wl, pre, rows=rows), "mixed chunks")


# ----------------------------------------------------------------- address math, bit-exact

def _encode_slots(wl):
    """V[p, o, h, :] := (p % 128, (p // 128) % 128, p // 16384, o, h, 0, ...): small
    integers, exact in bf16, that name the slot they sit in."""
    P, ps, H, d = wl.v_pool.shape
    dev = wl.v_pool.device
    p = torch.arange(P, device=dev, dtype=torch.float32)[:, None, None]
    o = torch.arange(ps, device=dev, dtype=torch.float32)[None, :, None]
    h = torch.arange(H, device=dev, dtype=torch.float32)[None, None, :]
    enc = torch.zeros(P, ps, H, d, device=dev, dtype=torch.float32)
    enc[..., 0] = (p % 128).expand(P, ps, H)
    enc[..., 1] = ((p // 128) % 128).expand(P, ps, H)
    enc[..., 2] = (p // 16384).expand(P, ps, H)
    enc[..., 3] = o.expand(P, ps, H)
    enc[..., 4] = h.expand(P, ps, H)
    wl.v_pool.copy_(enc.to(torch.bfloat16))


def _decode_slot(row: torch.Tensor):
    """Inverse of _encode_slots for output rows [..., d] -> (page, offset, head)."""
    r = row.float()
    page = r[..., 0] + 128 * r[..., 1] + 16384 * r[..., 2]
    return page.long(), r[..., 3].long(), r[..., 4].long()


def test_address_probe_decode():
    """Each sequence's query aligns with one spike key (margin ~260 in log2 units, so
    every other weight is exactly 0 in fp32): the output must be, bit for bit, the
    V row of the slot the block table names for that token."""
    G.banner("address probe, decode_64 layout")
    wl = W.decode_64(device="cuda")
    call = wl.calls[0]
    H, d, ps = wl.heads, wl.head_dim, wl.page_size
    wl.k_pool.zero_()
    _encode_slots(wl)
    rng = np.random.default_rng(3)
    lens = call.seq_lens_host
    q = torch.zeros(call.batch, H, d, device="cuda", dtype=torch.bfloat16)
    want = []
    for b in range(call.batch):
        t = int(rng.integers(0, lens[b])) if b % 3 else int(lens[b] - 1 - b % 2)
        phys = int(call.block_table_host[b, t // ps])
        wl.k_pool[phys, t % ps, :, 5] = 64.0
        q[b, :, 5] = 32.0
        want.append((phys, t % ps))
        # the spike channel of every other sequence is different (channel 5 vs none)
    call.q = q
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    page, off, head = _decode_slot(out)
    for b, (phys, o) in enumerate(want):
        assert torch.all(page[b] == phys) and torch.all(off[b] == o), (b, phys, o)
        assert torch.equal(head[b].cpu(), torch.arange(H))


def test_address_probe_prefill_paged():
    """Causal paged prefill on the 32k layout (shuffled pages of 256): 64 target tokens
    spread over every page, each on its own key channel; every sampled query row aligns
    with one visible target and must return that slot's V row exactly."""
    G.banner("address probe, prefill_32k layout")
    wl = W.prefill_32k(device="cuda")
    call = wl.calls[0]
    H, d, ps = wl.heads, wl.head_dim, wl.page_size
    wl.k_pool.zero_()
    _encode_slots(wl)
    rng = np.random.default_rng(4)
    L = 32768
    targets = np.sort(rng.choice(L, size=64, replace=False))
    targets[0] = 0
    q = torch.zeros(L, H, d, device="cuda", dtype=torch.bfloat16)
    slot_of = {}
    for c, t in enumerate(targets):
        phys = int(call.block_table_host[0, t // ps])
        wl.k_pool[phys, t % ps, :, c] = 64.0
        slot_of[c] = (phys, int(t % ps))
    rows = rng.choice(L, size=4096, replace=False)
    chan = np.empty(len(rows), dtype=np.int64)
    for i, r in enumerate(rows):
        visible = np.nonzero(targets <= r)[0]
        chan[i] = visible[rng.integers(0, len(visible))]
        q[int(r), :, int(chan[i])] = 32.0
    call.q = q
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    page, off, _ = _decode_slot(out[torch.as_tensor(rows, device="cuda")])
    want_p = torch.tensor([slot_of[int(c)][0] for c in chan], device="cuda")
    want_o = torch.tensor([slot_of[int(c)][1] for c in chan], device="cuda")
    assert torch.all(page == want_p[:, None]) and torch.all(off == want_o[:, None])


def _permute_pages(wl, calls, seed):
    P = wl.k_pool.shape[0]
    g = torch.Generator(device="cpu").manual_seed(seed)
    sigma = torch.randperm(P, generator=g)
    k2 = torch.empty_like(wl.k_pool)
    v2 = torch.empty_like(wl.v_pool)
    k2[sigma.cuda()] = wl.k_pool
    v2[sigma.cuda()] = wl.v_pool
    tables = []
    for c in calls:
        t = c.block_table.long()
        tables.append(torch.where(t >= 0, sigma.cuda()[t.clamp(min=0)], t).to(torch.int32))
    return k2, v2, tables


@pytest.mark.parametrize("which", ["decode_64", "prefill_32k"])
def test_permuting_physical_pages_is_bitwise_invariant(which):
    """Relabelling physical pages (moving them in the pool and remapping the table)
    must not change a single output bit: the kernels visit keys in logical order."""
    G.banner(f"page permutation invariance, {which}")
    wl = W.FULL_WORKLOADS[which](device="cuda", poison=True)
    call = wl.calls[0]
    base = G.run_call(wl, call)
    k2, v2, (t2,) = _permute_pages(wl, [call], seed=99)
    out = torch.empty_like(base)
    if call.kind == "prefill":
        B.pa_prefill(call.q, k2, v2, t2, call.seq_lens, call.causal, wl.scale, out,
                     call.q_start, call.max_q_len)
    else:
        ws = B.decode_workspace(call.q, k2, t2)
        B.pa_decode(call.q, k2, v2, t2, call.seq_lens, wl.scale, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(base, out)


def test_poisoned_and_clean_pools_agree_bitwise(prefill_path):
    """NaN in tail slots and unused pages must not change the output."""
    G.banner("poison vs clean, small prefill + decode")
    for kind in ("prefill", "decode"):
        a = W.build("p", 31, heads=2, head_dim=128, page_size=16, lens=[37, 300],
                    q_lens=[37, 100] if kind == "prefill" else None, kind=kind,
                    pool_slack=1.5, device="cuda", poison=False)
        b = W.build("p", 31, heads=2, head_dim=128, page_size=16, lens=[37, 300],
                    q_lens=[37, 100] if kind == "prefill" else None, kind=kind,
                    pool_slack=1.5, device="cuda", poison=True)
        oa = G.run_call(a, a.calls[0])
        ob = G.run_call(b, b.calls[0])
        torch.cuda.synchronize()
        assert torch.isfinite(ob.float()).all()
        assert torch.equal(oa, ob), kind


def test_constant_values_return_the_constant(prefill_path):
    G.banner("constant V")
    for kind, hq in (("prefill", 2), ("decode", 2), ("decode", 16)):
        wl = W.build("c", 41, heads=2, head_dim=128, page_size=16, lens=[1, 500, 64],
                     q_lens=[1, 500, 10] if kind == "prefill" else None, kind=kind,
                     device="cuda", poison=True, q_heads=hq)
        used = torch.isfinite(wl.v_pool.float())
        wl.v_pool[used] = 1.75
        out = G.run_call(wl, wl.calls[0]).float()
        torch.cuda.synchronize()
        # the row sum adds exactly the weights applied to V (prefill: the bf16-rounded P;
        # decode: the fp32 P), so O = c up to fp32 rounding, which bf16 rounds back to c
        assert torch.all(out == 1.75), (kind, (out - 1.75).abs().max().item())


def test_empty_batch_and_zero_rows_are_no_ops():
    G.banner("empty batch")
    wl = W.build("e", 1, heads=1, head_dim=64, page_size=16, lens=[5], q_lens=[5],
                 device="cuda")
    call = wl.calls[0]
    out = torch.full_like(call.q, 3.0)
    lay = B.layout_of(wl.k_pool, call.block_table)
    lib = B.load_library()
    import ctypes
    st = lib.pa_prefill(call.q.data_ptr(), wl.k_pool.data_ptr(), wl.v_pool.data_ptr(),
                        call.block_table.data_ptr(), call.seq_lens.data_ptr(), 1, wl.scale,
                        out.data_ptr(), call.q_start.data_ptr(), 0, 1, 5, ctypes.byref(lay),
                        None)
    torch.cuda.synchronize()
    assert st == B.PA_OK and torch.all(out == 3.0)


@pytest.mark.parametrize("hq,window", [(2, 0), (2, 100), (16, 0), (16, 100)])
def test_decode_empty_sequences_get_zeros(hq, window):
    """A sequence with L_b = 0 reads nothing (its table row holds only -1) and its output
    rows are exactly zero; the other sequences of the batch match the oracle.  hq=16 over
    2 K/V heads runs the grouped kernel, hq=2 the one-head-per-row kernel."""
    G.banner(f"decode with empty sequences Hq={hq} window={window}")
    wl = W.build("z", 3, heads=2, head_dim=128, page_size=16, lens=[0, 37, 0, 1300, 0],
                 kind="decode", pool_slack=1.2, device="cuda", poison=True, q_heads=hq)
    call = wl.calls[0]
    out = torch.full_like(call.q, 7.0)
    ws = B.decode_workspace(call.q, wl.k_pool, call.block_table)
    B.pa_decode(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, wl.scale, out,
                ws, window=window)
    torch.cuda.synchronize()
    got = G.bf16_out_to_f64(out)
    assert np.all(got[[0, 2, 4]] == 0.0)
    G.compare(got, G.oracle_for(wl, call, seqs=[1, 3], window=window), "decode, empty seqs")


# ----------------------------------------------------------------- sliding window

WINDOW_PREFILL_CASES = [
    # (head_dim, page_size, lens, q_lens, window)
    (128, 16, [300, 777], [300, 200], 1),
    (128, 16, [300, 777], [300, 200], 50),
    (128, 256, [1000, 129], [1000, 129], 64),
    (128, 32, [513, 90], [400, 90], 200),
    (64, 16, [259, 31], [259, 31], 17),
    (128, 64, [700], [700], 5000),   # window longer than the sequence: no window
]


@pytest.mark.parametrize("d,ps,lens,q_lens,window", WINDOW_PREFILL_CASES)
def test_prefill_sliding_window(d, ps, lens, q_lens, window, prefill_path):
    G.banner(f"prefill window={window} d={d} ps={ps} lens={lens} q_lens={q_lens}")
    wl = W.build("win", 300 + window, heads=3, head_dim=d, page_size=ps, lens=lens,
                 q_lens=q_lens, causal=True, pool_slack=1.3, device="cuda", poison=True)
    call = wl.calls[0]
    out = torch.empty_like(call.q)
    B.pa_prefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, True,
                 wl.scale, out, call.q_start, call.max_q_len, window=window)
    torch.cuda.synchronize()
    ref = G.oracle_for(wl, call, window=window)
    G.compare(G.bf16_out_to_f64(out), ref, f"prefill window={window}")


@pytest.mark.parametrize("window,hq", [(1, 4), (7, 4), (256, 4), (1000, 4), (100000, 4),
                                       (1, 16), (40, 16), (777, 16)])
def test_decode_sliding_window(window, hq):
    G.banner(f"decode window={window} Hq={hq}")
    wl = W.build("wdec", 400 + window, heads=4, head_dim=128, page_size=16,
                 lens=[1, 15, 300, 777, 3000], kind="decode", pool_slack=1.2, device="cuda",
                 poison=True, q_heads=hq)
    call = wl.calls[0]
    out = torch.empty_like(call.q)
    ws = B.decode_workspace(call.q, wl.k_pool, call.block_table)
    B.pa_decode(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, wl.scale, out,
                ws, window=window)
    torch.cuda.synchronize()
    ref = G.oracle_for(wl, call, window=window)
    G.compare(G.bf16_out_to_f64(out), ref, f"decode window={window} Hq={hq}")


@pytest.mark.parametrize("window,ps", [(1024, 16), (259, 16), (257, 64), (1024, 256),
                                       (513, 256), (3, 32)])
def test_decode_window_split_alignment(window, ps):
    """The one-head-per-row decode lays a window's splits from its first key rounded down
    to a multiple of 4, the last split running to the sequence end: lengths put that
    first key at every residue mod 4 and on both sides of page and split boundaries."""
    G.banner(f"decode window split alignment window={window} ps={ps}")
    lens = [window + r for r in (0, 1, 2, 3, 5, 17, 255, 256, 257)] + [1, window - 1, 4099]
    lens = [max(1, x) for x in lens]
    wl = W.build("walign", 500 + window + ps, heads=4, head_dim=128, page_size=ps, lens=lens,
                 kind="decode", pool_slack=1.2, device="cuda", poison=True)
    call = wl.calls[0]
    out = torch.empty_like(call.q)
    ws = B.decode_workspace(call.q, wl.k_pool, call.block_table)
    B.pa_decode(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, wl.scale, out,
                ws, window=window)
    torch.cuda.synchronize()
    G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call, window=window),
              f"decode window={window} ps={ps}")


def test_window_one_returns_own_value_row(prefill_path):
    """w = 1: every query sees only its own key, so O is exactly its own V row."""
    G.banner("window=1 exactness")
    wl = W.build("w1", 77, heads=2, head_dim=128, page_size=16, lens=[333], q_lens=[100],
                 causal=True, device="cuda", poison=True)
    call = wl.calls[0]
    out = torch.empty_like(call.q)
    B.pa_prefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, True,
                 wl.scale, out, call.q_start, call.max_q_len, window=1)
    torch.cuda.synchronize()
    bt = call.block_table_host[0]
    for i in range(100):
        t = 333 - 100 + i
        assert torch.equal(out[i], wl.v_pool[int(bt[t // 16]), t % 16]), i


# ----------------------------------------------------------------- edge cases

@pytest.mark.parametrize("causal,hq", [(True, 2), (False, 2), (True, 4)])
def test_prefill_ragged_batch_with_empty_chunks(causal, hq, prefill_path):
    """Sequences with no query rows in the middle of a batch, a one-row chunk on a long
    cache, a chunk that is the whole sequence: rows past each chunk are never written."""
    G.banner(f"prefill ragged batch with empty chunks causal={causal} Hq={hq}")
    lens, q_lens = [10, 5, 7, 300, 64, 1], [0, 5, 0, 300, 1, 1]
    wl = W.build("rag", 61, heads=2, head_dim=128, page_size=16, lens=lens, q_lens=q_lens,
                 causal=causal, pool_slack=1.3, device="cuda", poison=True, q_heads=hq)
    call = wl.calls[0]
    out = torch.full_like(call.q, float("nan"))
    B.pa_prefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, causal,
                 wl.scale, out, call.q_start, call.max_q_len)
    torch.cuda.synchronize()
    ref = G.oracle_for(wl, call)
    G.compare(G.bf16_out_to_f64(out), ref, f"ragged causal={causal} Hq={hq}")


def test_zero_scale_averages_the_visible_values(prefill_path):
    """scale = 0: every visible key gets the same weight, so O is the mean of the
    visible V rows (causal prefill: a running mean; decode: the mean of the cache)."""
    G.banner("scale 0")
    for kind in ("prefill", "decode"):
        wl = W.build("z", 71, heads=2, head_dim=128, page_size=16, lens=[1, 333, 70],
                     q_lens=[1, 333, 20] if kind == "prefill" else None, kind=kind,
                     device="cuda", poison=True, scale=0.0)
        call = wl.calls[0]
        out = G.run_call(wl, call)
        torch.cuda.synchronize()
        G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call), f"scale 0 {kind}")


def test_prefill_window_grouped_heads(prefill_path):
    G.banner("prefill window=100 with 8 query heads over 2 K/V heads")
    wl = W.build("wg", 81, heads=2, head_dim=128, page_size=32, lens=[777, 300],
                 q_lens=[500, 300], causal=True, pool_slack=1.2, device="cuda", poison=True,
                 q_heads=8)
    call = wl.calls[0]
    out = torch.empty_like(call.q)
    B.pa_prefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, True,
                 wl.scale, out, call.q_start, call.max_q_len, window=100)
    torch.cuda.synchronize()
    ref = G.oracle_for(wl, call, window=100)
    G.compare(G.bf16_out_to_f64(out), ref, "prefill window=100 grouped")


@pytest.mark.parametrize("hq", [1, 4])
def test_decode_half_million_token_sequence(hq):
    """A 524,288-token sequence (2048 splits merged by the combine pass) next to a
    one-token one, pages of 256 shuffled over the pool."""
    G.banner(f"decode L=524288 Hq={hq}")
    wl = W.build("long", 91, heads=1, head_dim=128, page_size=256, lens=[524288, 1],
                 kind="decode", device="cuda", poison=True, q_heads=hq, sigma=0.5)
    call = wl.calls[0]
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call), f"decode long Hq={hq}")


# ----------------------------------------------------------------- kernel against kernel

def test_grouped_decode_kernel_agrees_with_per_head_kernel():
    """The same attention computed by the two decode kernels: 8 query heads over 2 K/V
    heads (grouped kernel) and over 8 K/V heads holding copies of those 2 (one K/V head
    per query head, the per-head kernel).  Both meet the oracle bar; they differ only by
    rounding order, so they agree to well within it."""
    G.banner("grouped vs per-head decode kernels")
    lens = [1, 300, 2500, 1025]
    wl = W.build("ab", 13, heads=2, head_dim=128, page_size=16, lens=lens, kind="decode",
                 pool_slack=1.2, device="cuda", poison=True, q_heads=8)
    call = wl.calls[0]
    grouped = G.run_call(wl, call)
    k_rep = wl.k_pool.repeat_interleave(4, dim=2).contiguous()
    v_rep = wl.v_pool.repeat_interleave(4, dim=2).contiguous()
    out = torch.empty_like(call.q)
    ws = B.decode_workspace(call.q, k_rep, call.block_table)
    B.pa_decode(call.q, k_rep, v_rep, call.block_table, call.seq_lens, wl.scale, out, ws)
    torch.cuda.synchronize()
    ref = G.oracle_for(wl, call)
    G.compare(G.bf16_out_to_f64(grouped), ref, "grouped kernel")
    G.compare(G.bf16_out_to_f64(out), ref, "per-head kernel")
    G.compare(G.bf16_out_to_f64(grouped), G.bf16_out_to_f64(out), "grouped vs per-head",
              max_tol=8e-3, mean_tol=5e-4)


@pytest.mark.parametrize("hq", [4, 16])
def test_decode_agrees_with_last_prefill_row(hq, prefill_path):
    """Decode (split-K VALU or grouped MFMA kernel plus the combine pass) and the last row
    of a causal prefill (tiled MFMA kernel) over the same cache compute the same thing."""
    G.banner(f"decode vs last prefill row Hq={hq}")
    lens = [1, 64, 257, 3000]
    wl = W.build("dp", 17, heads=4, head_dim=128, page_size=16, lens=lens, q_lens=lens,
                 causal=True, pool_slack=1.2, device="cuda", poison=True, q_heads=hq)
    call = wl.calls[0]
    pre = G.run_call(wl, call)
    last = torch.tensor([int(call.q_start_host[b + 1]) - 1 for b in range(len(lens))],
                        device="cuda")
    q_dec = call.q.index_select(0, last).contiguous()
    out = torch.empty_like(q_dec)
    ws = B.decode_workspace(q_dec, wl.k_pool, call.block_table)
    B.pa_decode(q_dec, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, wl.scale, out,
                ws)
    torch.cuda.synchronize()
    G.compare(G.bf16_out_to_f64(out), G.bf16_out_to_f64(pre.index_select(0, last)),
              "decode vs prefill last row", max_tol=8e-3, mean_tol=5e-4)


def test_prefill_131072_tokens_sampled():
    """One 131,072-token causal sequence (1 head, d=128, shuffled pages of 256): 1024
    query tiles, up to 2048 key tiles per workgroup; rows spread over the sequence."""
    G.banner("prefill N=131072, 1 head, rows sampled")
    n = 131072
    wl = W.build("pf_128k", 23, heads=1, head_dim=128, page_size=256, lens=[n], q_lens=[n],
                 causal=True, device="cuda")
    call = wl.calls[0]
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    rng = np.random.default_rng(24)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 65535, 65536, n - 129, n - 128, n - 1],
                                     rng.integers(0, n, 12)]))
    G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call, rows={0: rows}),
              "prefill N=131072")


@pytest.mark.parametrize("hq", [1, 4])
def test_decode_batch_at_the_api_limit(hq):
    """65,535 sequences (the most one call accepts, the largest grid dimension) of 1-40
    cached tokens, 1 K/V head, d=64: 400 sampled sequences, the first and the last
    included, against the oracle."""
    G.banner(f"decode batch 65535 Hq={hq}")
    rng = np.random.default_rng(25)
    lens = [int(x) for x in rng.integers(1, 41, size=65535)]
    wl = W.build("dec_65535", 26, heads=1, head_dim=64, page_size=16, lens=lens,
                 kind="decode", pool_slack=1.1, device="cuda", q_heads=hq)
    call = wl.calls[0]
    out = G.run_call(wl, call)
    torch.cuda.synchronize()
    seqs = sorted(set([0, 65534] + [int(x) for x in rng.integers(0, 65535, 398)]))
    G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call, seqs=seqs),
              f"decode batch 65535 Hq={hq}")


@pytest.mark.parametrize("batch,heads,d,lens,window,want", [
    (2, 32, 128, [4096, 3000], 0, 256),     # 2 x 16 splits x 8 head groups = 256 units
    (1, 32, 128, [4096], 0, 128),           # 128 units at 256 keys, 256 at 128
    (1, 4, 128, [16384], 0, 64),            # one head group: 64 units at 256 keys
    (1, 32, 64, [4096], 0, 64),             # d = 64: 4 groups of 8 heads
    (1, 4, 128, [16384], 300, 64),          # windowed, laid back from the end
    (3, 4, 128, [7000, 1, 16384], 1000, 128),  # 192 units at 256 keys, 384 at 128
    (1, 32, 128, [4096], 5, 128),
    # grouped heads (64 query heads over 8 K/V heads): 1024 keys, halved for small batches
    (1, (8, 64), 128, [4096], 0, 128),
    (2, (8, 64), 128, [4096, 2000], 0, 256),
    (1, (8, 64), 128, [4096], 300, 128),
    (8, (8, 64), 128, [4096] * 8, 0, 1024),
])
def test_decode_split_lengths(batch, heads, d, lens, window, want):
    """Small batches take shorter decode splits so that the chip's CUs all get work:
    128 or 64 keys instead of 256, and down to 128 instead of 1024 with grouped heads;
    each length against the oracle."""
    hkv, hq = heads if isinstance(heads, tuple) else (heads, heads)
    G.banner(f"decode split length batch={batch} Hkv={hkv} Hq={hq} d={d} lens={lens} "
             f"window={window}")
    wl = W.build("dsplit", 700 + len(lens) + hq + window, heads=hkv, head_dim=d,
                 page_size=16, lens=lens, kind="decode", pool_slack=1.2, device="cuda",
                 poison=True, q_heads=hq)
    call = wl.calls[0]
    assert B.pa_decode_split_tokens(batch, hq, B.layout_of(wl.k_pool, call.block_table)) \
        == want
    out = torch.empty_like(call.q)
    ws = B.decode_workspace(call.q, wl.k_pool, call.block_table)
    B.pa_decode(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, wl.scale, out,
                ws, window=window)
    torch.cuda.synchronize()
    G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call, window=window),
              f"decode split {want} window={window}")


@pytest.mark.parametrize("offset", [(1, -1), (1, 0), (1, 1), (2, -1), (2, 0), (2, 1), (3, 5)])
def test_decode_unit_counts_around_the_fixed_claims(offset):
    """The persistent decode's workgroup i takes units i and grid + i without the claim
    counter, which the plan starts at 2 x grid.  Unit counts just below, at and just
    above one and two grids (some workgroups find one or both fixed units empty; the
    counter hands out nothing, one unit or more) each against the oracle: 4 heads at
    d = 128 are one head group, so the units are the (sequence, 256-key split) pairs."""
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    mult, extra = offset
    target = mult * grid + extra
    batch = 64
    assert batch <= target <= 16 * batch
    rng = np.random.default_rng(target)
    splits = [16] + [1] * (batch - 1)  # one 4096-key sequence keeps the split at 256
    left = target - sum(splits)
    while left > 0:
        b = int(rng.integers(1, batch))
        if splits[b] < 16:
            splits[b] += 1
            left -= 1
    lens = [256 * (n - 1) + int(rng.integers(1, 257)) for n in splits]
    G.banner(f"decode unit count {target} (grid {grid}): lens={lens[:8]}...")
    wl = W.build("dclaims", 800 + target, heads=4, head_dim=128, page_size=16, lens=lens,
                 kind="decode", pool_slack=1.2, device="cuda", poison=True)
    call = wl.calls[0]
    assert B.pa_decode_split_tokens(batch, 4, B.layout_of(wl.k_pool, call.block_table)) == 256
    out = torch.empty_like(call.q)
    ws = B.decode_workspace(call.q, wl.k_pool, call.block_table)
    for rnd in range(2):  # the second call finds the counter where the first left it
        out.fill_(float("nan"))
        B.pa_decode(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, wl.scale,
                    out, ws)
        torch.cuda.synchronize()
        G.compare(G.bf16_out_to_f64(out), G.oracle_for(wl, call), f"units={target} call {rnd}")


@pytest.mark.parametrize("lens,window", [([4096, 0, 1, 700], 0), ([4096, 0, 1, 700], 300),
                                         ([1, 2, 3000], 0), ([8192, 65], 1000)])
def test_small_batch_decode_without_plan(lens, window):
    """A batch whose (sequence, split slot, head group) space holds at most one unit per
    CU runs pass 1 without the plan: workgroup i takes unit i, and split slots with no
    keys (an empty sequence, a one-key one, slots before a window) leave their
    workgroups without work.  Against the oracle, twice in a row on one workspace."""
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    G.banner(f"small-batch decode without the plan: lens={lens} window={window}")
    wl = W.build("noplan", 850 + len(lens) + window, heads=4, head_dim=128, page_size=16,
                 lens=lens, kind="decode", pool_slack=1.2, device="cuda", poison=True)
    call = wl.calls[0]
    lay = B.layout_of(wl.k_pool, call.block_table)
    split = B.pa_decode_split_tokens(len(lens), 4, lay)
    slots = len(lens) * -(-call.block_table.shape[1] * 16 // split)  # one head group
    assert slots <= grid, "this case is meant for the plan-free path"
    out = torch.empty_like(call.q)
    ws = B.decode_workspace(call.q, wl.k_pool, call.block_table)
    for rnd in range(2):
        out.fill_(float("nan"))
        B.pa_decode(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, wl.scale,
                    out, ws, window=window)
        torch.cuda.synchronize()
        got = G.bf16_out_to_f64(out)
        live = [b for b, L in enumerate(lens) if L > 0]
        empty = [b for b, L in enumerate(lens) if L == 0]
        assert np.all(got[empty] == 0.0)
        G.compare(got, G.oracle_for(wl, call, seqs=live, window=window),
                  f"no plan lens={lens} window={window} call {rnd}")
