"""GPU parity of the KV-cache maintenance path: pa_kv_append and pa_copy_pages against
the oracle bit for bit (pure data movement), append-then-attend against the fp64
oracle, and the block manager driving the device pools through a serving loop
(prompts, forks that share a prefix, decode steps with copy on write, frees),
checked against the logical cache after every phase."""
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


def _bits(t: torch.Tensor) -> np.ndarray:
    return W.to_host_bits(t)


def _i32(x, device="cuda"):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=device)


APPEND_CASES = [
    # (head_dim, page_size, kv heads, lens of the sequences after the append)
    (128, 16, 4, [1, 17, 300, 64]),
    (64, 256, 1, [600, 255, 1]),
    (128, 256, 8, [513, 40]),
    (64, 32, 2, [95, 96, 97]),
]


@pytest.mark.parametrize("d,ps,hkv,lens", APPEND_CASES)
def test_kv_append_matches_oracle_bitwise(d, ps, hkv, lens):
    """Whole pools compared as bit patterns: every valid token lands in its slot, every
    other slot (NaN-poisoned tails, unused pages) keeps its bits; tokens with a bad
    sequence id, position or table entry are skipped."""
    G.banner(f"kv_append d={d} ps={ps} hkv={hkv} lens={lens}")
    wl = W.build("app", 500 + d + ps + hkv, heads=hkv, head_dim=d, page_size=ps, lens=lens,
                 kind="decode", pool_slack=1.4, device="cuda", poison=True)
    call = wl.calls[0]
    rng = np.random.default_rng(ps + d)
    # sequence 0 writes all its tokens (a prompt), the others their last few
    seq_ids, positions = [], []
    for b, L in enumerate(lens):
        first = 0 if b == 0 else max(0, L - 1 - b * 7)
        seq_ids += [b] * (L - first)
        positions += list(range(first, L))
    order = rng.permutation(len(seq_ids))
    seq_ids = [seq_ids[i] for i in order]
    positions = [positions[i] for i in order]
    n_valid = len(seq_ids)
    maxp = call.block_table_host.shape[1]
    # invalid tokens: bad sequence ids, negative or too-large positions, a -1 entry
    bad = [(len(lens), 0), (-1, 0), (0, -5), (0, maxp * ps), (0, maxp * ps + 17)]
    short = [b for b, L in enumerate(lens) if OA.pages_needed(L, ps) < maxp]
    if short:
        bad.append((short[0], maxp * ps - 1))   # maps to a table entry of -1
    seq_ids += [b for b, _ in bad]
    positions += [p for _, p in bad]
    n = len(seq_ids)
    k_new = W.normal_bf16((n, hkv, d), 1.0, 900 + n, "cuda")
    v_new = W.normal_bf16((n, hkv, d), 1.0, 901 + n, "cuda")
    k0, v0 = _bits(wl.k_pool), _bits(wl.v_pool)
    ref_k, ref_v = OA.kv_append(k0, v0, call.block_table_host, seq_ids[:n_valid],
                                positions[:n_valid], _bits(k_new)[:n_valid],
                                _bits(v_new)[:n_valid])
    B.pa_kv_append(k_new, v_new, _i32(seq_ids), _i32(positions), wl.k_pool, wl.v_pool,
                   call.block_table)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(wl.k_pool), ref_k)
    assert np.array_equal(_bits(wl.v_pool), ref_v)


def test_append_then_decode_matches_oracle():
    """The decode step: each sequence's newest token is written by pa_kv_append (its
    slot held NaN before), then pa_decode attends over the cache including it."""
    G.banner("append then decode")
    lens = [1, 16, 17, 500, 2049, 4096]
    hkv, d, ps = 4, 128, 16
    wl = W.build("ad", 77, heads=hkv, head_dim=d, page_size=ps, lens=lens, kind="decode",
                 pool_slack=1.2, device="cuda", poison=True)
    call = wl.calls[0]
    bt = call.block_table_host
    for b, L in enumerate(lens):     # the newest token is not in the cache yet
        page, slot = int(bt[b, (L - 1) // ps]), (L - 1) % ps
        wl.k_pool[page, slot] = float("nan")
        wl.v_pool[page, slot] = float("nan")
    k_new = W.normal_bf16((len(lens), hkv, d), 1.0, 78, "cuda")
    v_new = W.normal_bf16((len(lens), hkv, d), 1.0, 79, "cuda")
    seq_ids = list(range(len(lens)))
    positions = [L - 1 for L in lens]
    ref_k, ref_v = OA.kv_append(_bits(wl.k_pool), _bits(wl.v_pool), bt, seq_ids, positions,
                                _bits(k_new), _bits(v_new))
    B.pa_kv_append(k_new, v_new, _i32(seq_ids), _i32(positions), wl.k_pool, wl.v_pool,
                   call.block_table)
    out = torch.empty_like(call.q)
    ws = B.decode_workspace(call.q, wl.k_pool, call.block_table)
    B.pa_decode(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, wl.scale, out,
                ws)
    torch.cuda.synchronize()
    ref, _ = OA.paged_decode(_bits(call.q), ref_k, ref_v, bt, call.seq_lens_host, wl.scale)
    G.compare(G.bf16_out_to_f64(out), ref, "append+decode")


@pytest.mark.parametrize("d,ps,hkv", [(128, 16, 32), (64, 256, 8), (128, 256, 1)])
def test_copy_pages_matches_oracle_bitwise(d, ps, hkv):
    G.banner(f"copy_pages d={d} ps={ps} hkv={hkv}")
    num_pages = 40
    k = W.normal_bf16((num_pages, ps, hkv, d), 1.0, 11, "cuda")
    v = W.normal_bf16((num_pages, ps, hkv, d), 1.0, 12, "cuda")
    rng = np.random.default_rng(d + ps)
    perm = rng.permutation(num_pages)
    src, dst = list(perm[:12]), list(perm[12:24])
    k0, v0 = _bits(k), _bits(v)
    ref_k, ref_v = LC.copy_pages(k0, v0, src, dst)
    # pairs that must be skipped: out-of-range pages and src == dst
    src_all = src + [-1, num_pages, int(perm[30]), 5]
    dst_all = dst + [int(perm[31]), int(perm[32]), num_pages + 3, 5]
    B.pa_copy_pages(k, v, _i32(src_all), _i32(dst_all))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(k), ref_k)
    assert np.array_equal(_bits(v), ref_v)


class DeviceCache:
    """Block manager + device pools, mirrored by the logical cache."""

    def __init__(self, num_pages, ps, hkv, d, max_seqs, max_pages, seed):
        self.ps, self.hkv, self.d = ps, hkv, d
        self.seed = seed
        self.bm = B.BlockManager(num_pages, ps, max_seqs, max_pages)
        nan = torch.full((num_pages, ps, hkv, d), float("nan"), dtype=torch.bfloat16,
                         device="cuda")
        self.k, self.v = nan, nan.clone()
        self.ref = LC.LogicalCache(hkv, d)
        self.copies = 0
        self.table = None
        self.lens = None

    def _rows(self, n):
        self.seed += 2
        return (W.normal_bf16((n, self.hkv, self.d), 1.0, self.seed, "cuda"),
                W.normal_bf16((n, self.hkv, self.d), 1.0, self.seed + 1, "cuda"))

    def upload(self):
        table, lens = self.bm.export()
        self.table = torch.from_numpy(table).cuda()
        self.lens = lens

    def append_many(self, seqs_and_counts):
        """One batched pa_kv_append for several sequences (copies first)."""
        ids, pos, pairs = [], [], []
        for s, n in seqs_and_counts:
            start = self.bm.seq_len(s)
            pairs += self.bm.append(s, n)
            ids += [s] * n
            pos += list(range(start, start + n))
        if pairs:
            self.copies += len(pairs)
            B.pa_copy_pages(self.k, self.v, _i32([p[0] for p in pairs]),
                            _i32([p[1] for p in pairs]))
        self.upload()
        kn, vn = self._rows(len(ids))
        B.pa_kv_append(kn, vn, _i32(ids), _i32(pos), self.k, self.v, self.table)
        kb, vb = _bits(kn), _bits(vn)
        off = 0
        for s, n in seqs_and_counts:
            self.ref.append(s, kb[off:off + n], vb[off:off + n])
            off += n

    def check_contents(self):
        torch.cuda.synchronize()
        self.bm.validate()
        table, lens = self.bm.export()
        k, v = _bits(self.k), _bits(self.v)
        for s in self.ref.live():
            L = self.ref.length(s)
            assert lens[s] == L
            lk, lv = self.ref.rows(s)
            assert np.array_equal(OA.gather_sequence(k, table[s], L, self.ps),
                                  OA.bf16_to_f64(lk)), s
            assert np.array_equal(OA.gather_sequence(v, table[s], L, self.ps),
                                  OA.bf16_to_f64(lv)), s

    def check_decode(self, scale):
        """pa_decode over every live sequence against the oracle on the logical rows."""
        live = self.ref.live()
        self.upload()
        hq = self.hkv * 2   # two query heads per KV head
        q = W.normal_bf16((self.bm.max_seqs, hq, self.d), 1.0, self.seed + 99, "cuda")
        lens = torch.from_numpy(self.lens).cuda()
        out = torch.zeros_like(q)
        ws = B.decode_workspace(q, self.k, self.table)
        B.pa_decode(q, self.k, self.v, self.table, lens, scale, out, ws)
        torch.cuda.synchronize()
        got = G.bf16_out_to_f64(out)
        qf = OA.bf16_to_f64(_bits(q))
        ref = np.full(got.shape, np.nan)
        for s in live:
            lk, lv = self.ref.rows(s)
            L = lk.shape[0]
            # two query heads per K/V head: the oracle maps them onto the K/V heads
            o, _ = OA.attend(qf[s:s + 1], OA.bf16_to_f64(lk), OA.bf16_to_f64(lv),
                             np.array([L - 1]), True, scale)
            ref[s] = o[0]
        G.compare(got, ref, f"block-manager decode over {len(live)} sequences")


def test_block_manager_serving_loop_on_gpu():
    G.banner("block manager serving loop: prompts, forks, decode steps with copy on write")
    ps, hkv, d = 16, 4, 128
    dc = DeviceCache(num_pages=400, ps=ps, hkv=hkv, d=d, max_seqs=16, max_pages=64, seed=5)
    scale = float(np.float32(1 / np.sqrt(d)))
    a, b = dc.bm.add_sequence(), dc.bm.add_sequence()
    dc.ref.add(a)
    dc.ref.add(b)
    dc.append_many([(a, 333), (b, 64)])             # two prompts
    dc.check_contents()
    # parallel samples of prompt a share its 333 tokens (20 full pages + 13 tokens)
    forks = []
    for _ in range(3):
        c = dc.bm.fork(a, 333)
        dc.ref.fork(a, c, 333)
        forks.append(c)
    c2 = dc.bm.fork(b, 40)                          # a shorter shared prefix of b
    dc.ref.fork(b, c2, 40)
    live = [a, b] + forks + [c2]
    for step in range(24):                          # decode steps: one token each
        dc.append_many([(s, 1) for s in live])
        if step in (0, 5, 23):
            dc.check_contents()
    assert dc.copies >= 4                           # a's partial page for 3 forks + c2's
    dc.check_decode(scale)
    dc.bm.free_sequence(forks[0])
    dc.ref.free(forks[0])
    dc.bm.free_sequence(a)
    dc.ref.free(a)
    dc.append_many([(forks[1], 40), (c2, 3)])       # a chunk crossing pages
    dc.check_contents()
    dc.check_decode(scale)
