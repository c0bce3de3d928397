"""The library's host-side block manager (pa_bm_*) on the CPU.

The manager only does bookkeeping, so its parity check needs no GPU: its tables and
copy lists drive host copies of the pools (written with the oracle's kv_append and
copy_pages), and after every operation each live sequence gathered through its
exported table must equal the logical cache (oracle/logical_cache.py) bit for bit.
Reference counts are recounted independently from the exported table."""
import numpy as np
import pytest

from exact_tiled_attention_pa_amd import binding as B
from oracle import attention as A
from oracle import logical_cache as LC
from tests.oracle_pins import to_bf16_bits

NAN = np.uint16(0x7FC0)


class PagedHost:
    """Host pools + manager + the logical cache, kept in step."""

    def __init__(self, num_pages, page_size, max_seqs, max_pages, heads=2, d=4, seed=0):
        self.rng = np.random.default_rng(seed)
        self.ps = page_size
        self.heads, self.d = heads, d
        self.bm = B.BlockManager(num_pages, page_size, max_seqs, max_pages)
        self.k = np.full((num_pages, page_size, heads, d), NAN, dtype=np.uint16)
        self.v = self.k.copy()
        self.ref = LC.LogicalCache(heads, d)
        self.copies = 0

    def rows(self, n):
        return (to_bf16_bits(self.rng.normal(size=(n, self.heads, self.d))),
                to_bf16_bits(self.rng.normal(size=(n, self.heads, self.d))))

    def add(self):
        s = self.bm.add_sequence()
        self.ref.add(s)
        return s

    def fork(self, parent, n):
        c = self.bm.fork(parent, n)
        self.ref.fork(parent, c, n)
        return c

    def free(self, s):
        self.bm.free_sequence(s)
        self.ref.free(s)

    def append(self, s, n):
        start = self.bm.seq_len(s)
        pairs = self.bm.append(s, n)
        if pairs:
            self.copies += len(pairs)
            self.k, self.v = LC.copy_pages(self.k, self.v, [p[0] for p in pairs],
                                           [p[1] for p in pairs])
        table, _ = self.bm.export()
        kn, vn = self.rows(n)
        self.k, self.v = A.kv_append(self.k, self.v, table, [s] * n, range(start, start + n),
                                     kn, vn)
        self.ref.append(s, kn, vn)
        return pairs

    def check(self):
        self.bm.validate()
        table, lens = self.bm.export()
        counts = np.zeros(self.k.shape[0], dtype=np.int64)
        for s in range(table.shape[0]):
            n = -(-int(lens[s]) // self.ps)
            counts[table[s, :n]] += 1 if n else 0
        for p in range(self.k.shape[0]):
            assert self.bm.ref_count(p) == counts[p], p
        assert self.bm.free_page_count() == int(np.sum(counts == 0))
        live = self.ref.live()
        for s in range(table.shape[0]):
            if s not in live:
                assert lens[s] == 0 and np.all(table[s] == -1)
                continue
            L = self.ref.length(s)
            assert lens[s] == L and self.bm.seq_len(s) == L
            lk, lv = self.ref.rows(s)
            # gather through the exported table, as the kernels do
            assert np.array_equal(A.gather_sequence(self.k, table[s], L, self.ps),
                                  A.bf16_to_f64(lk)), s
            assert np.array_equal(A.gather_sequence(self.v, table[s], L, self.ps),
                                  A.bf16_to_f64(lv)), s


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_match_logical_cache(seed):
    rng = np.random.default_rng(100 + seed)
    ph = PagedHost(num_pages=96, page_size=4, max_seqs=12, max_pages=16, seed=seed)
    first = ph.add()
    ph.append(first, 6)
    assert len(ph.append(ph.fork(first, 6), 1)) == 1   # one copy on write up front
    for _ in range(150):
        live = ph.ref.live()
        op = rng.choice(["append", "append", "append", "fork", "add", "free"])
        try:
            if op == "add" or not live:
                ph.add()
            elif op == "fork":
                p = int(rng.choice(live))
                ph.fork(p, int(rng.integers(0, ph.ref.length(p) + 1)))
            elif op == "free" and len(live) > 1:
                ph.free(int(rng.choice(live)))
            else:
                s = int(rng.choice(live))
                room = 16 * 4 - ph.ref.length(s)
                n = int(rng.choice([1, 1, 2, 3, 4, 5, 9]))
                if n <= room:
                    ph.append(s, n)
        except B.PagedAttnError as e:
            assert e.status == B.PA_ERR_CAPACITY, e
            # a failing call changes nothing
        ph.check()


def test_copy_on_write_copies_only_a_shared_partial_page():
    ph = PagedHost(num_pages=20, page_size=4, max_seqs=4, max_pages=5)
    a = ph.add()
    assert ph.append(a, 10) == []            # pages 0,1 full, page 2 holds 2 tokens
    b = ph.fork(a, 10)                        # shares all three pages
    table, _ = ph.bm.export()
    assert [ph.bm.ref_count(p) for p in table[a, :3]] == [2, 2, 2]
    pairs = ph.append(b, 1)                   # writes into the shared partial page
    assert len(pairs) == 1 and pairs[0][0] == table[a, 2]
    assert ph.append(a, 1) == []              # a is now its sole owner
    c = ph.fork(a, 8)                         # page-aligned prefix: nothing partial
    assert ph.append(c, 3) == [] and ph.append(a, 2) == []
    ph.check()
    ph.free(a)
    ph.free(b)
    ph.check()
    assert ph.bm.free_page_count() == 20 - 3  # c: two shared-then-owned pages + one
    ph.free(c)
    ph.check()
    assert ph.bm.free_page_count() == 20


def test_capacity_errors_change_nothing():
    ph = PagedHost(num_pages=4, page_size=4, max_seqs=2, max_pages=8)
    a = ph.add()
    ph.append(a, 14)
    b = ph.fork(a, 14)
    before = ph.bm.export()
    with pytest.raises(B.PagedAttnError) as e:
        ph.bm.append(b, 3)                    # copy of the partial page + 1 new page
    assert e.value.status == B.PA_ERR_CAPACITY
    with pytest.raises(B.PagedAttnError) as e:
        ph.bm.add_sequence()                  # both rows in use
    assert e.value.status == B.PA_ERR_CAPACITY
    after = ph.bm.export()
    assert np.array_equal(before[0], after[0]) and np.array_equal(before[1], after[1])
    ph.check()
    ph.free(a)                                 # frees nothing: every page is shared
    assert ph.bm.free_page_count() == 0
    ph.append(b, 2)                            # b owns its pages now: no copy needed
    assert ph.copies == 0
    ph.check()


def test_argument_errors():
    bm = B.BlockManager(8, 16, 2, 2)
    s = bm.add_sequence()
    for call, status in [
        (lambda: bm.fork(s, 1), B.PA_ERR_INVALID_ARG),      # parent holds 0 tokens
        (lambda: bm.fork(5, 0), B.PA_ERR_INVALID_ARG),
        (lambda: bm.free_sequence(1), B.PA_ERR_INVALID_ARG),
        (lambda: bm.append(s, 33), B.PA_ERR_INVALID_ARG),   # 2 pages of 16
        (lambda: bm.append(s, -1), B.PA_ERR_INVALID_ARG),
    ]:
        with pytest.raises(B.PagedAttnError) as e:
            call()
        assert e.value.status == status
    assert bm.seq_len(1) == -1 and bm.ref_count(8) == -1 and bm.ref_count(-1) == -1
    with pytest.raises(B.PagedAttnError):
        B.BlockManager(0, 16, 1, 1)
    with pytest.raises(B.PagedAttnError):
        B.BlockManager(8, 256, 1, 1 << 23)                  # 2^31 tokens per row
    lib = B.load_library()
    assert lib.pa_bm_seq_len(None, 0) == -1
    assert lib.pa_bm_free_page_count(None) == -1
    assert lib.pa_bm_validate(None) == B.PA_ERR_NULL
    lib.pa_bm_destroy(None)
