"""Pins for the CPU oracle: checks against values the pages print, closed forms,
invariants, brute force and a library routine.  Each pin returns True/False so
that the same checks can be run against deliberately broken copies of the
oracle (see test_oracle_mutations.py) as well as against the real one.

Nothing here calls the HIP library.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import attention as A
from oracle import logical_cache as LC

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------- helpers

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32/fp64 values -> bf16 bit patterns, round to nearest even (via torch)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_of_int(v):
    """bf16 bits of a small non-negative integer (exact for 0..256)."""
    return to_bf16_bits(np.array(v, dtype=np.float32))


def random_paged_case(rng, batch, heads, d, page_size, lens, q_lens, extra_pages=3,
                      sigma=1.0, poison=True, q_heads=None):
    """A tiny paged problem with a shuffled pool, NaN in every unread slot.  heads is
    the pools' K/V head count; q_heads (default heads) the query head count."""
    n_pages = [A.pages_needed(L, page_size) for L in lens]
    num_pages = sum(n_pages) + extra_pages
    perm = rng.permutation(num_pages)
    maxp = max(n_pages)
    table = np.full((batch, maxp), -1, dtype=np.int64)
    cursor = 0
    for b, n in enumerate(n_pages):
        table[b, :n] = perm[cursor:cursor + n]
        cursor += n
    k = to_bf16_bits(rng.normal(0.0, sigma, (num_pages, page_size, heads, d)))
    v = to_bf16_bits(rng.normal(0.0, sigma, (num_pages, page_size, heads, d)))
    if poison:
        nan = np.uint16(0x7FC0)
        used = np.zeros((num_pages, page_size), dtype=bool)
        for b, L in enumerate(lens):
            for j in range(n_pages[b]):
                valid = min(page_size, L - j * page_size)
                used[table[b, j], :valid] = True
        k[~used] = nan
        v[~used] = nan
    q_start = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    q = to_bf16_bits(rng.normal(0.0, sigma, (int(q_start[-1]), q_heads or heads, d)))
    return dict(q=q, k=k, v=v, table=table, lens=np.array(lens), q_start=q_start)


def brute_force(q, k, v, table, lens, q_start, causal, scale, window=0, kv_of=None):
    """Scalar Python loops with math.exp; walks each sequence's pages in table order.

    Written independently of oracle.attention: no numpy arithmetic, and the
    keys of a sequence are collected page by page (slot o of the j-th listed
    page is token j*page_size + o) instead of by dividing token positions.
    kv_of: explicit list, query head -> the K/V head it reads (default: the same
    head, multi-head attention).
    """
    page_size = k.shape[1]
    heads, d = q.shape[1], q.shape[2]
    if kv_of is None:
        kv_of = list(range(heads))
    kf = k.astype(np.uint32) << 16
    vf = v.astype(np.uint32) << 16
    kf = kf.view(np.float32).astype(np.float64).tolist()
    vf = vf.view(np.float32).astype(np.float64).tolist()
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64).tolist()
    out = [[[0.0] * d for _ in range(heads)] for _ in range(len(qf))]
    for b in range(len(lens)):
        L = int(lens[b])
        keys, vals = [], []
        j = 0
        while len(keys) < L:
            phys = int(table[b][j])
            for o in range(page_size):
                if len(keys) == L:
                    break
                keys.append(kf[phys][o])
                vals.append(vf[phys][o])
            j += 1
        q_len = int(q_start[b + 1] - q_start[b])
        for i in range(q_len):
            row = int(q_start[b]) + i
            last = L - q_len + i if causal else L - 1
            first = max(0, last - window + 1) if window else 0
            for h in range(heads):
                s = []
                hk = kv_of[h]
                for t in range(first, last + 1):
                    acc = 0.0
                    for c in range(d):
                        acc += qf[row][h][c] * keys[t][hk][c]
                    s.append(scale * acc)
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = sum(e)
                for c in range(d):
                    acc = 0.0
                    for t in range(first, last + 1):
                        acc += e[t - first] * vals[t][hk][c]
                    out[row][h][c] = acc / tot
    return np.array(out)


# --------------------------------------------------------------------------- pins

def pin_practical_example_translation() -> bool:
    """The page's worked example: token 300 -> logical 1, offset 44, physical 1."""
    g = load_golden("paged_flashattention_practical_example.json")
    for tok in g["tokens"]:
        got = A.locate_token(g["block_table"], tok["token"], g["page_size"])
        want = (tok["logical_page"], tok["offset"], tok["physical_page"])
        if tuple(got) != want:
            return False
    return True


def pin_practical_example_gather() -> bool:
    """Encoded pool: slot (p, o, h) stores p, o//2, o%2 and h in its first channels
    (small integers, exact in bf16).  Gathering the worked example's sequence must
    return, at token 300, the slot (physical 1, offset 44), and must never read a
    NaN-poisoned slot (tail of page 9 past its 88 valid tokens, unused pages).
    """
    g = load_golden("paged_flashattention_practical_example.json")
    ps, L, table = g["page_size"], g["seq_len"], g["block_table"]
    num_pages, heads, d = 12, 2, 8
    pool = np.full((num_pages, ps, heads, d), 0x7FC0, dtype=np.uint16)
    enc = np.zeros((num_pages, ps, heads, d), dtype=np.float32)
    for p in range(num_pages):
        enc[p, :, :, 0] = p
    enc[:, :, :, 1] = (np.arange(ps) // 2)[None, :, None]
    enc[:, :, :, 2] = (np.arange(ps) % 2)[None, :, None]
    enc[:, :, :, 3] = np.arange(heads)[None, None, :]
    bits = to_bf16_bits(enc)
    for j, phys in enumerate(table):
        valid = min(ps, L - j * ps)
        pool[phys, :valid] = bits[phys, :valid]
    try:
        rows = A.gather_sequence(pool, table, L, ps)
    except (IndexError, ValueError):
        return False
    if not np.all(np.isfinite(rows)):
        return False
    for tok in g["tokens"]:
        r = rows[tok["token"]]
        phys = int(r[0, 0])
        off = int(r[0, 1]) * 2 + int(r[0, 2])
        if (phys, off) != (tok["physical_page"], tok["offset"]):
            return False
        if int(r[1, 3]) != 1:
            return False
    # the last page of the example holds L - 2*256 = 88 tokens (derived, not printed)
    last = rows[L - 1]
    return (int(last[0, 0]), int(last[0, 1]) * 2 + int(last[0, 2])) == (9, 87)


def pin_page_count_example() -> bool:
    """The vLLM flowchart: 200 tokens -> 13 pages with 8 in the last; 32 -> 2 pages."""
    g = load_golden("vllm_page_count_example.json")
    ps = g["page_size"]
    for r in g["requests"]:
        n = A.pages_needed(r["tokens"], ps)
        if n != r["pages"] or r["tokens"] - (n - 1) * ps != r["last_page_tokens"]:
            return False
    return True


def pin_brute_force(seed=0) -> bool:
    """Whole result vs scalar loops on tiny shapes, causal chunks and non-causal."""
    rng = np.random.default_rng(seed)
    cases = [
        dict(batch=2, heads=2, d=4, page_size=4, lens=[7, 13], q_lens=[7, 5]),
        dict(batch=1, heads=1, d=3, page_size=1, lens=[9], q_lens=[4]),
        dict(batch=2, heads=2, d=4, page_size=16, lens=[20, 3], q_lens=[2, 3]),
        dict(batch=2, heads=1, d=4, page_size=2, lens=[5, 11], q_lens=[1, 11]),
    ]
    for c in cases:
        case = random_paged_case(rng, c["batch"], c["heads"], c["d"], c["page_size"],
                                 c["lens"], c["q_lens"])
        for causal in (True, False):
            scale = float(np.float32(0.37))
            want = brute_force(case["q"], case["k"], case["v"], case["table"], case["lens"],
                               case["q_start"], causal, scale)
            try:
                got, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"],
                                         case["lens"], case["q_start"], causal, scale)
            except (AssertionError, ValueError, IndexError):
                return False
            if not np.all(np.isfinite(got)) or np.max(np.abs(got - want)) > 1e-13:
                return False
    return True


def pin_sdpa_fp64(seed=1) -> bool:
    """Identity block table vs torch's scaled_dot_product_attention in float64 on CPU:
    is_causal for a full prefill (q_len = L), an explicit bottom-right boolean mask for
    a chunk (q_len < L), no mask for a non-causal chunk."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    for (L, q_len, heads, d, ps, causal) in [(70, 70, 3, 16, 16, True), (70, 70, 2, 8, 8, False),
                                             (90, 33, 2, 16, 32, True), (90, 33, 2, 16, 32, False)]:
        n = A.pages_needed(L, ps)
        table = np.arange(n)[None, :]
        k = to_bf16_bits(rng.normal(size=(n, ps, heads, d)))
        v = to_bf16_bits(rng.normal(size=(n, ps, heads, d)))
        q = to_bf16_bits(rng.normal(size=(q_len, heads, d)))
        scale = float(np.float32(1.0 / math.sqrt(d)))
        try:
            got, _ = A.paged_prefill(q, k, v, table, [L], [0, q_len], causal, scale)
        except (AssertionError, ValueError, IndexError):
            return False
        kk = torch.from_numpy(A.bf16_to_f64(k).reshape(n * ps, heads, d)[:L]).permute(1, 0, 2)
        vv = torch.from_numpy(A.bf16_to_f64(v).reshape(n * ps, heads, d)[:L]).permute(1, 0, 2)
        qq = torch.from_numpy(A.bf16_to_f64(q)).permute(1, 0, 2)
        if causal and q_len == L:
            ref = F.scaled_dot_product_attention(qq, kk, vv, is_causal=True, scale=scale)
        elif causal:
            mask = torch.ones(q_len, L, dtype=torch.bool).tril(diagonal=L - q_len)
            ref = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale)
        else:
            ref = F.scaled_dot_product_attention(qq, kk, vv, scale=scale)
        ref = ref.permute(1, 0, 2).numpy()
        if np.max(np.abs(got - ref)) > 1e-12:
            return False
    return True


def pin_closed_forms(seed=2) -> bool:
    """Special cases with a closed-form answer."""
    rng = np.random.default_rng(seed)
    heads, d, ps = 2, 8, 4
    scale = float(np.float32(0.35355339))
    # (1) L = 1: the only key's value is the output, whatever q and k are
    case = random_paged_case(rng, 1, heads, d, ps, [1], [1])
    got, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"], case["lens"],
                             case["q_start"], True, scale)
    v0 = A.bf16_to_f64(case["v"][case["table"][0, 0], 0])
    if np.max(np.abs(got[0] - v0)) > 1e-15:
        return False
    # (2) causal full prefill: row 0 sees only key 0
    case = random_paged_case(rng, 1, heads, d, ps, [10], [10])
    got, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"], case["lens"],
                             case["q_start"], True, scale)
    v0 = A.bf16_to_f64(case["v"][case["table"][0, 0], 0])
    if np.max(np.abs(got[0] - v0)) > 1e-15:
        return False
    # (3) zero keys: uniform weights, output = mean of the visible values
    case = random_paged_case(rng, 1, heads, d, ps, [11], [5])
    used = case["table"][0, :A.pages_needed(11, ps)]
    case["k"][used] = 0
    got, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"], case["lens"],
                             case["q_start"], True, scale)
    vals = np.concatenate([A.bf16_to_f64(case["v"][p]) for p in used])[:11]
    for i in range(5):
        pos = 11 - 5 + i
        if np.max(np.abs(got[i] - vals[:pos + 1].mean(axis=0))) > 1e-14:
            return False
    # (4) constant values c: output = c for every row
    case = random_paged_case(rng, 1, heads, d, ps, [13], [13])
    used = case["table"][0, :A.pages_needed(13, ps)]
    case["v"][used] = to_bf16_bits(np.full((heads, d), 1.75, dtype=np.float32))
    got, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"], case["lens"],
                             case["q_start"], False, scale)
    if np.max(np.abs(got - 1.75)) > 1e-14:
        return False
    # (5) spike: one key scores 2048 above all others (exp(-2048) is exactly 0 in
    #     fp64), so the output is exactly that key's value
    L = 14
    case = random_paged_case(rng, 1, heads, d, ps, [L], [1])
    pages = case["table"][0, :A.pages_needed(L, ps)]
    case["k"][pages] = 0
    target = 9
    tp, to = pages[target // ps], target % ps
    k_spike = np.zeros((heads, d), dtype=np.float32)
    k_spike[:, 3] = 1024.0
    case["k"][tp, to] = to_bf16_bits(k_spike)
    qv = np.zeros((1, heads, d), dtype=np.float32)
    qv[0, :, 3] = 2.0
    case["q"] = to_bf16_bits(qv)
    got, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"], case["lens"],
                             case["q_start"], True, 1.0)
    return bool(np.array_equal(got[0], A.bf16_to_f64(case["v"][tp, to])))


def pin_permutation_invariance(seed=3) -> bool:
    """Relabel physical pages (shuffle the pool, remap the table): bit-identical output."""
    rng = np.random.default_rng(seed)
    case = random_paged_case(rng, 2, 2, 8, 4, [9, 14], [9, 6])
    base, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"], case["lens"],
                              case["q_start"], True, 0.3)
    num_pages = case["k"].shape[0]
    sigma = rng.permutation(num_pages)          # new physical slot of old page p
    k2 = np.empty_like(case["k"])
    v2 = np.empty_like(case["v"])
    k2[sigma] = case["k"]
    v2[sigma] = case["v"]
    t2 = np.where(case["table"] >= 0, sigma[np.maximum(case["table"], 0)], -1)
    moved, _ = A.paged_prefill(case["q"], k2, v2, t2, case["lens"], case["q_start"], True, 0.3)
    return bool(np.array_equal(base, moved))


def pin_shared_prefix(seed=4) -> bool:
    """Two block tables sharing their first two physical pages (the page's conceptual
    example).  For the same query rows inside the shared prefix the outputs are identical;
    past the prefix they differ."""
    g = load_golden("shared_prefix_block_tables.json")
    t1, t2 = g["block_tables"]["request_1"], g["block_tables"]["request_2"]
    rng = np.random.default_rng(seed)
    ps, heads, d = 4, 2, 8
    num_pages = 16
    k = to_bf16_bits(rng.normal(size=(num_pages, ps, heads, d)))
    v = to_bf16_bits(rng.normal(size=(num_pages, ps, heads, d)))
    L = 3 * ps
    table = np.array([t1, t2])
    q_one = to_bf16_bits(rng.normal(size=(L, heads, d)))
    q = np.concatenate([q_one, q_one])
    out, _ = A.paged_prefill(q, k, v, table, [L, L], [0, L, 2 * L], True, 0.3)
    prefix = g["shared_prefix_blocks"] * ps
    same = np.array_equal(out[:prefix], out[L:L + prefix])
    differ = not np.allclose(out[prefix:L], out[L + prefix:2 * L])
    return bool(same and differ)


def pin_rows_sum_to_one(seed=5) -> bool:
    """Every softmax row over visible keys sums to 1 (checked inside the oracle too)."""
    rng = np.random.default_rng(seed)
    s = rng.normal(size=(6, 9)) * 30
    mask = np.tril(np.ones((6, 9), dtype=bool), k=3)
    p, _ = A.softmax_rows(s, mask)
    return bool(np.max(np.abs(p.sum(axis=1) - 1)) < 1e-12 and np.all(p[~mask] == 0))


def pin_decode_matches_last_row(seed=6) -> bool:
    """A decode query equals the last row of a causal prefill over the same cache."""
    rng = np.random.default_rng(seed)
    case = random_paged_case(rng, 2, 2, 8, 4, [6, 17], [6, 17])
    full, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"], case["lens"],
                              case["q_start"], True, 0.4)
    last_rows = case["q_start"][1:] - 1
    dec, _ = A.paged_decode(case["q"][last_rows], case["k"], case["v"], case["table"],
                            case["lens"], 0.4)
    return bool(np.max(np.abs(dec - full[last_rows])) < 1e-14)


def pin_sliding_window(seed=7) -> bool:
    """Window w (the previous w tokens, own key included): brute force on chunked
    causal cases; w = 1 returns the query's own V row; w >= L changes no bit; a band
    mask in float64 SDPA agrees; decode sees the last w keys."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    case = random_paged_case(rng, 2, 2, 4, 4, [13, 9], [6, 9])
    scale = float(np.float32(0.41))
    for w in (1, 3, 7):
        want = brute_force(case["q"], case["k"], case["v"], case["table"], case["lens"],
                           case["q_start"], True, scale, window=w)
        got, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"], case["lens"],
                                 case["q_start"], True, scale, window=w)
        if np.max(np.abs(got - want)) > 1e-13:
            return False
    # w = 1: only the query's own key -> its V row, exactly
    got, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"], case["lens"],
                             case["q_start"], True, scale, window=1)
    for b, L in enumerate(case["lens"]):
        q0, q1 = case["q_start"][b], case["q_start"][b + 1]
        for i in range(q1 - q0):
            t = L - (q1 - q0) + i
            phys = case["table"][b][t // 4]
            if not np.array_equal(got[q0 + i], A.bf16_to_f64(case["v"][phys, t % 4])):
                return False
    # a window covering everything is no window
    full, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"], case["lens"],
                              case["q_start"], True, scale)
    wide, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"], case["lens"],
                              case["q_start"], True, scale, window=13)
    if not np.array_equal(full, wide):
        return False
    # SDPA with an explicit band mask, identity table
    L, q_len, heads, d, ps, w = 40, 40, 2, 8, 8, 5
    n = A.pages_needed(L, ps)
    k = to_bf16_bits(rng.normal(size=(n, ps, heads, d)))
    v = to_bf16_bits(rng.normal(size=(n, ps, heads, d)))
    q = to_bf16_bits(rng.normal(size=(q_len, heads, d)))
    got, _ = A.paged_prefill(q, k, v, np.arange(n)[None, :], [L], [0, q_len], True, scale,
                             window=w)
    kk = torch.from_numpy(A.bf16_to_f64(k).reshape(n * ps, heads, d)[:L]).permute(1, 0, 2)
    vv = torch.from_numpy(A.bf16_to_f64(v).reshape(n * ps, heads, d)[:L]).permute(1, 0, 2)
    qq = torch.from_numpy(A.bf16_to_f64(q)).permute(1, 0, 2)
    band = torch.ones(q_len, L, dtype=torch.bool).tril(0) & ~torch.ones(q_len, L, dtype=torch.bool).tril(-w)
    ref = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=band, scale=scale)
    if np.max(np.abs(got - ref.permute(1, 0, 2).numpy())) > 1e-12:
        return False
    # decode with a window = last row of the windowed causal prefill
    last_rows = case["q_start"][1:] - 1
    dec, _ = A.paged_decode(case["q"][last_rows], case["k"], case["v"], case["table"],
                            case["lens"], scale, window=3)
    pre, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"], case["lens"],
                             case["q_start"], True, scale, window=3)
    return bool(np.max(np.abs(dec - pre[last_rows])) < 1e-14)


def pin_kv_append_round_trip(seed=8) -> bool:
    """Appending a sequence's K/V token by token into an empty (NaN) paged pool and
    gathering it back returns exactly the appended rows; the worked example's token
    300 lands in physical page 1, slot 44; no other slot changes."""
    g = load_golden("paged_flashattention_practical_example.json")
    ps, L, table = g["page_size"], g["seq_len"], g["block_table"]
    rng = np.random.default_rng(seed)
    heads, d, num_pages = 2, 4, 12
    nan = np.uint16(0x7FC0)
    k0 = np.full((num_pages, ps, heads, d), nan, dtype=np.uint16)
    v0 = np.full((num_pages, ps, heads, d), nan, dtype=np.uint16)
    kn = to_bf16_bits(rng.normal(size=(L, heads, d)))
    vn = to_bf16_bits(rng.normal(size=(L, heads, d)))
    order = rng.permutation(L)  # append order must not matter
    k1, v1 = A.kv_append(k0, v0, [table], [0] * L, order, kn[order], vn[order])
    if not np.array_equal(A.gather_sequence(k1, table, L, ps), A.bf16_to_f64(kn)):
        return False
    if not np.array_equal(A.gather_sequence(v1, table, L, ps), A.bf16_to_f64(vn)):
        return False
    for tok in g["tokens"]:
        if not np.array_equal(k1[tok["physical_page"], tok["offset"]], kn[tok["token"]]):
            return False
    written = np.zeros((num_pages, ps), dtype=bool)
    for j, phys in enumerate(table):
        written[phys, :min(ps, L - j * ps)] = True
    return bool(np.all(k1[~written] == nan) and np.all(v1[~written] == nan))


def pin_logical_cache_fork_isolation(seed=9) -> bool:
    """A fork starts with exactly the parent's first n rows; appends to the fork and to
    the parent never show up in the other (copy on write); freeing one leaves the other
    whole; lengths add up."""
    rng = np.random.default_rng(seed)
    heads, d = 2, 4
    rows = lambda n: to_bf16_bits(rng.normal(size=(n, heads, d)))
    cache = LC.LogicalCache(heads, d)
    a_k, a_v = rows(10), rows(10)
    cache.add(0)
    cache.append(0, a_k[:4], a_v[:4])
    cache.append(0, a_k[4:], a_v[4:])
    cache.fork(0, 1, 6)
    cache.fork(0, 2, 0)
    b_k, b_v = rows(4), rows(4)
    c_k, c_v = rows(3), rows(3)
    cache.append(1, b_k, b_v)
    cache.append(0, c_k, c_v)
    k0, v0 = cache.rows(0)
    k1, v1 = cache.rows(1)
    ok = (np.array_equal(k0, np.concatenate([a_k, c_k])) and
          np.array_equal(v0, np.concatenate([a_v, c_v])) and
          np.array_equal(k1, np.concatenate([a_k[:6], b_k])) and
          np.array_equal(v1, np.concatenate([a_v[:6], b_v])) and
          cache.length(0) == 13 and cache.length(1) == 10 and cache.length(2) == 0)
    cache.free(0)
    k1b, v1b = cache.rows(1)
    return bool(ok and np.array_equal(k1, k1b) and np.array_equal(v1, v1b)
                and cache.live() == [1, 2])


def pin_shared_prefix_pages_hold_both_sequences(seed=10) -> bool:
    """The first page's shared-prefix example, paged: request 1 fills pages [3, 7, 12],
    request 2 shares its first two pages and continues in page 9.  Writing both through
    kv_append and gathering each through its own table gives each sequence's logical
    rows; the page copy of copy on write moves every slot of a page and nothing else."""
    g = load_golden("shared_prefix_block_tables.json")
    t1, t2 = g["block_tables"]["request_1"], g["block_tables"]["request_2"]
    shared = g["shared_prefix_blocks"]
    rng = np.random.default_rng(seed)
    ps, heads, d, num_pages = 4, 1, 4, 13
    rows = lambda n: to_bf16_bits(rng.normal(size=(n, heads, d)))
    nan = np.uint16(0x7FC0)
    k = np.full((num_pages, ps, heads, d), nan, dtype=np.uint16)
    v = k.copy()
    cache = LC.LogicalCache(heads, d)
    cache.add(1)
    k1, v1 = rows(3 * ps - 1), rows(3 * ps - 1)
    cache.append(1, k1, v1)
    k, v = A.kv_append(k, v, [t1], [0] * len(k1), range(len(k1)), k1, v1)
    cache.fork(1, 2, shared * ps)
    k2, v2 = rows(3), rows(3)
    cache.append(2, k2, v2)
    pos2 = range(shared * ps, shared * ps + 3)
    k, v = A.kv_append(k, v, [t1, t2], [1] * 3, pos2, k2, v2)
    for seq, table in ((1, t1), (2, t2)):
        L = cache.length(seq)
        lk, lv = cache.rows(seq)
        if not (np.array_equal(A.gather_sequence(k, table, L, ps), A.bf16_to_f64(lk)) and
                np.array_equal(A.gather_sequence(v, table, L, ps), A.bf16_to_f64(lv))):
            return False
    ck, cv = LC.copy_pages(k, v, [t1[2]], [0])
    untouched = [p for p in range(num_pages) if p != 0]
    return bool(np.array_equal(ck[0], k[t1[2]]) and np.array_equal(cv[0], v[t1[2]]) and
                np.array_equal(ck[untouched], k[untouched]) and
                np.array_equal(cv[untouched], v[untouched]))


def _flowchart_groups():
    """The flowchart's membership lists, zero-based: query head -> K/V head."""
    g = load_golden("gqa_attention_variants_flowchart.json")["gqa_flowchart"]
    kv_of = [None] * g["n_q_heads"]
    for group, members in g["groups"].items():
        for head in members:
            kv_of[head - 1] = int(group) - 1
    return g, kv_of


def pin_gqa_flowchart_mapping() -> bool:
    """The page's grouped-query flowchart, exactly: with 8 query heads over 2 K/V
    heads, heads 1-4 read group 1 and 5-8 read group 2; the 4x and 8x KV-cache
    reductions are the group sizes; MQA maps every head to the one K/V head and MHA
    maps each head to its own."""
    g, kv_of = _flowchart_groups()
    nq, nkv = g["n_q_heads"], g["n_kv_heads"]
    if [A.kv_head_of(h, nq, nkv) for h in range(nq)] != kv_of:
        return False
    if nq // nkv != g["kv_cache_reduction_vs_mha"]:
        return False
    big = load_golden("gqa_attention_variants_flowchart.json")["gqa_64_over_8"]
    got = [A.kv_head_of(h, big["n_q_heads"], big["n_kv_heads"]) for h in range(big["n_q_heads"])]
    sizes = [got.count(j) for j in range(big["n_kv_heads"])]
    if sizes != [big["kv_cache_reduction_vs_mha"]] * big["n_kv_heads"] or got != sorted(got):
        return False
    if any(A.kv_head_of(h, 7, 1) != 0 for h in range(7)):
        return False
    return all(A.kv_head_of(h, 5, 5) == h for h in range(5))


def pin_gqa_brute_force(seed=11) -> bool:
    """Grouped heads against scalar loops that read the flowchart's membership lists
    (8 query heads, 2 K/V heads), causal chunks, non-causal, and decode."""
    _, kv_of = _flowchart_groups()
    rng = np.random.default_rng(seed)
    case = random_paged_case(rng, 2, 2, 3, 4, [9, 6], [4, 6], q_heads=8)
    scale = float(np.float32(0.43))
    for causal in (True, False):
        want = brute_force(case["q"], case["k"], case["v"], case["table"], case["lens"],
                           case["q_start"], causal, scale, kv_of=kv_of)
        got, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"], case["lens"],
                                 case["q_start"], causal, scale)
        if not np.all(np.isfinite(got)) or np.max(np.abs(got - want)) > 1e-13:
            return False
    last_rows = case["q_start"][1:] - 1
    dec, _ = A.paged_decode(case["q"][last_rows], case["k"], case["v"], case["table"],
                            case["lens"], scale)
    want = brute_force(case["q"], case["k"], case["v"], case["table"], case["lens"],
                       case["q_start"], True, scale, kv_of=kv_of)
    return bool(np.max(np.abs(dec - want[last_rows])) < 1e-13)


def pin_gqa_equals_replicated_heads(seed=12) -> bool:
    """Grouped attention is multi-head attention over pools in which every query head
    has its own copy of the K/V head the flowchart assigns it: bit-identical."""
    _, kv_of = _flowchart_groups()
    rng = np.random.default_rng(seed)
    case = random_paged_case(rng, 2, 2, 8, 4, [11, 7], [5, 7], q_heads=8)
    k_rep = case["k"][:, :, kv_of, :]
    v_rep = case["v"][:, :, kv_of, :]
    for causal, window in ((True, 0), (False, 0), (True, 3)):
        grouped, _ = A.paged_prefill(case["q"], case["k"], case["v"], case["table"],
                                     case["lens"], case["q_start"], causal, 0.3, window=window)
        mha, _ = A.paged_prefill(case["q"], k_rep, v_rep, case["table"], case["lens"],
                                 case["q_start"], causal, 0.3, window=window)
        if not np.array_equal(grouped, mha):
            return False
    dq = case["q"][case["q_start"][1:] - 1]
    grouped, _ = A.paged_decode(dq, case["k"], case["v"], case["table"], case["lens"], 0.3)
    mha, _ = A.paged_decode(dq, k_rep, v_rep, case["table"], case["lens"], 0.3)
    return bool(np.array_equal(grouped, mha))


def pin_sampled_rows_match_full(seed=13) -> bool:
    """Evaluating only some query rows (the sampled evaluation used at full sizes) gives
    those rows of the full evaluation, NaN elsewhere: chunks whose rows sit at L - q_len
    and later, rows not starting at 0, sequences left out, windows, grouped heads."""
    rng = np.random.default_rng(seed)
    case = random_paged_case(rng, 3, 2, 4, 4, [13, 9, 17], [6, 9, 5], q_heads=4)
    rows = {0: np.array([5, 1, 3]), 2: np.array([4, 0])}
    for causal, window in ((True, 0), (False, 0), (True, 4)):
        full, full_lse = A.paged_prefill(case["q"], case["k"], case["v"], case["table"],
                                         case["lens"], case["q_start"], causal, 0.35,
                                         window=window)
        part, part_lse = A.paged_prefill(case["q"], case["k"], case["v"], case["table"],
                                         case["lens"], case["q_start"], causal, 0.35,
                                         rows=rows, window=window)
        picked = np.zeros(len(case["q"]), dtype=bool)
        for b, rr in rows.items():
            picked[case["q_start"][b] + rr] = True
        if not np.all(np.isnan(part[~picked])) or not np.all(np.isfinite(part[picked])):
            return False
        # BLAS may block a different number of rows differently: equal to rounding
        if np.max(np.abs(part[picked] - full[picked])) > 1e-13:
            return False
        if np.max(np.abs(part_lse[picked] - full_lse[picked])) > 1e-13:
            return False
    return True


def pin_sampled_seqs_match_full(seed=14) -> bool:
    """Decode over some sequences gives those sequences of the full decode, NaN
    elsewhere (grouped heads, with and without a window)."""
    rng = np.random.default_rng(seed)
    case = random_paged_case(rng, 4, 2, 4, 4, [13, 9, 1, 17], [1, 1, 1, 1], q_heads=6)
    seqs = [3, 1]
    for window in (0, 5):
        full, _ = A.paged_decode(case["q"], case["k"], case["v"], case["table"], case["lens"],
                                 0.4, window=window)
        part, _ = A.paged_decode(case["q"], case["k"], case["v"], case["table"], case["lens"],
                                 0.4, seqs=seqs, window=window)
        rest = [b for b in range(4) if b not in seqs]
        if not np.all(np.isnan(part[rest])):
            return False
        if np.max(np.abs(part[seqs] - full[seqs])) > 1e-13:
            return False
    return True


ALL_PINS = [
    pin_practical_example_translation,
    pin_practical_example_gather,
    pin_page_count_example,
    pin_brute_force,
    pin_sdpa_fp64,
    pin_closed_forms,
    pin_permutation_invariance,
    pin_shared_prefix,
    pin_rows_sum_to_one,
    pin_decode_matches_last_row,
    pin_sliding_window,
    pin_kv_append_round_trip,
    pin_logical_cache_fork_isolation,
    pin_shared_prefix_pages_hold_both_sequences,
    pin_gqa_flowchart_mapping,
    pin_gqa_brute_force,
    pin_gqa_equals_replicated_heads,
    pin_sampled_rows_match_full,
    pin_sampled_seqs_match_full,
]


def run_all_pins():
    """Returns {pin name: passed?}, treating an exception inside the oracle as a failure."""
    res = {}
    for pin in ALL_PINS:
        try:
            res[pin.__name__] = bool(pin())
        except Exception:  # a broken oracle may raise anywhere
            res[pin.__name__] = False
    return res
