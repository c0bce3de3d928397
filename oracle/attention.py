"""CPU fp64 oracle: exact attention over a paged KV cache, written as its plain definition.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check of the entry module and the
CPU-baseline leg of the bench use it.  It shares no code with the HIP library.

What it computes (for sequence b, head h, query row i of that sequence):

    K_b[t] = k_pool[ block_table[b, t // page_size], t % page_size ]
    V_b[t] = v_pool[ block_table[b, t // page_size], t % page_size ]
    s_it   = scale * < Q[b, i, h, :], K_b[t, h, :] >
    O[b, i, h, :] = sum_{t visible} softmax_t(s_it) * V_b[t, h, :]

Sources, by page title and section:
  * "FlashAttention and PagedAttention: Two Fixes for Two Different
    Bottlenecks", section "Why attention is costly": the attention formula
    softmax(Q K^T / sqrt(d)) V.
  * "Flash Attention: Fast, Memory-Efficient Attention for LLMs", section
    "Standard Attention: The Memory Problem" (flowchart S = Q K^T,
    P = softmax(S), O = P V): the three-step unfused definition, which this
    oracle follows literally, materialising complete rows of S and P.
  * "What is Paged FlashAttention?", sections "How does it work?" and
    "Practical example": the block-table translation logical = pos // page_size,
    offset = pos % page_size, physical = block_table[logical].
  * Same page, "Does it change the attention result or complexity?", and the
    first page's "How it works": the tiled method reaches exactly this result up
    to rounding, so this plain definition is the reference.

Readings where the pages leave a step open:
  * Causal alignment for a chunk of q_len rows over L keys is bottom-right:
    query row i sits at absolute position L - q_len + i and sees keys t <= that
    position (the pages only name a causal flag that skips future tokens).
  * A decode query is the newest token, already appended to the cache, and
    sees all L keys of its sequence (KV-cache flowchart, "Append new K_t, V_t").
  * The scale is the fp32 value handed to the kernel, widened exactly to fp64.
  * Sliding window ("What do FlashAttention and PagedAttention actually
    optimize?", section "Sort techniques into the two bins": attention over only
    the previous w tokens): with window w >= 1 a query at position p sees the w
    keys p - w + 1 .. p (its own key included); window 0 means no window.  Only
    meaningful together with causal attention.
  * Grouped heads ("Flash Attention: Fast, Memory-Efficient Attention for LLMs",
    section "Attention Variants: MHA, GQA, MQA"): with H_q query heads over H_kv
    K/V heads, consecutive blocks of g = H_q / H_kv query heads share one K/V
    head (the page's flowchart puts query heads 1-4 in K/V group 1 and 5-8 in
    group 2); zero-based, query head h reads K/V head h // g.  H_kv = H_q is
    multi-head attention, H_kv = 1 multi-query attention.  The K/V head count is
    the pools' head dimension, the query head count that of q.

Inputs are raw bf16 bit patterns (uint16 arrays).  Decoding them to fp64 is
exact.  The output stays in fp64; nothing here rounds to bf16.

Parity status: pinned (see tests/test_oracle_pins.py for each pin), including the
grouped-head mapping and the sampled evaluation (rows= / seqs=).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

# rows of S materialised at once; every row is always complete over its keys
ROW_BLOCK = 1024


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (upper half of a binary32) to fp64."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as uint16 bit patterns")
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pages_needed(seq_len: int, page_size: int) -> int:
    """Number of pages a sequence of seq_len tokens occupies: ceil(L / page_size).

    "Flash Attention: Fast, Memory-Efficient Attention for LLMs", section
    "PagedAttention (vLLM)", flowchart: a 200-token request in 16-token pages
    fills 13 pages, the last one partly.
    """
    return -(-int(seq_len) // int(page_size))


def locate_token(block_table_row: Sequence[int], t: int, page_size: int):
    """Block-table translation of token position t.

    "What is Paged FlashAttention?", section "Practical example": logical page
    is the quotient of the position by the page size, the offset is the
    remainder, and the physical page is the table entry at the logical page.
    Returns (logical, offset, physical).
    """
    logical = t // page_size
    offset = t % page_size
    physical = int(block_table_row[logical])
    return logical, offset, physical


def gather_sequence(pool_bits: np.ndarray, block_table_row: Sequence[int],
                    seq_len: int, page_size: int) -> np.ndarray:
    """Reads the seq_len tokens of one sequence out of the paged pool, token by token.

    pool_bits: uint16 [num_pages, page_size, heads, d].  Returns fp64 [L, heads, d].
    Only the slots the block table names for tokens 0..L-1 are read; tail slots
    and unused pages are never touched.
    """
    num_pages = pool_bits.shape[0]
    if pool_bits.shape[1] != page_size:
        raise ValueError("pool page dimension does not match page_size")
    rows = np.empty((seq_len,) + tuple(pool_bits.shape[2:]), dtype=np.uint16)
    for t in range(seq_len):
        _, offset, physical = locate_token(block_table_row, t, page_size)
        if not 0 <= physical < num_pages:
            raise IndexError(f"token {t}: physical page {physical} outside pool of {num_pages}")
        rows[t] = pool_bits[physical, offset]
    return bf16_to_f64(rows)


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """K/V head read by query head h (zero-based) when num_q_heads query heads share
    num_kv_heads K/V heads in consecutive equal groups.

    "Flash Attention: Fast, Memory-Efficient Attention for LLMs", section "Attention
    Variants: MHA, GQA, MQA": 8 query heads in 2 K/V groups, heads 1-4 in the first
    and 5-8 in the second, so a group is a run of g = num_q_heads / num_kv_heads
    adjacent query heads.
    """
    if num_kv_heads < 1 or num_q_heads % num_kv_heads:
        raise ValueError(f"{num_q_heads} query heads do not split into {num_kv_heads} "
                         "equal K/V groups")
    group = num_q_heads // num_kv_heads
    return h // group


def row_positions(seq_len: int, q_len: int, local_rows) -> np.ndarray:
    """Absolute positions of local query rows of a q_len-row chunk over seq_len keys.

    The chunk is the last q_len tokens of the sequence (bottom-right causal
    alignment; see the module docstring), so local row i sits at seq_len - q_len + i.
    """
    return int(seq_len) - int(q_len) + np.asarray(local_rows, dtype=np.int64)


def visible_mask(positions: np.ndarray, seq_len: int, causal: bool,
                 window: int = 0) -> np.ndarray:
    """Boolean [rows, L]: key t is visible to a query at absolute position p.

    Non-causal: every key 0 <= t < L.  Causal: keys t <= p (bottom-right
    alignment; see the module docstring).  Window w > 0 (causal only): also
    t >= p - w + 1.
    """
    keys = np.arange(seq_len)
    if not causal:
        if window:
            raise ValueError("a sliding window needs causal attention")
        return np.ones((len(positions), seq_len), dtype=bool)
    pos = np.asarray(positions)[:, None]
    mask = keys[None, :] <= pos
    if window:
        mask &= keys[None, :] >= pos - window + 1
    return mask


def scores(q_rows: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T for one head: q_rows [r, d], keys [L, d] -> [r, L]."""
    return scale * (q_rows @ keys.T)


def softmax_rows(s: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Row softmax over the visible keys, two passes (max, then exp and sum).

    Masked entries get probability exactly 0.  Each row must have at least one
    visible key.
    """
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row has no visible key")
    e = np.exp(s - m)
    total = e.sum(axis=1, keepdims=True)
    p = e / total
    if np.max(np.abs(p.sum(axis=1) - 1.0)) > 1e-12:
        raise AssertionError("softmax rows do not sum to 1")
    return p, m[:, 0] + np.log(total[:, 0])


def weighted_values(p: np.ndarray, values: np.ndarray) -> np.ndarray:
    """O = P V for one head: p [r, L], values [L, d] -> [r, d]."""
    return p @ values


def attend(q_rows: np.ndarray, k_seq: np.ndarray, v_seq: np.ndarray,
           positions: np.ndarray, causal: bool, scale: float, window: int = 0):
    """Attention of some query rows of one sequence over its gathered keys.

    q_rows [r, H_q, d] fp64, k_seq / v_seq [L, H_kv, d] fp64 (H_q a multiple of
    H_kv; query head h reads K/V head kv_head_of(h, H_q, H_kv)), positions [r]
    absolute.  Returns (O [r, H_q, d] fp64, lse [r, H_q] fp64 natural-log sum of exp).
    """
    r, heads, d = q_rows.shape
    seq_len, kv_heads = k_seq.shape[0], k_seq.shape[1]
    out = np.empty((r, heads, d), dtype=np.float64)
    lse = np.empty((r, heads), dtype=np.float64)
    for h in range(heads):
        hk = kv_head_of(h, heads, kv_heads)
        for r0 in range(0, r, ROW_BLOCK):
            r1 = min(r, r0 + ROW_BLOCK)
            mask = visible_mask(positions[r0:r1], seq_len, causal, window)
            s = scores(q_rows[r0:r1, h, :], k_seq[:, hk, :], scale)
            p, row_lse = softmax_rows(s, mask)
            out[r0:r1, h, :] = weighted_values(p, v_seq[:, hk, :])
            lse[r0:r1, h] = row_lse
    return out, lse


def paged_prefill(q_bits, k_pool_bits, v_pool_bits, block_table, seq_lens, q_start,
                  causal: bool, scale: float, rows: Optional[dict] = None, window: int = 0):
    """Prefill (or chunked prefill) over a paged cache.

    q_bits       uint16 [total_q, H_q, d]; rows of sequence b are q_start[b]..q_start[b+1]-1
    k/v_pool_bits uint16 [num_pages, page_size, H_kv, d]; H_q a multiple of H_kv
    block_table  int [batch, max_pages_per_seq]
    seq_lens     int [batch]: L_b, the KV length including this chunk
    scale        the fp32 scale value (widened exactly)
    rows         optional {b: array of local row indices} to evaluate only some rows
    window       sliding-window length w (0: none); needs causal

    Returns (O fp64 [total_q, H_q, d] with NaN where not evaluated, lse [total_q, H_q]).
    Evaluating only some rows gives, for those rows, what the full evaluation gives:
    each row is computed from its own query, position and the sequence's keys.
    """
    q_bits = np.asarray(q_bits)
    total_q, heads, d = q_bits.shape
    page_size = k_pool_bits.shape[1]
    scale = float(np.float32(scale))
    out = np.full((total_q, heads, d), np.nan)
    lse = np.full((total_q, heads), np.nan)
    for b in range(len(seq_lens)):
        seq_len = int(seq_lens[b])
        start, stop = int(q_start[b]), int(q_start[b + 1])
        q_len = stop - start
        if q_len == 0:
            continue
        if not 1 <= q_len <= seq_len:
            raise ValueError(f"sequence {b}: need 1 <= q_len ({q_len}) <= L ({seq_len})")
        if rows is not None and b not in rows:
            continue
        local = np.arange(q_len) if rows is None else np.asarray(rows[b], dtype=np.int64)
        k_seq = gather_sequence(k_pool_bits, block_table[b], seq_len, page_size)
        v_seq = gather_sequence(v_pool_bits, block_table[b], seq_len, page_size)
        positions = row_positions(seq_len, q_len, local)
        q_rows = bf16_to_f64(q_bits[start + local])
        o, l = attend(q_rows, k_seq, v_seq, positions, causal, scale, window)
        out[start + local] = o
        lse[start + local] = l
    return out, lse


def paged_decode(q_bits, k_pool_bits, v_pool_bits, block_table, seq_lens, scale: float,
                 seqs: Optional[Sequence[int]] = None, window: int = 0):
    """Decode: one query token per sequence over all L_b cached keys (itself included),
    or over the last `window` of them when window > 0.

    q_bits uint16 [batch, H_q, d], pools [num_pages, page_size, H_kv, d].  Returns
    (O fp64 [batch, H_q, d], lse [batch, H_q]); sequences not in `seqs` are left NaN.
    """
    q_bits = np.asarray(q_bits)
    batch, heads, d = q_bits.shape
    page_size = k_pool_bits.shape[1]
    scale = float(np.float32(scale))
    out = np.full((batch, heads, d), np.nan)
    lse = np.full((batch, heads), np.nan)
    for b in (range(batch) if seqs is None else seqs):
        seq_len = int(seq_lens[b])
        if seq_len < 1:
            raise ValueError(f"sequence {b}: decode needs L >= 1")
        k_seq = gather_sequence(k_pool_bits, block_table[b], seq_len, page_size)
        v_seq = gather_sequence(v_pool_bits, block_table[b], seq_len, page_size)
        q_rows = bf16_to_f64(q_bits[b:b + 1])
        o, l = attend(q_rows, k_seq, v_seq, np.array([seq_len - 1]), window > 0, scale,
                      window)
        out[b] = o[0]
        lse[b] = l[0]
    return out, lse


def kv_append(k_pool_bits: np.ndarray, v_pool_bits: np.ndarray, block_table,
              seq_ids: Sequence[int], positions: Sequence[int],
              k_new_bits: np.ndarray, v_new_bits: np.ndarray):
    """Writes new tokens' K/V rows into the paged pools (returns new pools).

    "Flash Attention: Fast, Memory-Efficient Attention for LLMs", section "KV
    Cache": each generated token's K_t, V_t are appended to the cache.  Token i
    of sequence seq_ids[i] at absolute position positions[i] goes to the slot the
    block table names for that position ("What is Paged FlashAttention?",
    "Practical example").  k_new_bits, v_new_bits: uint16 [num_tokens, H_kv, d].
    """
    k = np.array(k_pool_bits, copy=True)
    v = np.array(v_pool_bits, copy=True)
    page_size = k.shape[1]
    for i, (b, pos) in enumerate(zip(seq_ids, positions)):
        _, offset, physical = locate_token(block_table[int(b)], int(pos), page_size)
        if not 0 <= physical < k.shape[0]:
            raise IndexError(f"token {i}: physical page {physical} outside the pool")
        k[physical, offset] = k_new_bits[i]
        v[physical, offset] = v_new_bits[i]
    return k, v


__all__ = [
    "bf16_to_f64", "pages_needed", "locate_token", "gather_sequence", "kv_head_of",
    "row_positions", "visible_mask",
    "scores", "softmax_rows", "weighted_values", "attend", "paged_prefill", "paged_decode",
    "kv_append", "ROW_BLOCK",
]
