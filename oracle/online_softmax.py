"""fp64 model of the tiled online-softmax recurrence and of the split/merge combine.

TEST INFRASTRUCTURE ONLY (same rule as oracle.attention: never on the product path).

This is not the reference for parity; oracle.attention is.  It exists so that a
test can show, in exact-ish fp64 arithmetic, that the tiled algorithm the HIP
kernels run reaches the plain definition, and that the update as printed on the
page does not.

Source: "Flash Attention: Fast, Memory-Efficient Attention for LLMs", section
"Flash Attention: IO-Aware Tiling", subsection "The Algorithm" (the per-tile
update of the running max m, running sum l and output O, followed by the final
division by l).

Reading taken: the printed output update multiplies the old output by
(l_old / l_new) * exp(m_old - m_new) but adds the new tile's P~ V without any
division, and then divides by l once more at the end.  That mixes the
normalised and the unnormalised forms of the recurrence and does not give the
softmax result.  The consistent form that matches the page's own final step
("divide by l at the end") and the FlashAttention-2 remark on the same page
(fewer rescaling operations) is the unnormalised one:

    m_new = max(m_old, rowmax(S_tile))
    P~    = exp(S_tile - m_new)
    l_new = exp(m_old - m_new) * l_old + rowsum(P~)
    O_new = exp(m_old - m_new) * O_old + P~ V_tile
    O     = O_final / l_final

The split/merge used for decode applies the same algebra across independent
partial results (m_s, l_s, O_s):

    M = max_s m_s,   w_s = exp(m_s - M),   l = sum_s w_s l_s,   O = sum_s w_s O_s / l
"""
from __future__ import annotations

import numpy as np


def tiled_attention_row_block(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                              mask: np.ndarray, scale: float, tile: int,
                              printed_update: bool = False):
    """One head, rows q [r, d] over keys/values [L, d], keys visited in tiles of `tile`.

    mask [r, L] marks visible keys.  Returns (O [r, d], m [r], l [r]).
    With printed_update=True the output update is taken literally as printed.
    """
    r = q.shape[0]
    seq_len = keys.shape[0]
    m = np.full(r, -np.inf)
    l = np.zeros(r)
    o = np.zeros((r, values.shape[1]))
    for j0 in range(0, seq_len, tile):
        j1 = min(seq_len, j0 + tile)
        s = scale * (q @ keys[j0:j1].T)
        s = np.where(mask[:, j0:j1], s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        # rows that have seen no visible key yet keep m = -inf; guard their exps
        safe = np.isfinite(m_new)
        m_ref = np.where(safe, m_new, 0.0)
        p = np.where(safe[:, None], np.exp(s - m_ref[:, None]), 0.0)
        alpha = np.where(safe, np.exp(np.where(np.isfinite(m), m, -np.inf) - m_ref), 0.0)
        alpha = np.where(np.isfinite(m), alpha, 0.0)
        l_new = alpha * l + p.sum(axis=1)
        if printed_update:
            ratio = np.where(l_new > 0, l / np.where(l_new > 0, l_new, 1.0), 0.0)
            o = (ratio * alpha)[:, None] * o + p @ values[j0:j1]
        else:
            o = alpha[:, None] * o + p @ values[j0:j1]
        m, l = m_new, l_new
    return o / l[:, None], m, l


def split_partials(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float,
                   split: int):
    """Partial (m, l, O_unnormalised) of one decode row over key ranges of `split` keys."""
    parts = []
    for j0 in range(0, keys.shape[0], split):
        j1 = min(keys.shape[0], j0 + split)
        s = scale * (keys[j0:j1] @ q)
        m = s.max()
        p = np.exp(s - m)
        parts.append((m, p.sum(), p @ values[j0:j1]))
    return parts


def merge_partials(parts):
    """Combine partial (m, l, O_unnormalised) triples into the normalised output."""
    big_m = max(m for m, _, _ in parts)
    weights = [np.exp(m - big_m) for m, _, _ in parts]
    total = sum(w * l for w, (_, l, _) in zip(weights, parts))
    acc = sum(w * o for w, (_, _, o) in zip(weights, parts))
    return acc / total, big_m + np.log(total)
