"""Logical KV cache: what a paged cache must hold for each sequence, with no pages.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests use it.  It shares no code with the HIP
library or with its host-side page manager.

Sources, by page title and section:
  * "FlashAttention and PagedAttention: Two Fixes for Two Different
    Bottlenecks", "How it works" under PagedAttention: a sequence's cache is the
    list of its tokens' K and V rows; paging only decides where those rows live
    (fixed-size blocks found through a block table, allocated as the sequence
    grows).  Sequences with a common prompt prefix may map that prefix to the
    same physical blocks; a block is copied before one of its sharers writes a
    different token into it (copy on write), so no sequence ever sees another
    sequence's later tokens.
  * "Flash Attention: Fast, Memory-Efficient Attention for LLMs", "KV Cache":
    every new token's K_t and V_t are appended to its sequence's cache.

So the plain definition of the cache's contents is a per-sequence list of rows:
  add(s)              s starts empty
  fork(p, c, n)       c starts as the first n rows of p (a shared prefix)
  append(s, K, V)     s's list grows by the given rows, in order
  free(s)             s's list is gone
A paged implementation is correct exactly when, after every operation, gathering
each live sequence through its block table yields these lists bit for bit.

Rows are raw bf16 bit patterns (uint16 arrays of shape [heads, head_dim]).

Parity status: pinned (tests/oracle_pins.py: prefix fork, isolation of a fork's
appends from its parent, lengths; the shared-prefix block tables of the first
page's example).
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np


class LogicalCache:
    def __init__(self, heads: int, head_dim: int):
        self.heads = int(heads)
        self.head_dim = int(head_dim)
        self._k: Dict[int, List[np.ndarray]] = {}
        self._v: Dict[int, List[np.ndarray]] = {}

    def live(self) -> List[int]:
        return sorted(self._k)

    def add(self, seq: int) -> None:
        if seq in self._k:
            raise KeyError(f"sequence {seq} already exists")
        self._k[seq] = []
        self._v[seq] = []

    def fork(self, parent: int, child: int, num_tokens: int) -> None:
        if child in self._k:
            raise KeyError(f"sequence {child} already exists")
        if not 0 <= num_tokens <= len(self._k[parent]):
            raise ValueError(f"cannot share {num_tokens} of {len(self._k[parent])} tokens")
        # new lists holding the same row values: later appends to either list
        # leave the other unchanged
        self._k[child] = [r.copy() for r in self._k[parent][:num_tokens]]
        self._v[child] = [r.copy() for r in self._v[parent][:num_tokens]]

    def append(self, seq: int, k_rows: np.ndarray, v_rows: np.ndarray) -> None:
        k_rows = np.asarray(k_rows, dtype=np.uint16)
        v_rows = np.asarray(v_rows, dtype=np.uint16)
        shape = (self.heads, self.head_dim)
        if k_rows.shape[1:] != shape or v_rows.shape != k_rows.shape:
            raise ValueError(f"rows must be [n, {self.heads}, {self.head_dim}]")
        self._k[seq].extend(r.copy() for r in k_rows)
        self._v[seq].extend(r.copy() for r in v_rows)

    def free(self, seq: int) -> None:
        del self._k[seq]
        del self._v[seq]

    def length(self, seq: int) -> int:
        return len(self._k[seq])

    def rows(self, seq: int) -> Tuple[np.ndarray, np.ndarray]:
        """(K, V) of the sequence as uint16 [length, heads, head_dim]."""
        empty = np.zeros((0, self.heads, self.head_dim), dtype=np.uint16)
        k = np.stack(self._k[seq]) if self._k[seq] else empty
        v = np.stack(self._v[seq]) if self._v[seq] else empty.copy()
        return k, v


def copy_pages(k_pool_bits: np.ndarray, v_pool_bits: np.ndarray, src_pages, dst_pages):
    """Returns pools in which page dst_pages[i] holds what page src_pages[i] held
    (every slot, K and V): the copy step of copy on write, same page and section as
    above.  Sources are read from the pools as given, before any copy lands."""
    k = np.array(k_pool_bits, copy=True)
    v = np.array(v_pool_bits, copy=True)
    for s, d in zip(src_pages, dst_pages):
        k[int(d)] = k_pool_bits[int(s)]
        v[int(d)] = v_pool_bits[int(s)]
    return k, v


__all__ = ["LogicalCache", "copy_pages"]
