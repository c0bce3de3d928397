"""Plants plausible mistakes in the oracle (on the CPU, one at a time) and checks
that at least one pin catches each: evidence that the pins constrain every step
of the oracle, not just that it agrees with itself."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import logical_cache as LC
from tests import oracle_pins as P


def _swap_quotient_remainder(row, t, ps):
    return t % ps, t // ps, int(row[t % ps]) if t % ps < len(row) else -1


def _ignore_table(row, t, ps):
    return t // ps, t % ps, t // ps


def _offset_off_by_one(row, t, ps):
    return t // ps, (t + 1) % ps, int(row[t // ps])


def _window_off_by_one(positions, L, causal, window=0):
    mask = _ORIG["visible_mask"](positions, L, causal)
    if window:
        keys = np.arange(L)
        mask &= keys[None, :] >= np.asarray(positions)[:, None] - window
    return mask


def _causal_strict(positions, L, causal, window=0):
    keys = np.arange(L)
    if not causal:
        return np.ones((len(positions), L), dtype=bool)
    return keys[None, :] < np.asarray(positions)[:, None]


def _causal_top_left(positions, L, causal, window=0):
    keys = np.arange(L)
    if not causal:
        return np.ones((len(positions), L), dtype=bool)
    pos = np.asarray(positions)
    # forgets the L - q_len shift: row index instead of absolute position
    return keys[None, :] <= (pos - pos.min())[:, None]


def _no_scale(q, keys, scale):
    return q @ keys.T


def _scale_squared(q, keys, scale):
    return scale * scale * (q @ keys.T)


def _mask_after_softmax(s, mask):
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    p = np.where(mask, p, 0.0)
    return p, m[:, 0]


def _softmax_sign_flip(s, mask):
    return A.softmax_rows.__wrapped__(-s, mask) if hasattr(A.softmax_rows, "__wrapped__") else \
        _ORIG["softmax_rows"](-s, mask)


def _values_from_keys_layout(p, values):
    # transposed operand: contracts over the wrong axis of a square-ish block
    return p @ values[::-1]


def _wrong_bf16_shift(bits):
    bits = np.asarray(bits)
    return (bits.astype(np.uint32) << 15).view(np.float32).astype(np.float64)


def _fork_aliases_parent(self, parent, child, num_tokens):
    # shares the parent's lists instead of starting new ones: no copy on write
    self._k[child] = self._k[parent]
    self._v[child] = self._v[parent]


def _fork_drops_last_row(self, parent, child, num_tokens):
    _ORIG_FORK(self, parent, child, max(0, num_tokens - 1))


def _copy_pages_reversed(k_pool_bits, v_pool_bits, src_pages, dst_pages):
    return _ORIG_COPY(k_pool_bits, v_pool_bits, dst_pages, src_pages)


def _append_skips_v(k_pool_bits, v_pool_bits, block_table, seq_ids, positions, k_new, v_new):
    k, _ = _ORIG["kv_append"](k_pool_bits, v_pool_bits, block_table, seq_ids, positions,
                              k_new, v_new)
    return k, np.array(v_pool_bits, copy=True)


def _heads_interleaved(h, num_q_heads, num_kv_heads):
    # query heads dealt round-robin over the K/V heads instead of in adjacent groups
    return h % num_kv_heads


def _heads_divided_by_kv_count(h, num_q_heads, num_kv_heads):
    # divides by the K/V head count instead of the group size
    return h // num_kv_heads


def _positions_from_sample_index(seq_len, q_len, local_rows):
    # numbers the sampled rows 0, 1, ... instead of using their row indices
    return int(seq_len) - int(q_len) + np.arange(len(local_rows))


_ORIG_FORK = LC.LogicalCache.fork
_ORIG_COPY = LC.copy_pages

_ORIG = {name: getattr(A, name) for name in
         ("locate_token", "visible_mask", "scores", "softmax_rows", "weighted_values", "bf16_to_f64",
          "kv_append", "kv_head_of", "row_positions")}

MUTANTS = [
    ("locate_token", _swap_quotient_remainder),
    ("locate_token", _ignore_table),
    ("locate_token", _offset_off_by_one),
    ("visible_mask", _causal_strict),
    ("visible_mask", _causal_top_left),
    ("visible_mask", _window_off_by_one),
    ("scores", _no_scale),
    ("scores", _scale_squared),
    ("softmax_rows", _mask_after_softmax),
    ("softmax_rows", _softmax_sign_flip),
    ("weighted_values", _values_from_keys_layout),
    ("bf16_to_f64", _wrong_bf16_shift),
    ("kv_append", _append_skips_v),
    ("LogicalCache.fork", _fork_aliases_parent),
    ("LogicalCache.fork", _fork_drops_last_row),
    ("copy_pages", _copy_pages_reversed),
    ("kv_head_of", _heads_interleaved),
    ("kv_head_of", _heads_divided_by_kv_count),
    ("row_positions", _positions_from_sample_index),
]


@pytest.mark.parametrize("name,fn", MUTANTS, ids=[f"{n}:{f.__name__}" for n, f in MUTANTS])
def test_some_pin_catches_mutant(monkeypatch, name, fn):
    if name == "LogicalCache.fork":
        monkeypatch.setattr(LC.LogicalCache, "fork", fn)
    elif name == "copy_pages":
        monkeypatch.setattr(LC, name, fn)
    else:
        monkeypatch.setattr(A, name, fn)
    results = P.run_all_pins()
    assert not all(results.values()), f"no pin caught mutant {fn.__name__}: {results}"


def test_unmutated_oracle_passes_every_pin():
    results = P.run_all_pins()
    assert all(results.values()), results
