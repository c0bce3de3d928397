"""The oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import online_softmax as OS
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    assert pin()


def test_oracle_rejects_out_of_pool_page():
    table = [0, 5]
    pool = np.zeros((2, 4, 1, 2), dtype=np.uint16)
    with pytest.raises(IndexError):
        A.gather_sequence(pool, table, 6, 4)


def test_oracle_rejects_row_without_keys():
    with pytest.raises(ValueError):
        A.softmax_rows(np.zeros((1, 3)), np.zeros((1, 3), dtype=bool))


def test_oracle_never_reads_unused_slots():
    """Every unread slot is NaN in random_paged_case; outputs stay finite."""
    rng = np.random.default_rng(11)
    case = P.random_paged_case(rng, 2, 2, 8, 4, [5, 10], [5, 3])
    out, lse = A.paged_prefill(case["q"], case["k"], case["v"], case["table"], case["lens"],
                               case["q_start"], True, 0.3)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


@pytest.mark.parametrize("tile", [1, 5, 16, 64])
def test_online_softmax_recurrence_reaches_definition(tile):
    """The unnormalised tiled recurrence (reading of the page's update) equals the
    plain definition to fp64 rounding at any tile size, causal or not."""
    rng = np.random.default_rng(tile)
    r, L, d = 11, 37, 8
    q = rng.normal(size=(r, d))
    k = rng.normal(size=(L, d)) * 2
    v = rng.normal(size=(L, d))
    for causal in (False, True):
        pos = np.arange(L - r, L)
        mask = A.visible_mask(pos, L, causal)
        p, _ = A.softmax_rows(A.scores(q, k, 0.5), mask)
        want = p @ v
        got, _, _ = OS.tiled_attention_row_block(q, k, v, mask, 0.5, tile)
        assert np.max(np.abs(got - want)) < 1e-12


def test_printed_update_is_not_the_softmax():
    """The output update exactly as printed (old output scaled by l_old/l_new as well,
    new tile not divided, then a final division by l) misses the definition by far
    more than rounding: evidence that it is garbled and must be read as above."""
    rng = np.random.default_rng(7)
    r, L, d = 4, 37, 8
    q, k, v = rng.normal(size=(r, d)), rng.normal(size=(L, d)), rng.normal(size=(L, d))
    mask = np.ones((r, L), dtype=bool)
    p, _ = A.softmax_rows(A.scores(q, k, 1.0), mask)
    got, _, _ = OS.tiled_attention_row_block(q, k, v, mask, 1.0, 5, printed_update=True)
    assert np.max(np.abs(got - p @ v)) > 1e-3


@pytest.mark.parametrize("split", [1, 7, 16, 512])
def test_split_merge_reaches_definition(split):
    rng = np.random.default_rng(split)
    L, d = 300, 16
    q, k, v = rng.normal(size=d), rng.normal(size=(L, d)) * 3, rng.normal(size=(L, d))
    p, lse = A.softmax_rows(A.scores(q[None, :], k, 0.25), np.ones((1, L), dtype=bool))
    got, got_lse = OS.merge_partials(OS.split_partials(q, k, v, 0.25, split))
    assert np.max(np.abs(got - (p @ v)[0])) < 1e-12
    assert abs(got_lse - lse[0]) < 1e-12
