"""The opt-in host-side check of the device-array contract (CPU only).

Bad block tables, lengths and chunk offsets are built on the host and must be
refused with a message naming the sequence and page; the tensor-level wrappers
must refuse them before anything reaches a device.  Nothing here runs a kernel.
"""
import numpy as np
import pytest
import torch

from exact_tiled_attention_pa_amd import binding as B
from exact_tiled_attention_pa_amd import workloads as W


def _good():
    wl = W.build("contract", 3, heads=2, head_dim=64, page_size=16, lens=[40, 7, 300],
                 q_lens=[40, 3, 100], kind="prefill", pool_slack=1.3, device="cpu")
    return wl, wl.calls[0]


def test_valid_arrays_pass():
    wl, call = _good()
    assert B.contract_violations(call.block_table_host, call.seq_lens_host, wl.num_pages,
                                 wl.page_size, q_start=call.q_start_host,
                                 max_q_len=call.max_q_len, total_q=call.q.shape[0]) == []
    # the worked example of the pages: 600 tokens over [5, 1, 9] in a pool of 12 pages of 256
    assert B.contract_violations([[5, 1, 9]], [600], 12, 256) == []


@pytest.mark.parametrize("mutate,needle", [
    (lambda bt, L, qs: bt.__setitem__((2, 3), -1), "sequence 2: logical page 3"),
    (lambda bt, L, qs: bt.__setitem__((0, 1), 10_000), "physical page 10000"),
    (lambda bt, L, qs: L.__setitem__(1, -1), "sequence 1: length -1"),
    (lambda bt, L, qs: L.__setitem__(0, 10_000), "sequence 0: length 10000"),
    (lambda bt, L, qs: L.__setitem__(1, 2), "3 query rows over only 2 keys"),
    (lambda bt, L, qs: qs.__setitem__(1, 50), "q_start decreases"),
    (lambda bt, L, qs: qs.__setitem__(0, 1), "q_start[0] is 1"),
    (lambda bt, L, qs: qs.__setitem__(3, 10_000), "exceeds the 143 query rows"),
])
def test_broken_arrays_are_named(mutate, needle):
    wl, call = _good()
    bt = call.block_table_host.copy()
    L = call.seq_lens_host.copy()
    qs = call.q_start_host.copy()
    mutate(bt, L, qs)
    bad = B.contract_violations(bt, L, wl.num_pages, wl.page_size, q_start=qs,
                                max_q_len=call.max_q_len, total_q=call.q.shape[0])
    assert any(needle in m for m in bad), bad


def test_entries_past_the_last_page_are_not_checked():
    """Entries beyond ceil(L / page_size) are never read: any value is allowed there."""
    bt = np.array([[3, -7, 99999]], dtype=np.int32)
    assert B.contract_violations(bt, [16], 4, 16) == []
    assert B.contract_violations(bt, [17], 4, 16) != []


def test_wrappers_refuse_before_any_device_check(monkeypatch):
    """With the check on, pa_prefill and pa_decode raise ContractError on a bad table
    before the device checks; a good table passes the contract and then fails the
    device check (these are CPU tensors), so nothing is ever launched."""
    wl, call = _good()
    out = torch.empty_like(call.q)
    bad_table = call.block_table.clone()
    bad_table[1, 0] = wl.num_pages
    monkeypatch.setattr(B, "_check_contract", True)
    with pytest.raises(B.ContractError, match="sequence 1: logical page 0"):
        B.pa_prefill(call.q, wl.k_pool, wl.v_pool, bad_table, call.seq_lens, True, wl.scale,
                     out, call.q_start, call.max_q_len)
    with pytest.raises(ValueError, match="must be on a GPU") as e:
        B.pa_prefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, True,
                     wl.scale, out, call.q_start, call.max_q_len)
    assert not isinstance(e.value, B.ContractError)
    dq = call.q[:3].contiguous()
    ws = torch.empty(16, dtype=torch.uint8)
    with pytest.raises(B.ContractError, match="physical page"):
        B.pa_decode(dq, wl.k_pool, wl.v_pool, bad_table, call.seq_lens, wl.scale,
                    torch.empty_like(dq), ws)
    # off by default: the same bad table goes straight to the device checks
    monkeypatch.setattr(B, "_check_contract", False)
    with pytest.raises(ValueError, match="must be on a GPU"):
        B.pa_prefill(call.q, wl.k_pool, wl.v_pool, bad_table, call.seq_lens, True, wl.scale,
                     out, call.q_start, call.max_q_len)
