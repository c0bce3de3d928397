"""pa_decode_noalloc, the decode entry point that allocates nothing (its split partials
live in the library's static per-GPU array), against pa_decode with a caller
workspace: bit-identical outputs, and within the oracle bar, on two calls in a row,
the second smaller than the first (the array keeps the first call's partials)."""
import numpy as np
import pytest
import torch

from exact_tiled_attention_pa_amd import binding as B
from exact_tiled_attention_pa_amd import workloads as W
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    G.gpu_or_skip()


def _check_against_pa_decode(wl, seqs, what):
    call = wl.calls[0]
    want = G.run_call(wl, call)                     # pa_decode, torch-allocated workspace
    got = torch.full_like(call.q, float("nan"))
    B.pa_decode_noalloc(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens,
                        wl.scale, got)
    torch.cuda.synchronize()
    assert torch.equal(got, want), f"{what}: pa_decode_noalloc differs from pa_decode"
    G.compare(G.bf16_out_to_f64(got), G.oracle_for(wl, call, seqs=seqs), what)


def test_noalloc_decode_twice_second_smaller():
    G.banner("pa_decode_noalloc: decode_64 at full size, then a smaller grouped-head batch")
    big = W.decode_64(device="cuda", poison=True)
    lens = big.calls[0].seq_lens_host
    _check_against_pa_decode(big, sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 63}),
                             "noalloc decode_64")
    del big
    small = W.build("noalloc_small", 17, heads=2, head_dim=128, page_size=16,
                    lens=[1, 300, 2049, 17], kind="decode", pool_slack=1.3, device="cuda",
                    poison=True, q_heads=8)
    _check_against_pa_decode(small, [0, 1, 2, 3], "noalloc small grouped")


def test_noalloc_decode_refuses_requests_above_its_array():
    """128 sequences x 32 heads over up to 32768 tokens need 272 MB of partials: refused
    with PA_ERR_WORKSPACE before anything is enqueued; the output is untouched."""
    G.banner("pa_decode_noalloc: request above the static array is refused")
    q = torch.zeros(128, 32, 128, dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros(4, 16, 32, 128, dtype=torch.bfloat16, device="cuda")
    table = torch.zeros(128, 2048, dtype=torch.int32, device="cuda")
    lens = torch.ones(128, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 3.0)
    with pytest.raises(B.PagedAttnError) as e:
        B.pa_decode_noalloc(q, pool, pool, table, lens, 0.1, out)
    assert e.value.status == B.PA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
