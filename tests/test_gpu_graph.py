"""The attention calls under HIP graph capture: every call only enqueues kernels on
the caller's stream (no allocation, no memset, no synchronisation), so a captured
decode step or prefill replays.  Each replay is compared bit for bit with the eager
result of the same inputs, with eager work and synchronisations between replays, and
the inputs are changed in place between replays to show the graph reads them anew."""
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


def _bits(t):
    return W.to_host_bits(t)


def test_decode_step_replays_from_a_graph():
    G.banner("graph capture: decode (partial + combine)")
    wl = W.build("gdec", 61, heads=4, head_dim=128, page_size=16, lens=[1, 300, 2049, 5000],
                 kind="decode", pool_slack=1.2, device="cuda", poison=True, q_heads=8)
    call = wl.calls[0]
    ws = B.decode_workspace(call.q, wl.k_pool, call.block_table)
    out_g = torch.zeros_like(call.q)
    out_e = torch.zeros_like(call.q)

    def run(out):
        B.pa_decode(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, wl.scale,
                    out, ws)

    run(out_e)                          # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(out_g)
    for rep in range(4):
        call.q.copy_(W.normal_bf16(tuple(call.q.shape), 1.0, 700 + rep, "cuda"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        run(out_e)                      # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out_g), _bits(out_e)), f"replay {rep}"
    G.compare(G.bf16_out_to_f64(out_g), G.oracle_for(wl, call),
              "graph decode, last replay")


def test_prefill_replays_from_a_graph():
    G.banner("graph capture: causal prefill")
    wl = W.build("gpre", 62, heads=2, head_dim=128, page_size=32, lens=[700, 300],
                 q_lens=[700, 129], causal=True, pool_slack=1.2, device="cuda", poison=True)
    call = wl.calls[0]
    out_g = torch.zeros_like(call.q)
    out_e = torch.zeros_like(call.q)

    def run(out):
        B.pa_prefill(call.q, wl.k_pool, wl.v_pool, call.block_table, call.seq_lens, True,
                     wl.scale, out, call.q_start, call.max_q_len)

    run(out_e)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(out_g)
    for rep in range(3):
        call.q.copy_(W.normal_bf16(tuple(call.q.shape), 1.0, 800 + rep, "cuda"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        run(out_e)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out_g), _bits(out_e)), f"replay {rep}"
    G.compare(G.bf16_out_to_f64(out_g), G.oracle_for(wl, call), "graph prefill, last replay")
