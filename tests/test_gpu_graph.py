"""The path under HIP graph capture.

The library enqueues kernels only: no allocation, no memset, no host
synchronisation. So a serving loop can capture the whole prompt step (block
scores -> selections -> union -> attention) or a decode call into one graph
and replay it. These tests capture each through the C ABI, with torch's graph
capture on a side stream. They replay the graph several times, with new inputs
copied into the captured tensors in between, together with the program's own
eager work and synchronisations. Every replay is checked bit for bit against
the eager calls on the same inputs, and the last replay also against the
oracle. The oracle's definitions follow page #2808 "sycl: prompt attention over
8-query selection unions on XMX", section Summary.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_selection_amd as sa
from oracle import selection
import synth
from gpu_helpers import assert_close

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _static_problem(n_ctx, n_q, n_kv, seed):
    d = synth.small_random(seed, n_ctx=n_ctx, n_q=n_q, n_kv=n_kv, nonresident_frac=0.1)
    dev = {k: torch.from_numpy(np.ascontiguousarray(d[k])).cuda()
           for k in ("q", "k_pool", "v_pool", "k_scale", "v_scale", "page_table")}
    return d, dev


def test_prompt_step_replays_match_eager_calls():
    n_ctx, n_q, n_kv = 5000, 45, 2
    first = n_ctx - n_q
    d, dev = _static_problem(n_ctx, n_q, n_kv, seed=71)
    dims = sa.make_dims(n_ctx, n_q, n_kv, d["k_pool"].shape[0], sel_cap=sa.SEL_MAX)
    n_blocks = -(-n_ctx // 64)
    g = -(-n_q // 8)
    ucap = 8 * sa.SEL_MAX
    scale = float(d["softmax_scale"])

    def buffers():
        return dict(sel=torch.empty((n_q, sa.SEL_MAX), dtype=torch.int32, device="cuda"),
                    sel_len=torch.empty(n_q, dtype=torch.int32, device="cuda"),
                    cells=torch.empty((g, ucap), dtype=torch.int32, device="cuda"),
                    mask=torch.empty((g, ucap), dtype=torch.uint8, device="cuda"),
                    rows=torch.empty((g, ucap), dtype=torch.int32, device="cuda"),
                    length=torch.empty(g, dtype=torch.int32, device="cuda"),
                    out=torch.empty_like(dev["q"]),
                    status=sa.new_status("cuda"))

    scores = torch.empty((n_q, n_blocks), dtype=torch.float32, device="cuda")

    def step(b, stream):
        sa.sel_attn_select_blocks(dims, first, scores, b["sel"], b["sel_len"], stream)
        sa.sel_attn_build_union(dims, b["sel"], b["sel_len"], dev["page_table"], b["cells"],
                                b["mask"], b["rows"], b["length"], b["status"], stream)
        sa.sel_attn_prefill(dims, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                            dev["v_scale"], b["rows"], b["mask"], b["length"], scale, b["out"],
                            b["status"], stream)

    cap_b, eager_b = buffers(), buffers()
    scores.copy_(torch.from_numpy(synth.block_scores(n_q, n_ctx, 0.9, seed=0)))
    step(eager_b, torch.cuda.current_stream())   # host-side caches filled before capture
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        step(cap_b, torch.cuda.current_stream())
    torch.cuda.synchronize()

    rng = np.random.default_rng(5)
    for r in range(REPLAYS):
        # new inputs copied into the captured tensors, the outputs poisoned
        host_scores = synth.block_scores(n_q, n_ctx, 0.5 + 0.2 * r, seed=100 + r)
        host_q = rng.standard_normal(tuple(dev["q"].shape), dtype=np.float32)
        scores.copy_(torch.from_numpy(host_scores))
        dev["q"].copy_(torch.from_numpy(host_q))
        for key in ("sel", "sel_len", "cells", "rows", "length"):
            cap_b[key].fill_(-7)
        cap_b["mask"].fill_(0xA5)
        cap_b["out"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(eager_b, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert sa.status_value(cap_b["status"]) == 0 and sa.status_value(eager_b["status"]) == 0
        for key in ("sel_len", "length", "out"):
            assert torch.equal(cap_b[key], eager_b[key]), "replay %d: %s differs" % (r, key)
        sl = cap_b["sel_len"].cpu().numpy()
        ln = cap_b["length"].cpu().numpy()
        for j in range(n_q):
            assert torch.equal(cap_b["sel"][j, :sl[j]], eager_b["sel"][j, :sl[j]])
        for gi in range(g):
            for key in ("cells", "mask", "rows"):
                assert torch.equal(cap_b[key][gi, :ln[gi]], eager_b[key][gi, :ln[gi]])

    # the last replay against the oracle (selections taken from the graph's own output)
    prob = dict(d)
    prob["q"] = dev["q"].cpu().numpy()
    prob["sel"] = cap_b["sel"].cpu().numpy()
    prob["sel_len"] = cap_b["sel_len"].cpu().numpy()
    ref_sel, ref_len = selection.select_blocks(host_scores, first, n_ctx)
    assert np.array_equal(prob["sel_len"], ref_len)
    for j in range(n_q):
        assert np.array_equal(prob["sel"][j, :ref_len[j]], ref_sel[j, :ref_len[j]])
    assert_close(cap_b["out"].cpu().numpy(), oracle.attention_of(prob), "graph replay")


@pytest.mark.parametrize("n_q", [1, 5])
def test_decode_replays_match_eager_calls(n_q):
    n_ctx, n_kv = 6000, 3
    d, dev = _static_problem(n_ctx, n_q, n_kv, seed=90 + n_q)
    dims = sa.make_dims(n_ctx, n_q, n_kv, d["k_pool"].shape[0], sel_cap=d["sel"].shape[1])
    ws_bytes = sa.sel_attn_decode_workspace_bytes(dims)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    sel = torch.from_numpy(d["sel"]).cuda()
    sel_len = torch.from_numpy(d["sel_len"]).cuda()
    scale = float(d["softmax_scale"])
    out_cap, out_eager = torch.empty_like(dev["q"]), torch.empty_like(dev["q"])
    st_cap, st_eager = sa.new_status("cuda"), sa.new_status("cuda")

    def call(out, status, stream):
        sa.sel_attn_decode(dims, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                           dev["v_scale"], dev["page_table"], sel, sel_len, scale, out, ws,
                           ws_bytes, status, stream)

    call(out_eager, st_eager, torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        call(out_cap, st_cap, torch.cuda.current_stream())
    torch.cuda.synchronize()

    rng = np.random.default_rng(11)
    for r in range(REPLAYS):
        dev["q"].copy_(torch.from_numpy(rng.standard_normal(tuple(dev["q"].shape),
                                                            dtype=np.float32)))
        out_cap.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        call(out_eager, st_eager, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert sa.status_value(st_cap) == 0 and sa.status_value(st_eager) == 0
        assert torch.equal(out_cap, out_eager), "replay %d differs" % r
    prob = dict(d)
    prob["q"] = dev["q"].cpu().numpy()
    assert_close(out_cap.cpu().numpy(), oracle.attention_of(prob), "decode graph replay")
