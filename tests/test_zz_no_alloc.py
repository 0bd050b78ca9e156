"""The allocation-free decode call (sel_attn_decode_noalloc) against the decode
call with a caller workspace (sel_attn_decode), through the C ABI.

Both run the same kernels on the same inputs, so their outputs must agree bit
for bit; both must also meet the oracle gate (max abs <= 8e-3, mean abs
<= 1e-3 against FP64). Calls follow each other on one GPU, the second with a
smaller input, so the second finds the static scratch as the first left it.

Page cited: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
section Summary: every position attends to exactly its own selected cells.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    name = torch.cuda.get_device_properties(0).gcnArchName
    if not name.startswith("gfx950"):
        pytest.skip("not gfx950: %s" % name)


import gpu_helpers as H  # noqa: E402
import sparse_top_selection_amd as sa  # noqa: E402


def last_positions(d: dict, n: int, sel_cap: int = None) -> dict:
    """The problem restricted to its last n positions (same pools); rows
    optionally padded with -1 to a wider stride."""
    e = dict(d)
    e["q"] = np.ascontiguousarray(d["q"][-n:])
    sel = d["sel"][-n:]
    if sel_cap is not None and sel_cap > sel.shape[1]:
        pad = np.full((n, sel_cap - sel.shape[1]), -1, np.int32)
        sel = np.concatenate([sel, pad], axis=1)
    e["sel"] = np.ascontiguousarray(sel)
    e["sel_len"] = np.ascontiguousarray(d["sel_len"][-n:])
    e["n_q"] = n
    return e


def both_calls(d: dict):
    """(noalloc output, workspace output, noalloc status) for one problem."""
    dev = H.to_device(d)
    n_q, cap = d["sel"].shape
    n_kv = d["k_pool"].shape[1]
    dims = sa.make_dims(int(d["n_ctx"]), n_q, n_kv, d["k_pool"].shape[0], sel_cap=cap)
    scale = float(d["softmax_scale"])
    out_a = torch.full_like(dev["q"], float("nan"))
    st_a = sa.new_status(dev["q"].device)
    sa.sel_attn_decode_noalloc(dims, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                               dev["v_scale"], dev["page_table"], dev["sel"], dev["sel_len"], scale,
                               out_a, st_a)
    torch.cuda.synchronize()
    out_b = torch.full_like(dev["q"], float("nan"))
    st_b = sa.new_status(dev["q"].device)
    need = sa.sel_attn_decode_workspace_bytes(dims)
    ws = torch.empty(need, dtype=torch.uint8, device=dev["q"].device)
    sa.sel_attn_decode(dims, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                       dev["v_scale"], dev["page_table"], dev["sel"], dev["sel_len"], scale, out_b,
                       ws, need, st_b)
    torch.cuda.synchronize()
    assert sa.status_value(st_b) == 0
    return out_a.cpu().numpy(), out_b.cpu().numpy(), sa.status_value(st_a)


def check_case(d: dict, what: str):
    print("case", what, "n_q", d["sel"].shape[0], "sel_cap", d["sel"].shape[1], flush=True)
    got, ref_ws, status = both_calls(d)
    assert status == 0
    assert np.array_equal(got.view(np.uint32), ref_ws.view(np.uint32)), \
        "noalloc output differs from the workspace call (%s)" % what
    H.assert_close(got, oracle.attention_of(d), what)


def test_noalloc_matches_workspace_call_twice_second_smaller():
    """Two calls in a row on one GPU: a 5-position verify window at the end of
    the 64K context (sel_cap 2,560: 5 x 4 x 40 records), then one position at
    the end of the 8K context (4 x 33 records), each bit-identical to the call
    with a caller workspace."""
    big = last_positions(synth.as_problem(synth.generate(synth.workload(4))), 5, sel_cap=2560)
    check_case(big, "ctx64k_independent last 5 (sel_cap 2560)")
    small = last_positions(synth.as_problem(synth.generate(synth.workload(1))), 1)
    check_case(small, "ctx8k_drift005 last 1")


def test_noalloc_largest_accepted_size_then_small():
    """The largest call the 8 MiB array takes at sel_cap 2,560 (8 positions x 4
    KV heads x 40 splits = 1,280 records), then a single position of another
    context."""
    d = last_positions(synth.as_problem(synth.generate(synth.workload(3))), 8, sel_cap=2560)
    n_q, cap = d["sel"].shape
    dims = sa.make_dims(int(d["n_ctx"]), n_q, 4, d["k_pool"].shape[0], sel_cap=cap)
    assert sa.sel_attn_decode_workspace_bytes(dims) <= sa.DECODE_NOALLOC_MAX_BYTES
    check_case(d, "ctx40k_drift05_shuffled last 8 (sel_cap 2560)")
    one = last_positions(synth.as_problem(synth.generate(synth.workload(0))), 1)
    check_case(one, "ctx1536_dense last 1")


def test_noalloc_rejects_sizes_beyond_the_array():
    """9 positions x 4 KV heads x 40 splits do not fit: EINVAL, nothing enqueued."""
    d = synth.as_problem(synth.generate(synth.workload(1)))
    dev = H.to_device(last_positions(d, 9, sel_cap=2560))
    dims = sa.make_dims(int(d["n_ctx"]), 9, 4, d["k_pool"].shape[0], sel_cap=2560)
    out = torch.full_like(dev["q"], 7.0)
    with pytest.raises(sa.SelAttnError) as e:
        sa.sel_attn_decode_noalloc(dims, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                                   dev["v_scale"], dev["page_table"], dev["sel"], dev["sel_len"],
                                   float(d["softmax_scale"]), out, sa.new_status(dev["q"].device))
    assert e.value.code == sa.EINVAL and "static scratch" in sa.sel_attn_last_error()
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
