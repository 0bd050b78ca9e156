"""Parity of sel_attn_prefill_split against the FP64 oracle, through the C ABI.

Grids of fewer than 512 (group, KV head) work-groups are split when their
unions can be long enough: each group's union is divided at chunk boundaries
over several work-groups whose states (running maximum, probability sum, O) a
merge kernel combines. Checked here: the dense 1,536-cell workload (32 groups,
4 splits each) on every output, small random problems in which many splits are
empty or short (empty groups, short rows, repeats, non-resident pages), the
one-dominant-cell closed form with the cell in one split and the other splits of
its rows weighted to exactly 0, a bitwise rerun, and grids that do not split
(large, or unions too short), which must equal sel_attn_prefill bit for bit.

Page cited: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
section Summary (every position attends to exactly its own selected cells, over
the group's union) and the accuracy list in section Summary (the parity cases).
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
from test_gpu_exact_k import DOMINANT, dominant_problem, pinned_rows, assert_exact  # noqa: E402


def expected_splits(n_q: int, n_kv: int, n_ctx: int, sel_cap: int) -> int:
    """The split rule of include/sel_attn.h, restated."""
    items = (n_q + 7) // 8 * n_kv
    if items >= 512:
        return 1
    chunks = -(-min(8 * sel_cap, n_ctx) // 32)
    return max(1, min(16, -(-512 // items), chunks // 12))


def run_split(d: dict, dev: dict = None):
    """Union, then the split attention. Returns numpy (out, status, splits)."""
    if dev is None:
        dev = H.to_device(d)
    n_ctx = int(d["n_ctx"])
    out, _, status = sa.attention(dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                                  dev["v_scale"], dev["page_table"], dev["sel"], dev["sel_len"],
                                  float(d["softmax_scale"]), n_ctx, split=True)
    torch.cuda.synchronize()
    n_q, n_kv = d["q"].shape[0], d["k_pool"].shape[1]
    sel_cap = d["sel"].shape[1]
    dims = sa.make_dims(n_ctx, n_q, n_kv, d["k_pool"].shape[0], sel_cap=sel_cap)
    items = (n_q + 7) // 8 * n_kv
    splits = max(1, sa.sel_attn_prefill_workspace_bytes(dims) // (items * 49920))
    assert splits == expected_splits(n_q, n_kv, n_ctx, sel_cap)
    return out.cpu().numpy(), sa.status_value(status), splits


def test_split_dense_workload_all_rows():
    w = synth.workload(0)
    print("case", w.name, flush=True)
    d = synth.as_problem(synth.generate(w))
    out, status, splits = run_split(d)
    assert status == 0 and splits == 4
    H.assert_close(out, oracle.attention_of(d), "split " + w.name)


@pytest.mark.parametrize("seed,n_ctx,n_q,n_kv,dup,nonres,max_len", [
    (51, 2600, 40, 2, 0.3, 0.3, 300),    # 10 items, 6 splits: short unions, many empty splits
    (52, 5000, 9, 1, 0.0, 0.2, None),    # 2 items, 13 splits, long rows (ragged last group of 1)
    (53, 1600, 13, 3, 0.5, 0.0, None),   # 6 items, 4 splits
    (54, 40000, 64, 4, 0.1, 0.1, None)])  # 32 items, 16 splits over a long context
def test_split_random_problems_all_rows(seed, n_ctx, n_q, n_kv, dup, nonres, max_len):
    print("case", seed, n_ctx, n_q, n_kv, flush=True)
    kw = {} if max_len is None else {"max_len": max_len}
    d = synth.small_random(seed, n_ctx=n_ctx, n_q=n_q, n_kv=n_kv, dup_frac=dup,
                           nonresident_frac=nonres, pool_extra=2, **kw)
    if seed == 51:
        d["sel_len"][8:16] = 0            # group 1: an empty union, every split empty
        d["sel"][8:16] = -1
    out, status, splits = run_split(d)
    assert status == 0 and splits > 1
    H.assert_close(out, oracle.attention_of(d), "split random seed %d" % seed)
    assert np.all(out[d["sel_len"] == 0] == 0)


@pytest.mark.parametrize("cell", DOMINANT)
def test_split_dominant_cell_exact(cell):
    """A 64-position window of the dominant-cell problem (8 groups x 4 KV heads,
    16 splits each): the rows that chose the cell must output exactly its V."""
    d = dominant_problem(cell)
    rows, ref = pinned_rows(d)
    # the aligned 64-position window holding the most pinned rows
    starts = np.arange(0, d["q"].shape[0], 64)
    counts = [int(np.sum((rows >= s) & (rows < s + 64))) for s in starts]
    s0 = int(starts[int(np.argmax(counts))])
    assert max(counts) >= 8
    win = dict(d)
    for key in ("q", "sel", "sel_len"):
        win[key] = np.ascontiguousarray(d[key][s0:s0 + 64])
    out, status, splits = run_split(win)
    assert status == 0 and splits == 16
    local = rows[(rows >= s0) & (rows < s0 + 64)] - s0
    assert_exact(out, local, ref, "split path, cell %d" % cell)


def test_split_rerun_is_bitwise():
    d = synth.small_random(55, n_ctx=3000, n_q=48, n_kv=2, dup_frac=0.2, nonresident_frac=0.2,
                           pool_extra=1)
    dev = H.to_device(d)
    a, _, _ = run_split(d, dev)
    b, _, _ = run_split(d, dev)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_large_grid_does_not_split():
    """8K chunk: 128 groups x 4 KV heads = 512 work-groups, no split: the call
    is sel_attn_prefill, bit for bit."""
    w = synth.workload(1)
    d = synth.as_problem(synth.generate(w))
    dev = H.to_device(d)
    out_split, status, splits = run_split(d, dev)
    assert splits == 1 and status == 0
    out_ref, _, _, _, _ = H.run_path(d, dev)
    assert np.array_equal(out_split.view(np.uint32), out_ref.view(np.uint32))


def test_short_context_does_not_split():
    """A small grid over a 300-cell context (10 chunks at most): too short to
    share out, so the call is sel_attn_prefill, bit for bit."""
    d = synth.small_random(56, n_ctx=300, n_q=24, n_kv=2, dup_frac=0.2, nonresident_frac=0.1,
                           pool_extra=1)
    dev = H.to_device(d)
    out_split, status, splits = run_split(d, dev)
    assert splits == 1 and status == 0
    out_ref, _, _, _, _ = H.run_path(d, dev)
    assert np.array_equal(out_split.view(np.uint32), out_ref.view(np.uint32))
    H.assert_close(out_split, oracle.attention_of(d), "short context")
