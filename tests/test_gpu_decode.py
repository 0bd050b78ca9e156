"""Parity of the decode call (a few positions, each split over its cells) with
the CPU oracle, through the C ABI.

Page cited: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
section Summary: every position attends to exactly its own selected cells; the
page leaves decode and its speculative verify window as they are, and this call
computes the same definition for that workload. Gate as for the prompt path:
max abs <= 8e-3 and mean abs <= 1e-3 against FP64.
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


def last_positions(d: dict, n: int) -> dict:
    """The problem restricted to its last n query positions (same pools)."""
    e = dict(d)
    for k in ("q", "sel", "sel_len"):
        e[k] = np.ascontiguousarray(d[k][-n:])
    e["n_q"] = n
    return e


def run_decode(d: dict, dev: dict = None, workspace=None):
    if dev is None:
        dev = H.to_device(d)
    out, status = sa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                            dev["v_scale"], dev["page_table"], dev["sel"], dev["sel_len"],
                            float(d["softmax_scale"]), int(d["n_ctx"]), workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy(), sa.status_value(status)


@pytest.mark.parametrize("idx,n", [(0, 1), (1, 1), (2, 1), (3, 5), (4, 1), (4, 5), (2, 8)])
def test_decode_last_positions(idx, n):
    """One position (decode) or a verify window of 5 or 8 at the end of each
    workload's context."""
    w = synth.workload(idx)
    print("case decode", w.name, n, flush=True)
    d = last_positions(synth.as_problem(synth.generate(w)), n)
    out, status = run_decode(d)
    assert status == 0
    H.assert_close(out, oracle.attention_of(d), "decode %s x%d" % (w.name, n))


@pytest.mark.parametrize("seed,n_ctx,n_q,n_kv,dup,nonres", [
    (81, 1000, 6, 2, 0.3, 0.3), (82, 3000, 3, 1, 0.0, 0.5), (83, 9000, 4, 5, 0.4, 0.2),
    (84, 70000, 2, 4, 0.2, 0.1)])
def test_decode_random_selections(seed, n_ctx, n_q, n_kv, dup, nonres):
    """Unsorted rows with repeats, not-resident pages, empty rows, 1 to 5 KV
    heads, rows shorter than one split and up to the cap."""
    print("case decode random", seed, flush=True)
    d = synth.small_random(seed, n_ctx=n_ctx, n_q=n_q, n_kv=n_kv, dup_frac=dup,
                           nonresident_frac=nonres, pool_extra=2)
    out, status = run_decode(d)
    assert status == 0
    H.assert_close(out, oracle.attention_of(d), "decode random %d" % seed)
    assert np.all(out[d["sel_len"] == 0] == 0)


def test_decode_matches_positions_call_and_reruns_bitwise():
    """A shared workspace across calls of different sizes; the same bits on a
    rerun; agreement with the per-position prompt call to rounding."""
    w = synth.workload(4)
    print("case decode rerun", flush=True)
    d = last_positions(synth.as_problem(synth.generate(w)), 5)
    dev = H.to_device(d)
    dims = sa.make_dims(w.n_ctx, 5, w.n_kv, w.pool_pages, sel_cap=w.sel_cap)
    ws = torch.empty(sa.sel_attn_decode_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    a, _ = run_decode(d, dev, ws)
    one = last_positions(d, 1)
    b1, _ = run_decode(one, None, ws)                # a smaller call in the same workspace
    b, _ = run_decode(d, dev, ws)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    pos, status = sa.prefill_positions(dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                                       dev["v_scale"], dev["page_table"], dev["sel"],
                                       dev["sel_len"], float(d["softmax_scale"]), w.n_ctx)
    torch.cuda.synchronize()
    assert np.max(np.abs(pos.cpu().numpy().astype(np.float64) - a)) <= 2e-3
    assert np.max(np.abs(b1[0].astype(np.float64) - a[-1])) <= 2e-3


def test_decode_flags_data_errors():
    d = synth.small_random(91, n_ctx=640, n_q=4, n_kv=1)
    dev = H.to_device(d)
    pt = dev["page_table"].clone()
    pt[2] = d["n_pages"] + 5
    vs = dev["v_scale"].clone()
    vs[int(d["page_table"][0])] = 8.0
    sel = dev["sel"].clone()
    sel_len = dev["sel_len"].clone()
    sel[1, 0] = 700
    sel_len[1] = max(int(sel_len[1]), 1)
    sel_len[2] = sel.shape[1] + 3
    sel[0, :3] = torch.tensor([0, 130, 150], dtype=torch.int32, device="cuda")
    sel_len[0] = max(int(sel_len[0]), 3)
    out, st = sa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], vs, pt, sel,
                        sel_len, float(d["softmax_scale"]), 640)
    torch.cuda.synchronize()
    v = sa.status_value(st)
    assert v & sa.STATUS_PAGE_RANGE and v & sa.STATUS_V_SCALE
    assert v & sa.STATUS_CELL_RANGE and v & sa.STATUS_SEL_LEN
    assert np.all(np.isfinite(out.cpu().numpy()))


def test_decode_rows_at_the_cap():
    """Rows of 2,560 entries (the cap, 40 splits): 2,560 distinct cells shuffled
    (the dedup table at its fullest) or ascending, and 1,280 cells twice each."""
    print("case decode rows at the cap", flush=True)
    rng = np.random.default_rng(91)
    n_ctx = 70000
    d = synth.small_random(91, n_ctx=n_ctx, n_q=3, n_kv=2, sel_cap=2560, max_len=10,
                           nonresident_frac=0.1)
    sel = np.empty((3, 2560), np.int32)
    for j in range(3):
        p = n_ctx - 3 + j
        if j < 2:
            cells = rng.choice(p + 1, size=2560, replace=False)
            sel[j] = cells if j == 0 else np.sort(cells)
        else:
            cells = rng.choice(p + 1, size=1280, replace=False)
            sel[j] = rng.permutation(np.concatenate([cells, cells]))
    d["sel"], d["sel_len"] = sel, np.full(3, 2560, np.int32)
    out, status = run_decode(d)
    assert status == 0
    H.assert_close(out, oracle.attention_of(d), "decode rows at the cap")
