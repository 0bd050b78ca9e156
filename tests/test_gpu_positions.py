"""Parity of the per-position attention (no union) with the CPU oracle, through
the C ABI.

Page cited: #2808 "sycl: prompt attention over 8-query selection unions on XMX".
Section Summary: every position gathers its own selected cells (the FP32
kernel), which defines the output. Section Extra Notes: the union path wins
only where adjacent positions' selections share cells; this call serves
batches where they do not. Gate as for the union path: max abs <= 8e-3 and mean abs <= 1e-3 against
FP64, every output of every workload at full size.
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


def run_positions(d: dict, dev: dict = None):
    """Per-position attention; returns numpy (out, status)."""
    if dev is None:
        dev = H.to_device(d)
    out, status = sa.prefill_positions(dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                                       dev["v_scale"], dev["page_table"], dev["sel"],
                                       dev["sel_len"], float(d["softmax_scale"]), int(d["n_ctx"]))
    torch.cuda.synchronize()
    return out.cpu().numpy(), sa.status_value(status)


def _check(d, rows=None, what=""):
    out, status = run_positions(d)
    assert status == 0, status
    ref = oracle.attention_of(d, rows=rows)
    H.assert_close(out if rows is None else out[rows], ref, what)
    return out


@pytest.mark.parametrize("idx", range(5))
def test_positions_workloads_all_rows(idx):
    w = synth.workload(idx)
    print("case positions", w.name, flush=True)
    d = synth.as_problem(synth.generate(w))
    out = _check(d, what="positions " + w.name)
    vmax = float(np.abs(d["v_pool"].astype(np.float32) * d["v_scale"][..., None]).max())
    assert float(np.abs(out).max()) <= vmax * (1 + 1e-2)


@pytest.mark.parametrize("seed,n_ctx,n_q,n_kv,dup,nonres", [
    (51, 1000, 45, 2, 0.3, 0.3), (52, 3000, 64, 1, 0.0, 0.5), (53, 700, 13, 3, 0.5, 0.0),
    (54, 4100, 9, 4, 0.2, 0.1), (55, 9000, 30, 5, 0.4, 0.2), (56, 2600, 17, 8, 0.1, 0.0)])
def test_positions_random_selections(seed, n_ctx, n_q, n_kv, dup, nonres):
    """Unsorted rows with repeats, not-resident pages, empty rows, 1 to 8 KV
    heads (more than one head per wave at 5 and 8), rows of every length."""
    print("case positions random", seed, flush=True)
    d = synth.small_random(seed, n_ctx=n_ctx, n_q=n_q, n_kv=n_kv, dup_frac=dup,
                           nonresident_frac=nonres, pool_extra=2)
    out = _check(d, what="positions random %d" % seed)
    assert np.all(out[d["sel_len"] == 0] == 0)


def test_positions_repeats_fill_the_dedup_table():
    """Rows of 2,560 entries (the cap) holding 1,280 distinct cells twice each,
    or one cell 2,560 times, in shuffled order; and 2,560 distinct cells,
    shuffled (the table at its fullest) or ascending (no table)."""
    print("case positions dedup", flush=True)
    rng = np.random.default_rng(61)
    d = synth.small_random(61, n_ctx=70000, n_q=6, n_kv=2, sel_cap=2560, max_len=10)
    sel = np.full((6, 2560), -1, np.int32)
    sel_len = np.full(6, 2560, np.int32)
    for j in range(6):
        p = 70000 - 6 + j
        if j == 3:
            sel[j] = rng.integers(0, p + 1)
        elif j >= 4:
            cells = rng.choice(p + 1, size=2560, replace=False)
            sel[j] = cells if j == 4 else np.sort(cells)
        else:
            cells = rng.choice(p + 1, size=1280, replace=False)
            sel[j] = rng.permutation(np.concatenate([cells, cells]))
    d["sel"], d["sel_len"] = sel, sel_len
    _check(d, what="positions dedup")


def test_positions_exact_mean_catches_single_cell_errors():
    """k_scale = 0 and v_scale = 2^-6: every probability is exactly 1 and every
    sum exact, so the output is 2^-6 * mean(v_int over the set) within 2 ulp."""
    w = synth.workload(4)
    print("case positions exact mean", flush=True)
    d = synth.as_problem(synth.generate(w))
    d["k_scale"] = np.zeros_like(d["k_scale"])
    d["v_scale"] = np.full_like(d["v_scale"], np.float32(2.0 ** -6))
    pt = d["page_table"].copy()
    pt[[5, 300, 777]] = -1
    d["page_table"] = pt
    out, status = run_positions(d)
    assert status == 0
    rows = H.sample_rows(w.n_q, 12, seed=9)
    ref = np.zeros((rows.size, w.n_qh, w.head_dim))
    for r, j in enumerate(rows):
        cells = np.unique(d["sel"][j, :d["sel_len"][j]])
        pp = pt[cells // 64]
        cells, pp = cells[pp >= 0], pp[pp >= 0]
        for kv in range(w.n_kv):
            tot = d["v_pool"][pp, kv, cells % 64, :].astype(np.int64).sum(axis=0)
            ref[r, kv * 12:(kv + 1) * 12] = (tot / cells.size) * 2.0 ** -6
    got = out[rows].astype(np.float64)
    tol = 2 * np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (np.argwhere(bad)[:5], got[bad][:5], ref[bad][:5])


def test_positions_bitwise_rerun_and_agreement_with_union_path():
    w = synth.workload(3)
    print("case positions rerun", flush=True)
    d = synth.as_problem(synth.generate(w))
    dev = H.to_device(d)
    a, _ = run_positions(d, dev)
    b, _ = run_positions(d, dev)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    u = H.run_path(d, dev)[0]
    assert np.max(np.abs(a.astype(np.float64) - u)) <= 2 * H.MAX_ABS


def test_positions_flags_data_errors():
    d = synth.small_random(71, n_ctx=640, n_q=16, n_kv=1)
    dev = H.to_device(d)
    pt = dev["page_table"].clone()
    pt[2] = d["n_pages"] + 5
    vs = dev["v_scale"].clone()
    vs[int(d["page_table"][0])] = 8.0
    sel = dev["sel"].clone()
    sel_len = dev["sel_len"].clone()
    sel[3, 0] = 700            # outside [0, n_ctx)
    sel_len[3] = max(int(sel_len[3]), 1)
    sel_len[5] = sel.shape[1] + 3
    out, st = sa.prefill_positions(dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], vs, pt,
                                   sel, sel_len, float(d["softmax_scale"]), 640)
    torch.cuda.synchronize()
    v = sa.status_value(st)
    assert v & sa.STATUS_PAGE_RANGE and v & sa.STATUS_V_SCALE
    assert v & sa.STATUS_CELL_RANGE and v & sa.STATUS_SEL_LEN
    assert np.all(np.isfinite(out.cpu().numpy()))
