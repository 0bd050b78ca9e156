"""Exact pins of the K path on the GPU: one dominant cell.

The tolerance gate (max abs 8e-3) cannot see one mis-gathered K row among
~2,000 cells, and the exact-mean test zeroes k_scale, so K itself never
matters there. Here K decides everything: every q row is a positive multiple
of a fixed +-1 vector sigma and one cell's K row (in every KV head) is
127 * sigma, so that cell's logit beats every other logit of every row that
chose it by more than 160 log2 units. Every other FP16 probability then
underflows to 0, and when the cell first arrives in a later chunk, the running
maximum moves and what was accumulated before is multiplied by exp2(<= -160),
which is 0 in FP32. With v_scale * 2^6 exact in FP16, the output of every such
row is then exactly v_scale * v_int of that cell: any wrong K row, page
translation, chunk position or rescale step shows up as a wrong value.

Page cited: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
section Summary: every position attends to exactly its own selected cells
(-inf for the cells it did not choose), which here reduces to the one cell.
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

# Cells of the 32K chunk (positions 24,576..32,767): a sink (chunk 0 of every
# union, no rescale), the start of a local block near the end of the context
# (last chunks of its own groups' unions, and a far block of other positions),
# and one in the middle of the context.
DOMINANT = (1, 30000, 25000)


def dominant_problem(cell: int, seed: int = 0) -> dict:
    w = synth.workload(2)
    d = synth.as_problem(synth.generate(w))
    rng = np.random.default_rng(seed)
    sigma = np.where(rng.random(w.head_dim) < 0.5, -1.0, 1.0).astype(np.float32)
    a = rng.uniform(0.5, 1.5, size=(w.n_q, w.n_qh, 1)).astype(np.float32)
    d["q"] = np.ascontiguousarray(a * sigma[None, None, :])
    page = int(d["page_table"][cell // 64])
    assert page >= 0
    k = d["k_pool"].copy()
    k[page, :, cell % 64, :] = (127 * sigma).astype(np.int8)
    d["k_pool"] = k
    # k_scale 0.5 everywhere: the dominant logit exceeds every other by
    # 0.5 * 0.0884 * 1.4427 * (16256 - max |sigma.k|) * min(a) > 160 log2 units
    d["k_scale"] = np.full_like(d["k_scale"], np.float32(0.5))
    # v_scale * 2^6 exact in FP16: (1 + i/16) * 2^-8, i = 0..15
    i = rng.integers(0, 16, size=d["v_scale"].shape)
    d["v_scale"] = ((1.0 + i / 16.0) * 2.0 ** -8).astype(np.float32)
    d["dominant"] = (cell, page)
    return d


def pinned_rows(d: dict):
    """Query indices whose (resident) selection contains the dominant cell, and
    the exact expected output of each of their rows."""
    cell, page = d["dominant"]
    rows = [j for j in range(d["sel"].shape[0]) if np.any(d["sel"][j, :d["sel_len"][j]] == cell)]
    n_kv = d["k_pool"].shape[1]
    ref = np.zeros((n_kv * 12, 128), np.float64)
    for kv in range(n_kv):
        ref[kv * 12:(kv + 1) * 12] = (np.float64(d["v_scale"][page, kv, cell % 64]) *
                                      d["v_pool"][page, kv, cell % 64, :].astype(np.float64))
    return np.array(rows, np.int64), ref


def assert_exact(got: np.ndarray, rows: np.ndarray, ref: np.ndarray, what: str):
    sub = got[rows].astype(np.float64)
    tol = 2 * np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    bad = np.abs(sub - ref[None]) > tol[None]
    print("%s: %d pinned rows, %d outputs off" % (what, rows.size, int(bad.sum())), flush=True)
    assert not bad.any(), (what, np.argwhere(bad)[:5])


@pytest.mark.parametrize("cell", DOMINANT)
def test_union_path_dominant_cell_exact(cell):
    d = dominant_problem(cell)
    rows, ref = pinned_rows(d)
    assert rows.size >= 16
    out, cells, mask, length, status = H.run_path(d)
    assert status == 0
    # where the cell sits in its groups' unions: the late and middle cells come
    # after the first chunk in every group, so the rescale path runs
    pos = []
    for g in sorted(set((rows // 8).tolist())):
        idx = int(np.searchsorted(cells[g, :length[g]], cell))
        pos.append(idx // 32)
    print("chunk of the dominant cell in its unions: min %d max %d" % (min(pos), max(pos)), flush=True)
    if cell != 1:
        assert min(pos) > 0
    assert_exact(out, rows, ref, "union path, cell %d" % cell)
    # the oracle agrees with the closed form
    assert np.max(np.abs(oracle.attention_of(d, rows=rows[:4].astype(np.int32)) - ref[None])) <= 1e-12


@pytest.mark.parametrize("cell", DOMINANT)
def test_positions_call_dominant_cell_exact(cell):
    d = dominant_problem(cell)
    rows, ref = pinned_rows(d)
    dev = H.to_device(d)
    out, status = sa.prefill_positions(dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                                       dev["v_scale"], dev["page_table"], dev["sel"],
                                       dev["sel_len"], float(d["softmax_scale"]), int(d["n_ctx"]))
    torch.cuda.synchronize()
    assert sa.status_value(status) == 0
    assert_exact(out.cpu().numpy(), rows, ref, "per-position call, cell %d" % cell)


@pytest.mark.parametrize("cell", DOMINANT)
def test_decode_call_dominant_cell_exact(cell):
    """Decode over 5 pinned positions (first, last and three between): the
    dominant cell falls in different splits of different rows."""
    d = dominant_problem(cell)
    rows, ref = pinned_rows(d)
    pick = rows[np.linspace(0, rows.size - 1, 5).round().astype(int)]
    e = dict(d)
    for k in ("q", "sel", "sel_len"):
        e[k] = np.ascontiguousarray(d[k][pick])
    e["n_q"] = pick.size
    splits = [int(np.argmax(e["sel"][r, :e["sel_len"][r]] == d["dominant"][0])) // 64
              for r in range(pick.size)]
    print("decode splits holding the cell:", splits, flush=True)
    dev = H.to_device(e)
    out, status = sa.decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                            dev["v_scale"], dev["page_table"], dev["sel"], dev["sel_len"],
                            float(e["softmax_scale"]), int(e["n_ctx"]))
    torch.cuda.synchronize()
    assert sa.status_value(status) == 0
    assert_exact(out.cpu().numpy(), np.arange(pick.size), ref, "decode, cell %d" % cell)


def test_union_path_flags_rows_outside_the_pools():
    """A union row whose KV-head rows would leave the pools (at or past
    (n_pages n_kv - n_kv + 1) 64, or negative other than -1) sets PAGE_RANGE;
    the cell is treated as not resident, every output stays finite, and the
    groups that do not hold it are unchanged. The last row inside the limit
    reads without a flag."""
    d = synth.small_random(35, n_ctx=640, n_q=24, n_kv=2)
    dev = H.to_device(d)
    n_pages = d["k_pool"].shape[0]
    cells, mask, rows, length, status = sa.build_union(dev["sel"], dev["sel_len"], 640,
                                                       dev["page_table"], 2, n_pages)
    torch.cuda.synchronize()
    assert sa.status_value(status) == 0
    ref_out, st0 = sa.prefill(dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                              dev["v_scale"], rows, mask, length, float(d["softmax_scale"]), 640)
    torch.cuda.synchronize()
    assert sa.status_value(st0) == 0
    lens = length.cpu().numpy()
    limit = (n_pages * 2 - 2 + 1) * 64
    r = ref_out.cpu().numpy()
    keep = np.r_[0:8, 16:24]                      # groups 0 and 2
    for bad_row, flagged in ((limit, True), (limit + 10 ** 6, True), (-2, True),
                             (-5000, True), (limit - 1, False)):
        print("case row", bad_row, flush=True)
        r2 = rows.clone()
        r2[1, int(lens[1]) // 2] = bad_row        # group 1 only
        out, st = sa.prefill(dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                             dev["v_scale"], r2, mask, length, float(d["softmax_scale"]), 640)
        torch.cuda.synchronize()
        v = sa.status_value(st)
        assert v == (sa.STATUS_PAGE_RANGE if flagged else 0), (bad_row, v)
        o = out.cpu().numpy()
        assert np.all(np.isfinite(o))
        assert np.array_equal(o[keep].view(np.uint32), r[keep].view(np.uint32))
