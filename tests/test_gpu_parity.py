"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Union: bit-exact (cells, masks, lengths). Attention: max abs <= 8e-3 and mean
abs <= 1e-3 against FP64 on every workload, plus an exact-arithmetic case that
catches a single wrong cell or mask bit, non-resident pages, empty rows, ragged
groups, long contexts (several union windows) and a bitwise rerun.
Page cited: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
the accuracy list in section Summary (the parity self-test's cases).
"""
import dataclasses

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


import gpu_helpers as H  # noqa: E402  (imports the binding; only after the skip check)
import sparse_top_selection_amd as sa  # noqa: E402


# ----------------------------------------------------------------------------- union
def _random_table(rng, n_ctx: int, n_pages: int, nonresident: float):
    """A page table over n_pages physical pages: logical pages in a random
    order, a share of them not resident (-1)."""
    n_lp = -(-n_ctx // 64)
    table = rng.integers(0, n_pages, size=n_lp).astype(np.int32)
    table[rng.random(n_lp) < nonresident] = -1
    return table


def _union_on_gpu(sel, sel_len, n_ctx, table, n_kv, n_pages, sel_dev=None):
    """build_union through the C ABI; numpy (cells, mask, rows, length, status)."""
    sel_dev = torch.from_numpy(sel).cuda() if sel_dev is None else sel_dev
    cells, mask, rows, length, status = sa.build_union(
        sel_dev, torch.from_numpy(sel_len).cuda(), n_ctx, torch.from_numpy(table).cuda(), n_kv,
        n_pages)
    torch.cuda.synchronize()
    return (cells.cpu().numpy(), mask.cpu().numpy(), rows.cpu().numpy(), length.cpu().numpy(),
            sa.status_value(status))


def _check_union_on_gpu(sel, sel_len, n_ctx, table, n_kv, n_pages, sel_dev=None):
    cells, mask, rows, length, st = _union_on_gpu(sel, sel_len, n_ctx, table, n_kv, n_pages,
                                                  sel_dev)
    assert st == 0
    ref = oracle.union(sel, sel_len, n_ctx)
    H.assert_union_equal(cells, mask, length, ref)
    ref_rows, flags = oracle.union_rows(ref[0], ref[2], table, n_kv, n_pages)
    assert flags == 0
    H.assert_union_rows_equal(rows, length, ref_rows)


@pytest.mark.parametrize("idx", range(5))
def test_union_bit_exact_on_workloads(idx):
    w = synth.workload(idx)
    d = synth.as_problem(synth.generate(w, with_q=False, with_pools=False))
    print("case", w.name, flush=True)
    table = _random_table(np.random.default_rng(100 + idx), w.n_ctx, w.pool_pages, 0.2)
    _check_union_on_gpu(d["sel"], d["sel_len"], w.n_ctx, table, w.n_kv, w.pool_pages)


@pytest.mark.parametrize("n_ctx,n_q,seed", [(300, 45, 1), (5000, 33, 2), (70000, 17, 3),
                                            (200001, 9, 4), (64, 8, 5), (1, 3, 6)])
def test_union_bit_exact_edge_cases(n_ctx, n_q, seed):
    """Ragged groups, repeats, unsorted rows, empty rows, contexts over one window."""
    print("case", n_ctx, n_q, seed, flush=True)
    rng = np.random.default_rng(seed)
    cap = 2051
    sel = np.full((n_q, cap), -1, np.int32)
    sel_len = np.zeros(n_q, np.int32)
    for j in range(n_q):
        kind = j % 4
        if kind == 0:
            row = np.zeros(0, np.int32)
        elif kind == 1:
            row = np.array([n_ctx - 1], np.int32)          # a cell on the last page
        else:
            n = int(rng.integers(1, cap + 1))
            row = rng.integers(0, n_ctx, size=n).astype(np.int32)   # with repeats
        sel[j, :row.size] = row
        sel_len[j] = row.size
    n_pages = 1 + seed % 5
    _check_union_on_gpu(sel, sel_len, n_ctx, _random_table(rng, n_ctx, n_pages, 0.3), 1 + seed % 3,
                        n_pages)


@pytest.mark.parametrize("n_ctx,n_q,cap,offset,seed", [(100, 11, 13, 1, 7), (40000, 20, 5003, 3, 8),
                                                        (9000, 16, 3, 2, 9), (2000, 9, 1, 1, 10),
                                                        (70000, 24, 2051, 1, 11)])
def test_union_bit_exact_any_row_stride_and_alignment(n_ctx, n_q, cap, offset, seed):
    """Row strides that put groups at every 4-byte alignment, rows shorter than
    a 16-byte block, and groups too long for one pass of loads."""
    print("case", n_ctx, n_q, cap, offset, seed, flush=True)
    rng = np.random.default_rng(seed)
    sel = np.full((n_q, cap), -7, np.int32)
    sel_len = rng.integers(0, cap + 1, size=n_q).astype(np.int32)
    sel_len[0] = cap
    for j in range(n_q):
        sel[j, :sel_len[j]] = rng.integers(0, n_ctx, size=sel_len[j])
    # the rows start `offset` int32 into a device buffer, so the sel pointer is
    # only 4-byte aligned
    flat = torch.full((offset + n_q * cap + 5,), -3, dtype=torch.int32)
    flat[offset:offset + n_q * cap] = torch.from_numpy(sel.reshape(-1))
    dev = flat.cuda()[offset:offset + n_q * cap].view(n_q, cap)
    assert dev.data_ptr() % 16 != 0
    _check_union_on_gpu(sel, sel_len, n_ctx, _random_table(rng, n_ctx, 50, 0.1), 4, 50,
                        sel_dev=dev)


def test_union_flags_bad_cells_and_lengths():
    sel = np.full((10, 16), -1, np.int32)
    sel_len = np.full(10, 3, np.int32)
    sel[:, :3] = [1, 2, 3]
    sel[4, 1] = 100           # outside [0, n_ctx)
    sel[6, 0] = -5
    sel_len[8] = 17           # over the cap: clamped
    table = np.array([3, 1], np.int32)
    cells, mask, rows, length, st = _union_on_gpu(sel, sel_len, 100, table, 2, 4)
    assert st == sa.STATUS_CELL_RANGE | sa.STATUS_SEL_LEN
    # the bad cells are dropped, the rest of the group is intact
    assert length.tolist()[0] == 3
    assert cells[0, :3].tolist() == [1, 2, 3]
    assert mask[0, :3].tolist() == [0xFF ^ 0x40, 0xFF ^ 0x10, 0xFF]
    assert rows[0, :3].tolist() == [3 * 128 + 1, 3 * 128 + 2, 3 * 128 + 3]


@pytest.mark.parametrize("entry", [4, 1 << 30, -2, -(1 << 31)])
def test_union_rows_flag_page_entries_outside_the_pool(entry):
    """A page-table entry outside [-1, n_pages) sets PAGE_RANGE and gives row -1
    for that page's cells only; -1 gives row -1 without a flag."""
    print("case", entry, flush=True)
    sel = np.full((12, 8), -1, np.int32)
    sel_len = np.full(12, 4, np.int32)
    sel[:, :4] = [5, 70, 130, 199]
    table = np.array([3, entry, 0, -1], np.int32)
    cells, mask, rows, length, st = _union_on_gpu(sel, sel_len, 256, table, 2, 4)
    assert st == sa.STATUS_PAGE_RANGE
    assert length.tolist() == [4, 4]
    for g in range(2):
        assert cells[g, :4].tolist() == [5, 70, 130, 199]
        assert rows[g, :4].tolist() == [3 * 128 + 5, -1, 2, -1]
    ref_rows, flags = oracle.union_rows(cells, length, table, 2, 4)
    assert flags == sa.STATUS_PAGE_RANGE
    H.assert_union_rows_equal(rows, length, ref_rows)


# ------------------------------------------------------------------------- attention
def _check_problem(d, rows=None, what=""):
    dev = H.to_device(d)
    out, cells, mask, length, status = H.run_path(d, dev)
    assert status == 0, status
    H.assert_union_equal(cells, mask, length, oracle.union(d["sel"], d["sel_len"], d["n_ctx"]))
    ref = oracle.attention_of(d, rows=rows)
    got = out if rows is None else out[rows]
    H.assert_close(got, ref, what)
    return out


def test_attention_dense_workload_all_rows():
    w = synth.workload(0)
    print("case", w.name, flush=True)
    _check_problem(synth.as_problem(synth.generate(w)), what=w.name)


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_attention_workloads_all_rows(idx):
    """Full-size inputs in the benchmark's launch configuration, every output."""
    w = synth.workload(idx)
    print("case", w.name, flush=True)
    d = synth.as_problem(synth.generate(w))
    out = _check_problem(d, what=w.name)
    # a property that holds for every output: a convex combination of V rows
    vmax = float(np.abs(d["v_pool"].astype(np.float32) * d["v_scale"][..., None]).max())
    assert float(np.abs(out).max()) <= vmax * (1 + 1e-2)


@pytest.mark.parametrize("seed", [2004, 3004])
def test_attention_independent_workload_other_seeds(seed):
    """The 64K workload (independent selections, scales up to 0.05) has the
    largest error against FP64; two more draws of all its inputs, every output
    checked, so that the margin to the gate is not the luck of one seed."""
    w = dataclasses.replace(synth.workload(4), seed=seed)
    print("case", w.name, "seed", seed, flush=True)
    _check_problem(synth.as_problem(synth.generate(w)), what="%s seed %d" % (w.name, seed))


@pytest.mark.parametrize("seed,n_ctx,n_q,n_kv,dup,nonres", [
    (21, 1000, 45, 2, 0.3, 0.3), (22, 3000, 64, 1, 0.0, 0.5), (23, 700, 13, 3, 0.5, 0.0),
    (24, 4100, 9, 4, 0.2, 0.1)])
def test_attention_random_selections_all_rows(seed, n_ctx, n_q, n_kv, dup, nonres):
    print("case", seed, n_ctx, n_q, n_kv, flush=True)
    d = synth.small_random(seed, n_ctx=n_ctx, n_q=n_q, n_kv=n_kv, dup_frac=dup,
                           nonresident_frac=nonres, pool_extra=2)
    out = _check_problem(d, what="random seed %d" % seed)
    empty = d["sel_len"] == 0
    assert np.all(out[empty] == 0)


@pytest.mark.parametrize("seed,n_ctx,n_q,n_kv,cap", [(25, 3000, 27, 2, 37), (26, 5001, 19, 1, 3001),
                                                     (27, 130, 11, 3, 5)])
def test_attention_other_row_strides(seed, n_ctx, n_q, n_kv, cap):
    """Selection rows (and so union rows, 8 * sel_cap) of other strides; contexts
    that end inside a page; ragged last groups; repeats and non-resident pages."""
    print("case", seed, n_ctx, n_q, n_kv, cap, flush=True)
    d = synth.small_random(seed, n_ctx=n_ctx, n_q=n_q, n_kv=n_kv, sel_cap=cap, dup_frac=0.2,
                           nonresident_frac=0.2, pool_extra=1)
    assert d["sel"].shape == (n_q, cap)
    _check_problem(d, what="row stride %d" % cap)


def test_attention_empty_groups_and_chunk_remainders():
    """Groups whose union is empty (every position selected nothing: the chunk
    loop runs zero times) next to groups whose unions end in every position of
    a 4-chunk unroll; rows without a resident chosen cell output 0."""
    print("case empty groups", flush=True)
    d = synth.small_random(41, n_ctx=2600, n_q=40, n_kv=2, max_len=300)
    sel, sel_len = d["sel"].copy(), d["sel_len"].copy()
    sel_len[8:16] = 0                     # group 1: empty union
    sel[8:16] = -1
    sel_len[30] = 0                       # one empty position inside group 3
    sel[30] = -1
    for j, n in zip(range(16, 24), (1, 33, 65, 97, 3, 40, 70, 100)):
        sel_len[j] = min(n, int(sel_len[j]))   # group 2: short rows
    d["sel"], d["sel_len"] = sel, sel_len
    out = _check_problem(d, what="empty groups")
    assert np.all(out[8:16] == 0) and np.all(out[30] == 0)


def test_attention_union_at_full_capacity():
    """Eight positions with disjoint full selections: the group's union holds
    8 * 2,051 = 16,408 cells, its row's whole capacity (513 chunks of 32, the
    last one a quarter full). The last group of the call is such a group, so
    its union row ends where the union arrays end; the group before it is the
    same with its rows in random order, and some pages are not resident."""
    print("case full-capacity union", flush=True)
    cap = 2051
    n_ctx = 8 * cap + 700
    d = synth.small_random(43, n_ctx=n_ctx, n_q=16, n_kv=2, sel_cap=cap, max_len=1,
                           nonresident_frac=0.1, pool_extra=1)
    rng = np.random.default_rng(44)
    sel = np.empty((16, cap), dtype=np.int32)
    for g in range(2):
        cells = rng.permutation(n_ctx)[:8 * cap].astype(np.int32).reshape(8, cap)
        sel[8 * g:8 * g + 8] = cells if g == 0 else np.sort(cells, axis=1)
    d["sel"], d["sel_len"] = sel, np.full(16, cap, dtype=np.int32)
    ref_union = oracle.union(d["sel"], d["sel_len"], n_ctx)
    assert np.all(ref_union[2] == 8 * cap)
    _check_problem(d, what="full-capacity union")


def test_attention_exact_mean_catches_single_cell_errors():
    """k_scale = 0 and v_scale = 2^-6: every logit is exactly 0, so every chosen
    probability is exactly 1 in FP16 and the sums are exact in FP32; the output
    is 2^-6 * mean(v_int over the resident set) to within 2 ulp. Dropping or
    adding one cell of ~2,000 would move it far more. (Zero scales rather than
    zero K integers: the kernel keeps K with a constant offset in its FP16 tile
    and removes it in FP32, which is exact only up to rounding.)"""
    w = synth.workload(2)
    print("case exact mean", w.name, flush=True)
    d = synth.as_problem(synth.generate(w))
    d["k_scale"] = np.zeros_like(d["k_scale"])
    d["v_scale"] = np.full_like(d["v_scale"], np.float32(2.0 ** -6))
    pt = d["page_table"].copy()
    pt[[3, 100, 257, 511]] = -1               # some pages not resident
    d["page_table"] = pt
    dev = H.to_device(d)
    out, cells, mask, length, status = H.run_path(d, dev)
    assert status == 0
    rows = H.sample_rows(w.n_q, 16, seed=7)
    # closed form in integer arithmetic: 2^-6 * sum(v_int) / |R_j|
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
    # the oracle agrees with the closed form
    assert np.max(np.abs(oracle.attention_of(d, rows=rows[:8]) - ref[:8])) <= 1e-15


def test_attention_bitwise_rerun_and_row_order():
    w = synth.workload(3)            # shuffled rows
    print("case rerun", w.name, flush=True)
    d = synth.as_problem(synth.generate(w))
    dev = H.to_device(d)
    out1 = H.run_path(d, dev)[0]
    out2 = H.run_path(d, dev)[0]
    assert np.array_equal(out1.view(np.uint32), out2.view(np.uint32))
    # sorting every selection row changes nothing (the union is a set)
    s = d["sel"].copy()
    for j in range(w.n_q):
        s[j, :d["sel_len"][j]] = np.sort(s[j, :d["sel_len"][j]])
    e = dict(d)
    e["sel"] = s
    out3 = H.run_path(e)[0]
    assert np.array_equal(out1.view(np.uint32), out3.view(np.uint32))


def test_attention_flags_data_errors():
    d = synth.small_random(31, n_ctx=640, n_q=16, n_kv=1)
    dev = H.to_device(d)
    n_pages = d["k_pool"].shape[0]
    # a page-table entry past the pool: flagged when the union is built, and
    # that page's cells get row -1 (not resident)
    pt = dev["page_table"].clone()
    pt[2] = n_pages + 5
    cells, mask, rows, length, status = sa.build_union(dev["sel"], dev["sel_len"], 640, pt, 1,
                                                       n_pages)
    torch.cuda.synchronize()
    assert sa.status_value(status) == sa.STATUS_PAGE_RANGE
    c, r, n = cells.cpu().numpy(), rows.cpu().numpy(), length.cpu().numpy()
    on_page_2 = [r[g, i] for g in range(n.size) for i in range(n[g]) if c[g, i] // 64 == 2]
    assert on_page_2 and all(x == -1 for x in on_page_2)
    # a too-large v_scale
    vs = dev["v_scale"].clone()
    vs[int(d["page_table"][0])] = 8.0
    out, st = sa.prefill(dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], vs, rows, mask,
                         length, float(d["softmax_scale"]), 640)
    torch.cuda.synchronize()
    assert sa.status_value(st) == sa.STATUS_V_SCALE
    # a union length over the capacity is clamped and flagged (the entries past
    # the real union are whatever the buffer holds, so other flags may join it)
    bad_len = length.clone()
    bad_len[0] = cells.shape[1] + 1
    out, st = sa.prefill(dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                         dev["v_scale"], rows, mask, bad_len, float(d["softmax_scale"]), 640)
    torch.cuda.synchronize()
    assert sa.status_value(st) & sa.STATUS_UNION_LEN


# ------------------------------------------------ residency stress and replayed selections
@pytest.mark.parametrize("resident", [0.7, 0.05])
def test_attention_partially_resident_pool_full_size(resident):
    """The 32K chunk with a seeded share of its pages not resident (the page's
    untested residency option), in the benchmark's launch configuration;
    sampled groups against the oracle, rows without a resident cell output 0."""
    w = synth.workload(2)
    print("case resident", resident, flush=True)
    d = synth.as_problem(synth.generate(w))
    d["page_table"] = synth.drop_pages(d["page_table"], resident, seed=5)
    out, cells, mask, length, status = H.run_path(d)
    assert status == 0
    H.assert_union_equal(cells, mask, length, oracle.union(d["sel"], d["sel_len"], w.n_ctx))
    rows = H.sample_rows(w.n_q, 24, seed=4)
    H.assert_close(out[rows], oracle.attention_of(d, rows=rows), "resident %.2f" % resident)
    pt = d["page_table"]
    for j in rows:
        if not np.any(pt[d["sel"][j, :d["sel_len"][j]] // 64] >= 0):
            assert np.all(out[j] == 0)


def test_attention_replayed_selection_file(tmp_path):
    """Selections written to a file and read back (the page's replay of a
    selection dump); here the file holds the selection step's rows for
    AR(1) block scores, replayed over the 8K workload's pools."""
    from oracle import selection
    w = synth.workload(1)
    print("case replay", w.name, flush=True)
    scores = synth.block_scores(w.n_q, w.n_ctx, 0.95, seed=21)
    sel, sel_len = selection.select_blocks(scores, w.first_pos, w.n_ctx)
    path = str(tmp_path / "dump.npz")
    synth.save_selections(path, sel, sel_len, w.n_ctx, w.first_pos)
    rec = synth.load_selections(path)
    d = synth.as_problem(synth.generate(w, with_sel=False))
    d["sel"], d["sel_len"] = rec["sel"], rec["sel_len"]
    _check_problem(d, rows=H.sample_rows(w.n_q, 40, seed=6), what="replay " + w.name)
