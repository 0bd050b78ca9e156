"""Pins of the CPU oracle to things other than itself.

Page cited: #2808 "sycl: prompt attention over 8-query selection unions on XMX".
The page prints no input/output values, so the oracle is pinned by
- a dense brute force written in matrix form (scores for every cell of the
  context, a boolean selection matrix, a row softmax), which shares no code
  and no formulation with the oracle's per-position gather;
- closed forms (single cell, K = 0, constant V, two cells);
- invariances the definition implies (order, duplicates, page permutation,
  non-resident pages);
- for the union: Python-set brute force, a hand-worked fixture, and the closed
  form of the dense workload.
A plausible mistake in the oracle (a dropped scale, a wrong head index, a
transposed operand, a missing dedupe, residency ignored, a wrong mask bit)
fails at least one test here.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# dense brute force (matrix form), written independently of the oracle
# --------------------------------------------------------------------------
def dense_bruteforce(d):
    n_ctx, n_q, n_kv = d["n_ctx"], d["n_q"], d["n_kv"]
    pt = d["page_table"]
    n_qh = d["q"].shape[1]
    q_per_kv = n_qh // n_kv
    cells = np.arange(n_ctx)
    phys = pt[cells // 64]
    resident = phys >= 0
    ph = np.where(resident, phys, 0)
    # K_full[kv, c, :] = dequantised key of logical cell c (zero when not resident)
    k_full = (d["k_pool"][ph, :, cells % 64, :].astype(np.float64)
              * d["k_scale"][ph, :, cells % 64][:, :, None].astype(np.float64))
    v_full = (d["v_pool"][ph, :, cells % 64, :].astype(np.float64)
              * d["v_scale"][ph, :, cells % 64][:, :, None].astype(np.float64))
    k_full = np.transpose(k_full, (1, 0, 2))       # [kv][c][d]
    v_full = np.transpose(v_full, (1, 0, 2))
    allowed = np.zeros((n_q, n_ctx), bool)
    for j in range(n_q):
        allowed[j, d["sel"][j, :d["sel_len"][j]]] = True
    allowed &= resident[None, :]
    out = np.zeros((n_q, n_qh, d["q"].shape[2]))
    scale = float(np.float32(d["softmax_scale"]))
    for h in range(n_qh):
        kv = h // q_per_kv
        s = scale * (d["q"][:, h, :].astype(np.float64) @ k_full[kv].T)   # [n_q][n_ctx]
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        w = np.exp(s - m)
        z = w.sum(axis=1, keepdims=True)
        p = np.divide(w, z, out=np.zeros_like(w), where=z > 0)
        out[:, h, :] = p @ v_full[kv]
    return out


def test_dense_workload_matches_bruteforce():
    d = synth.as_problem(synth.generate(synth.workload(0)))
    ref = dense_bruteforce(d)
    got = oracle.attention_of(d)
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("seed,n_kv,dup,nonres", [(1, 2, 0.3, 0.25), (2, 4, 0.0, 0.0),
                                                 (3, 3, 0.5, 0.5)])
def test_random_selections_match_bruteforce(seed, n_kv, dup, nonres):
    d = synth.small_random(seed, n_ctx=900, n_q=29, n_kv=n_kv, dup_frac=dup,
                           nonresident_frac=nonres, pool_extra=3)
    ref = dense_bruteforce(d)
    got = oracle.attention_of(d)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_head_mapping_is_contiguous_blocks_of_12():
    """Query head h reads KV head h // 12: zero every KV head but one."""
    d = synth.small_random(11, n_ctx=300, n_q=5, n_kv=3)
    d["v_pool"][:, [0, 2]] = 0
    got = oracle.attention_of(d)
    assert np.all(got[:, :12] == 0) and np.all(got[:, 24:] == 0)
    assert np.all(np.any(got[:, 12:24] != 0, axis=-1)[d["sel_len"] > 0])


def _one_cell_problem(seed=5):
    d = synth.small_random(seed, n_ctx=256, n_q=6, n_kv=2)
    rng = np.random.default_rng(seed)
    d["sel"][:] = -1
    for j in range(6):
        c = int(rng.integers(0, 256))
        d["sel"][j, 0] = c
        d["sel_len"][j] = 1
    return d


def test_single_cell_returns_dequantised_v():
    d = _one_cell_problem()
    got = oracle.attention_of(d)
    for j in range(d["n_q"]):
        c = d["sel"][j, 0]
        pp = d["page_table"][c // 64]
        for h in range(24):
            kv = h // 12
            v = d["v_pool"][pp, kv, c % 64].astype(np.float64) * float(d["v_scale"][pp, kv, c % 64])
            assert np.array_equal(got[j, h], v)


def test_zero_keys_give_plain_mean_of_values():
    d = synth.small_random(6, n_ctx=500, n_q=9, n_kv=2, nonresident_frac=0.2)
    d["k_pool"][:] = 0
    got = oracle.attention_of(d)
    for j in range(d["n_q"]):
        cells = np.unique(d["sel"][j, :d["sel_len"][j]])
        pp = d["page_table"][cells // 64]
        cells, pp = cells[pp >= 0], pp[pp >= 0]
        for kv in range(2):
            if cells.size == 0:
                assert np.all(got[j, kv * 12:(kv + 1) * 12] == 0)
                continue
            v = (d["v_pool"][pp, kv, cells % 64].astype(np.float64)
                 * d["v_scale"][pp, kv, cells % 64][:, None].astype(np.float64))
            mean = v.mean(axis=0)
            for h in range(kv * 12, (kv + 1) * 12):
                assert np.allclose(got[j, h], mean, rtol=1e-13, atol=1e-16)


def test_constant_values_show_probabilities_sum_to_one():
    d = synth.small_random(8, n_ctx=640, n_q=12, n_kv=1)
    d["v_pool"][:] = 37
    d["v_scale"][:] = np.float32(0.015625)
    got = oracle.attention_of(d)
    nonempty = d["sel_len"] > 0
    assert np.all(np.abs(got[nonempty] - 37 * 0.015625) <= 1e-13)
    assert np.all(got[~nonempty] == 0)


def test_two_cells_closed_form():
    """out = v1 * sigmoid(s1 - s2) + v2 * sigmoid(s2 - s1), written by hand."""
    d = synth.small_random(9, n_ctx=128, n_q=1, n_kv=1)
    d["sel"][:] = -1
    d["sel"][0, :2] = [3, 70]
    d["sel_len"][0] = 2
    d["q"][:] = 0
    d["q"][0, 0, 0] = 1.5
    d["q"][0, 0, 1] = -2.0
    d["k_pool"][:] = 0
    d["v_pool"][:] = 0
    pt = d["page_table"]
    p3, p70 = pt[0], pt[1]
    d["k_pool"][p3, 0, 3, :2] = [10, 4]
    d["k_pool"][p70, 0, 6, :2] = [-5, 20]
    d["k_scale"][p3, 0, 3] = np.float32(0.5)
    d["k_scale"][p70, 0, 6] = np.float32(0.25)
    d["v_pool"][p3, 0, 3, 0] = 100
    d["v_pool"][p70, 0, 6, 0] = -60
    d["v_scale"][p3, 0, 3] = np.float32(0.125)
    d["v_scale"][p70, 0, 6] = np.float32(0.0625)
    sc = float(np.float32(1 / math.sqrt(128)))
    s1 = sc * (1.5 * 10 * 0.5 + (-2.0) * 4 * 0.5)
    s2 = sc * (1.5 * -5 * 0.25 + (-2.0) * 20 * 0.25)
    w1 = 1 / (1 + math.exp(s2 - s1))
    w2 = 1 / (1 + math.exp(s1 - s2))
    expect0 = 100 * 0.125 * w1 + (-60) * 0.0625 * w2
    got = oracle.attention_of(d)
    assert abs(got[0, 0, 0] - expect0) <= 1e-14
    assert np.all(got[0, 0, 1:] == 0)


def test_selection_order_and_duplicates_do_not_matter():
    d = synth.small_random(10, n_ctx=800, n_q=17, n_kv=2, shuffle=False)
    base = oracle.attention_of(d)
    rng = np.random.default_rng(0)
    e = dict(d)
    e["sel"] = d["sel"].copy()
    e["sel_len"] = d["sel_len"].copy()
    for j in range(d["n_q"]):
        n = d["sel_len"][j]
        row = rng.permutation(d["sel"][j, :n])
        extra = min(2051 - n, n)
        dup = rng.choice(row, size=extra) if n else np.zeros(0, np.int32)
        row = rng.permutation(np.concatenate([row, dup]))
        e["sel"][j, :row.size] = row
        e["sel_len"][j] = row.size
    got = oracle.attention_of(e)
    assert np.array_equal(got, base)


def test_nonresident_page_equals_deleting_its_cells():
    d = synth.small_random(12, n_ctx=1024, n_q=13, n_kv=2)
    off_pages = [2, 5, 11]
    a = dict(d)
    a["page_table"] = d["page_table"].copy()
    a["page_table"][off_pages] = -1
    b = dict(d)
    b["sel"] = np.full_like(d["sel"], -1)
    b["sel_len"] = np.zeros_like(d["sel_len"])
    for j in range(d["n_q"]):
        row = d["sel"][j, :d["sel_len"][j]]
        row = row[~np.isin(row // 64, off_pages)]
        b["sel"][j, :row.size] = row
        b["sel_len"][j] = row.size
    assert np.array_equal(oracle.attention_of(a), oracle.attention_of(b))


def test_page_permutation_invariance():
    d = synth.small_random(13, n_ctx=768, n_q=11, n_kv=2, pool_extra=4)
    perm = np.random.default_rng(1).permutation(d["n_pages"])  # new slot of old page
    e = dict(d)
    for key in ("k_pool", "v_pool", "k_scale", "v_scale"):
        arr = np.empty_like(d[key])
        arr[perm] = d[key]
        e[key] = arr
    e["page_table"] = np.where(d["page_table"] >= 0, perm[np.maximum(d["page_table"], 0)], -1)
    e["page_table"] = e["page_table"].astype(np.int32)
    assert np.array_equal(oracle.attention_of(e), oracle.attention_of(d))


def test_empty_selection_outputs_zero():
    d = synth.small_random(14, n_ctx=200, n_q=4, n_kv=1)
    d["sel_len"][1] = 0
    d["sel_len"][3] = 0
    got = oracle.attention_of(d)
    assert np.all(got[[1, 3]] == 0)


def test_rows_subset_matches_full():
    d = synth.small_random(15, n_ctx=600, n_q=21, n_kv=2)
    full = oracle.attention_of(d)
    rows = [20, 0, 7, 7, 13]
    assert np.array_equal(oracle.attention_of(d, rows=rows), full[rows])


def test_invalid_cell_is_rejected():
    d = synth.small_random(16, n_ctx=200, n_q=3, n_kv=1)
    d["sel"][1, 0] = 200
    d["sel_len"][1] = max(1, d["sel_len"][1])
    with pytest.raises(ValueError):
        oracle.attention_of(d)
    with pytest.raises(ValueError):
        oracle.union(d["sel"], d["sel_len"], 200)


# --------------------------------------------------------------------------
# union
# --------------------------------------------------------------------------
def union_bruteforce(sel, sel_len):
    """Python sets: the definition in its most literal form."""
    n_q = sel.shape[0]
    groups = []
    for g in range((n_q + 7) // 8):
        chooser = {}
        for i in range(min(8, n_q - 8 * g)):
            j = 8 * g + i
            for c in set(sel[j, :sel_len[j]].tolist()):
                chooser[c] = chooser.get(c, 0) | (1 << i)
        groups.append(sorted(chooser.items()))
    return groups


def _check_union(sel, sel_len, n_ctx):
    cells, mask, length = oracle.union(sel, sel_len, n_ctx)
    ref = union_bruteforce(sel, sel_len)
    for g, items in enumerate(ref):
        assert length[g] == len(items)
        assert cells[g, :length[g]].tolist() == [c for c, _ in items]
        assert mask[g, :length[g]].tolist() == [m for _, m in items]


def test_union_golden_fixture():
    lines = [l.strip() for l in open(os.path.join(GOLDEN, "union_example.txt"))
             if l.strip() and not l.startswith("#")]
    rows = [list(map(int, l.split(":")[1].split())) for l in lines if l.startswith("sel")]
    expect = [tuple(map(int, t.split(":"))) for t in
              [l for l in lines if l.startswith("union:")][0].split(":", 1)[1].split()]
    sel = np.full((len(rows), 4), -1, np.int32)
    sel_len = np.zeros(len(rows), np.int32)
    for j, r in enumerate(rows):
        sel[j, :len(r)] = r
        sel_len[j] = len(r)
    cells, mask, length = oracle.union(sel, sel_len, 16)
    assert length.tolist() == [len(expect)]
    assert list(zip(cells[0, :length[0]].tolist(), mask[0, :length[0]].tolist())) == expect


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_union_matches_set_bruteforce(seed):
    d = synth.small_random(seed, n_ctx=5000, n_q=45, n_kv=1, dup_frac=0.4)
    _check_union(d["sel"], d["sel_len"], 5000)


def test_union_dense_workload_closed_form():
    """All causal cells selected: U_g = [0, p_max], bit i set iff c <= p_i."""
    w = synth.workload(0)
    d = synth.generate(w, with_q=False, with_pools=False)
    cells, mask, length = oracle.union(d["sel"], d["sel_len"], w.n_ctx)
    pos = d["positions"]
    for g in range(w.n_groups):
        ps = pos[8 * g: 8 * g + 8]
        assert length[g] == ps.max() + 1
        c = np.arange(ps.max() + 1)
        assert np.array_equal(cells[g, :length[g]], c)
        expect = np.zeros(c.size, np.int64)
        for i, p in enumerate(ps):
            expect |= (c <= p).astype(np.int64) << i
        assert np.array_equal(mask[g, :length[g]].astype(np.int64), expect)


@pytest.mark.parametrize("idx", [1, 3])
def test_union_invariants(idx):
    w = synth.workload(idx)
    d = synth.generate(w, with_q=False, with_pools=False)
    cells, mask, length = oracle.union(d["sel"], d["sel_len"], w.n_ctx)
    for g in range(0, w.n_groups, max(1, w.n_groups // 50)):
        u = cells[g, :length[g]]
        m = mask[g, :length[g]]
        assert np.all(np.diff(u) > 0)
        assert np.all(m != 0)
        n_pos = min(8, w.n_q - 8 * g)
        assert np.all(m < (1 << n_pos))
        pop = sum(int(bin(x).count("1")) for x in m.tolist())
        assert pop == int(d["sel_len"][8 * g: 8 * g + n_pos].sum())
        for i in range(n_pos):
            j = 8 * g + i
            assert set(u[(m >> i) & 1 == 1].tolist()) == set(d["sel"][j, :d["sel_len"][j]].tolist())


def test_union_identical_rows_and_ragged_group():
    sel = np.full((11, 6), -1, np.int32)
    sel[:, :4] = [9, 2, 40, 2]
    sel_len = np.full(11, 4, np.int32)
    cells, mask, length = oracle.union(sel, sel_len, 64)
    assert length.tolist() == [3, 3]
    assert cells[0, :3].tolist() == [2, 9, 40] and cells[1, :3].tolist() == [2, 9, 40]
    assert mask[0, :3].tolist() == [0xFF] * 3
    assert mask[1, :3].tolist() == [0b111] * 3


def test_union_empty_rows():
    sel = np.full((8, 3), -1, np.int32)
    sel_len = np.zeros(8, np.int32)
    sel[5, :2] = [7, 1]
    sel_len[5] = 2
    cells, mask, length = oracle.union(sel, sel_len, 10)
    assert length.tolist() == [2]
    assert cells[0, :2].tolist() == [1, 7] and mask[0, :2].tolist() == [32, 32]


# --------------------------------------------------------------------------
# union rows (each union cell resolved through the page table once)
# --------------------------------------------------------------------------
def test_union_rows_golden_fixture():
    lines = [l.strip() for l in open(os.path.join(GOLDEN, "union_rows_example.txt"))
             if l.strip() and not l.startswith("#")]
    field = {l.split(":")[0]: list(map(int, l.split(":")[1].split())) for l in lines}
    cells = np.array([field["cells"]], np.int32)
    length = np.array([len(field["cells"])], np.int32)
    rows, flags = oracle.union_rows(cells, length, np.array(field["page_table"], np.int32),
                                    n_kv=2, n_pages=8)
    assert rows[0].tolist() == field["rows"]
    assert flags == field["flags"][0]


@pytest.mark.parametrize("seed,n_kv,nonres", [(0, 1, 0.0), (1, 3, 0.3), (2, 4, 0.6)])
def test_union_rows_address_the_cells_pool_entries(seed, n_kv, nonres):
    """Flattened to rows, each pool and scale array holds cell c of KV head h at
    union row + 64 h: the same bytes as indexing the pool by (page, head, slot);
    rows of non-resident pages are -1, and only they."""
    d = synth.small_random(seed, n_ctx=3000, n_q=21, n_kv=n_kv, dup_frac=0.2,
                           nonresident_frac=nonres, pool_extra=2)
    cells, mask, length = oracle.union(d["sel"], d["sel_len"], d["n_ctx"])
    n_pages = d["k_pool"].shape[0]
    rows, flags = oracle.union_rows(cells, length, d["page_table"], n_kv, n_pages)
    assert flags == 0
    flat = {k: d[k].reshape(n_pages * n_kv * 64, -1) for k in ("k_pool", "v_pool")}
    flat_s = {k: d[k].reshape(-1) for k in ("k_scale", "v_scale")}
    checked = 0
    for g in range(length.size):
        for c, r in zip(cells[g, :length[g]].tolist(), rows[g, :length[g]].tolist()):
            page = int(d["page_table"][c // 64])
            assert (r == -1) == (page == -1)
            if page < 0:
                continue
            for h in range(n_kv):
                for k in ("k_pool", "v_pool"):
                    assert np.array_equal(flat[k][r + 64 * h], d[k][page, h, c % 64])
                for k in ("k_scale", "v_scale"):
                    assert flat_s[k][r + 64 * h] == d[k][page, h, c % 64]
                checked += 1
    assert checked > 100
    assert nonres == 0.0 or (rows[rows != 0] == -1).any()
