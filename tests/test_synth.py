"""Generator checks: determinism, causality, caps and the selection recipe."""
import numpy as np
import pytest

import synth


def test_deterministic_bytes():
    w = synth.workload(0)
    a = synth.generate(w)
    b = synth.generate(w)
    for key in ("page_table", "k_pool", "v_pool", "k_scale", "v_scale", "q", "sel", "sel_len"):
        assert np.array_equal(a[key], b[key]), key


def test_streams_independent_of_skipped_parts():
    w = synth.workload(1)
    full = synth.generate(w)
    sel_only = synth.generate(w, with_q=False, with_pools=False)
    assert np.array_equal(full["sel"], sel_only["sel"])
    assert np.array_equal(full["page_table"], sel_only["page_table"])


@pytest.mark.parametrize("idx", range(5))
def test_selection_shape_and_causality(idx):
    w = synth.workload(idx)
    d = synth.generate(w, with_q=False, with_pools=False)
    sel, sel_len, pos = d["sel"], d["sel_len"], d["positions"]
    assert sel.shape == (w.n_q, 2051) and sel_len.shape == (w.n_q,)
    assert sel_len.min() >= 1 and sel_len.max() <= 2051
    cols = np.arange(sel.shape[1])[None, :]
    valid = cols < sel_len[:, None]
    assert np.all(sel[~valid] == -1)
    # every selected cell is causal: 0 <= c <= p
    assert np.all(sel[valid] >= 0)
    assert np.all(np.where(valid, sel, -1) <= pos[:, None])
    # a page table is a permutation of the pool's pages
    assert sorted(d["page_table"].tolist()) == list(range(w.pool_pages))
    # rows hold no repeated cells
    for j in range(0, w.n_q, max(1, w.n_q // 64)):
        row = sel[j, :sel_len[j]]
        assert np.unique(row).size == row.size
        if not w.shuffle_rows:
            assert np.all(np.diff(row) > 0)


def test_dense_workload_selects_every_causal_cell():
    w = synth.workload(0)
    d = synth.generate(w, with_q=False, with_pools=False)
    for j, p in enumerate(d["positions"]):
        assert d["sel_len"][j] == p + 1
        assert np.array_equal(d["sel"][j, :p + 1], np.arange(p + 1))


@pytest.mark.parametrize("idx", [1, 2, 4])
def test_sparse_selection_recipe(idx):
    """3 sinks + own partial block + 31 full causal blocks of 64."""
    w = synth.workload(idx)
    d = synth.generate(w, with_q=False, with_pools=False)
    for j in range(0, w.n_q, max(1, w.n_q // 97)):
        p = int(d["positions"][j])
        row = np.sort(d["sel"][j, :d["sel_len"][j]])
        own = p // 64
        assert {0, 1, 2} <= set(row.tolist())
        assert np.array_equal(row[row >= own * 64], np.arange(own * 64, p + 1))
        far = row[row < own * 64]
        blocks, counts = np.unique(far // 64, return_counts=True)
        full = blocks[counts == 64]
        assert full.size == 31
        # only block 0 may be partial (the sinks alone)
        partial = blocks[counts != 64]
        assert partial.size == 0 or (partial.tolist() == [0] and set(far[far < 64]) == {0, 1, 2})


def test_drift_statistics():
    """Neighbouring selections keep about (1 - drift) of their far blocks."""
    for idx, lo, hi in [(2, 0.90, 0.99), (3, 0.40, 0.60), (4, 0.0, 0.10)]:
        w = synth.workload(idx)
        d = synth.generate(w, with_q=False, with_pools=False)
        keep = []
        for j in range(1, min(w.n_q, 600)):
            a = set((d["sel"][j - 1, :d["sel_len"][j - 1]] // 64).tolist())
            b = set((d["sel"][j, :d["sel_len"][j]] // 64).tolist())
            keep.append(len(a & b) / len(a))
        m = float(np.mean(keep))
        assert lo <= m <= hi, (w.name, m)


def test_shuffled_rows_are_unsorted_sets():
    w = synth.workload(3)
    d = synth.generate(w, with_q=False, with_pools=False)
    n_unsorted = 0
    for j in range(0, w.n_q, 64):
        row = d["sel"][j, :d["sel_len"][j]]
        n_unsorted += int(np.any(np.diff(row) < 0))
        assert np.unique(row).size == row.size
    assert n_unsorted > 0


def test_small_random_edge_features():
    d = synth.small_random(7, n_ctx=700, n_q=37, n_kv=2, dup_frac=0.3, nonresident_frac=0.3)
    assert np.any(d["page_table"] == -1)
    dup_rows = sum(np.unique(d["sel"][j, :d["sel_len"][j]]).size < d["sel_len"][j]
                   for j in range(37))
    assert dup_rows > 0
    assert d["sel_len"].max() <= 2051


def test_block_scores_recipe():
    a = synth.block_scores(200, 5000, 0.9, seed=3)
    b = synth.block_scores(200, 5000, 0.9, seed=3)
    assert a.shape == (200, 79) and a.dtype == np.float32
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # AR(1): lag-1 correlation near rho, unit variance
    x, y = a[:-1].ravel().astype(np.float64), a[1:].ravel().astype(np.float64)
    assert abs(np.corrcoef(x, y)[0, 1] - 0.9) < 0.03
    assert abs(a.std() - 1.0) < 0.1
    t = synth.block_scores(50, 640, 0.0, seed=4, levels=3)
    assert set(np.unique(t).tolist()) <= {0.0, 1.0, 2.0}


def test_selection_file_round_trip(tmp_path):
    w = synth.workload(1)
    d = synth.generate(w, with_q=False, with_pools=False)
    path = str(tmp_path / "sel.npz")
    synth.save_selections(path, d["sel"], d["sel_len"], w.n_ctx, w.first_pos)
    rec = synth.load_selections(path)
    assert np.array_equal(rec["sel"], d["sel"]) and np.array_equal(rec["sel_len"], d["sel_len"])
    assert rec["n_ctx"] == w.n_ctx and rec["first_pos"] == w.first_pos
    # a non-causal entry is refused
    bad = d["sel"].copy()
    bad[0, 0] = w.first_pos + 1
    synth.save_selections(path, bad, d["sel_len"], w.n_ctx, w.first_pos)
    with pytest.raises(ValueError):
        synth.load_selections(path)


def test_drop_pages_fraction_and_seed():
    pt = np.random.default_rng(0).permutation(1000).astype(np.int32)
    a = synth.drop_pages(pt, 0.7, seed=3)
    b = synth.drop_pages(pt, 0.7, seed=3)
    assert np.array_equal(a, b) and np.count_nonzero(a == -1) == 300
    keep = a >= 0
    assert np.array_equal(a[keep], pt[keep])
