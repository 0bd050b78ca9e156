"""Pins of the selection oracle (block scores -> selection rows).

Page cited: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
section What changed (the selection, block scores then top-k, comes before the
prompt attention) and the accuracy list in section Summary (a selection holds
at most 2,051 cells).
The page prints no example, so the oracle is pinned by
- a hand-worked fixture (ties, NaN, -0.0, sinks outside a dropped block 0,
  positions inside the first blocks);
- subset brute force: with distinct scores the 31 chosen blocks are the one
  31-subset with the largest score sum, found by enumerating every subset;
- closed forms: monotone scores choose the first or last 31 blocks, equal scores
  the first 31, and positions with at most 31 earlier blocks select [0, p];
- invariants on seeded workloads (sorted, distinct, causal, sinks and own
  block present, lengths, every chosen score >= every dropped one).
"""
import itertools
import math
import os

import numpy as np
import pytest

import synth
from oracle import selection as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_fixture():
    cases = []
    for line in open(os.path.join(GOLDEN, "selection_example.txt")):
        line = line.strip()
        if not line.startswith("case"):
            continue
        name, rest = line.split(":", 1)
        fields = dict(f.strip().split(" ", 1) if " " in f.strip() else (f.strip(), "")
                      for f in rest.split(";"))
        p = int(fields["p"])
        own = p // 64
        scores = np.full(max(own, 1), 0.5, np.float32)
        for item in fields["scores"].split():
            k, v = item.split("=")
            if k == "all":
                scores[:] = float(v)
            else:
                scores[int(k)] = np.float32(float(v))
        dropped = [int(x) for x in fields["dropped"].split()]
        cases.append((name, p, scores, dropped, int(fields["length"])))
    return cases


@pytest.mark.parametrize("case", _parse_fixture(), ids=lambda c: c[0])
def test_golden_fixture(case):
    name, p, scores, dropped, length = case
    row = S.selection_row(scores, p)
    own = p // 64
    kept = [b for b in range(own) if b not in dropped]
    expect = set(range(min(3, p + 1))) | {64 * b + i for b in kept for i in range(64)} \
        | set(range(64 * own, p + 1))
    assert row.size == length
    assert row.tolist() == sorted(expect)


@pytest.mark.parametrize("own,seed", [(32, 0), (33, 1), (34, 2), (35, 3)])
def test_top_blocks_maximise_the_score_sum(own, seed):
    """Distinct scores: the chosen set is the unique 31-subset of largest sum,
    found by enumerating the dropped blocks (every (own-31)-subset)."""
    rng = np.random.default_rng(seed)
    scores = rng.permutation(own).astype(np.float32) * np.float32(0.37) - np.float32(3)
    total = float(scores.astype(np.float64).sum())
    best, best_set = -math.inf, None
    for drop in itertools.combinations(range(own), own - 31):
        v = total - float(scores[list(drop)].astype(np.float64).sum())
        if v > best:
            best, best_set = v, sorted(set(range(own)) - set(drop))
    assert S.chosen_blocks(scores, own).tolist() == best_set


@pytest.mark.parametrize("own", [32, 40, 100, 511])
def test_monotone_and_equal_scores(own):
    up = np.arange(own, dtype=np.float32)
    assert S.chosen_blocks(up, own).tolist() == list(range(own - 31, own))
    assert S.chosen_blocks(-up, own).tolist() == list(range(31))
    assert S.chosen_blocks(np.zeros(own, np.float32), own).tolist() == list(range(31))


def test_positions_with_few_blocks_select_every_causal_cell():
    rng = np.random.default_rng(4)
    for p in list(range(0, 70)) + [127, 128, 1000, 2046, 2047]:
        row = S.selection_row(rng.standard_normal(64).astype(np.float32), p)
        assert row.tolist() == list(range(p + 1))
    # the first position with 32 earlier blocks is sparse: equal scores keep
    # blocks 0..30 (sinks inside block 0) and drop block 31
    row = S.selection_row(np.zeros(40, np.float32), 2048)
    assert row.tolist() == list(range(31 * 64)) + [2048]


@pytest.mark.parametrize("idx,rho,levels", [(2, 0.99, None), (4, 0.0, None), (1, 0.5, 3)])
def test_invariants_on_workloads(idx, rho, levels):
    w = synth.workload(idx)
    n_q = min(w.n_q, 300)
    first = w.n_ctx - n_q
    scores = synth.block_scores(n_q, w.n_ctx, rho, seed=7 + idx, levels=levels)
    sel, sel_len = S.select_blocks(scores, first, w.n_ctx)
    for j in range(n_q):
        p = first + j
        own = p // 64
        row = sel[j, :sel_len[j]]
        assert np.all(np.diff(row) > 0) and row[0] == 0 and row[-1] == p
        assert np.all(sel[j, sel_len[j]:] == -1)
        cells = set(row.tolist())
        assert {0, 1, 2} <= cells and set(range(64 * own, p + 1)) <= cells
        far = sorted({c // 64 for c in row.tolist() if 3 <= c < 64 * own} |
                     ({0} if 63 in cells else set()))
        assert len(far) == min(own, 31)
        # every far block is whole
        for b in far:
            assert set(range(64 * b, 64 * b + 64)) <= cells
        n_expect = (0 if 0 in far else 3) + 64 * len(far) + (p - 64 * own + 1)
        assert sel_len[j] == n_expect <= 2051
        if own > 31:
            s = scores[j, :own].astype(np.float64)
            dropped = sorted(set(range(own)) - set(far))
            assert s[far].min() >= s[dropped].max()


def test_rejects_bad_arguments():
    s = np.zeros((4, 8), np.float32)
    with pytest.raises(ValueError):
        S.select_blocks(s, 510, 512)
    with pytest.raises(ValueError):
        S.select_blocks(s, 0, 512, sel_cap=2050)
