"""Parity of the HIP selection step (block scores -> selection rows) with the CPU
oracle, bit-exact on every row and length, through the C ABI.

Page cited: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
section What changed (the selection, block scores then top-k, precedes the
prompt attention) and the accuracy list in section Summary (the selection cap
of 2,051).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import selection as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    name = torch.cuda.get_device_properties(0).gcnArchName
    if not name.startswith("gfx950"):
        pytest.skip("not gfx950: %s" % name)


import gpu_helpers as H  # noqa: E402
import oracle  # noqa: E402
import sparse_top_selection_amd as sa  # noqa: E402

SENTINEL = 0x5EEDF00D


def _run(scores: np.ndarray, first_pos: int, n_ctx: int, sel_cap: int = 2051):
    """GPU selection into outputs pre-filled with a sentinel; returns numpy."""
    n_q = scores.shape[0]
    sel = torch.full((n_q, sel_cap), SENTINEL, dtype=torch.int32, device="cuda")
    sel_len = torch.full((n_q,), -7, dtype=torch.int32, device="cuda")
    sa.select_blocks(torch.from_numpy(scores).cuda(), first_pos, n_ctx, out=(sel, sel_len))
    torch.cuda.synchronize()
    return sel.cpu().numpy(), sel_len.cpu().numpy()


def _check(scores, first_pos, n_ctx, sel_cap=2051):
    sel, sel_len = _run(scores, first_pos, n_ctx, sel_cap)
    ref, ref_len = S.select_blocks(scores, first_pos, n_ctx, sel_cap)
    bad_len = np.flatnonzero(sel_len != ref_len)
    assert bad_len.size == 0, ("lengths differ at", bad_len[:5], sel_len[bad_len[:5]],
                               ref_len[bad_len[:5]])
    valid = np.arange(sel_cap)[None, :] < ref_len[:, None]
    bad = np.argwhere(valid & (sel != ref))
    assert bad.size == 0, ("rows differ at (row, index)", bad[:5].tolist())
    # entries past each row's length are untouched
    assert np.all(sel[~valid] == SENTINEL)
    return sel, sel_len


@pytest.mark.parametrize("idx,rho,levels", [(0, 0.99, None), (1, 0.99, None), (2, 0.99, None),
                                            (3, 0.5, None), (4, 0.0, None), (2, 0.9, 3)])
def test_select_workloads_bit_exact(idx, rho, levels):
    """The five workloads' context lengths and positions; AR(1) scores from
    nearly shared (rho 0.99) to independent (rho 0), and integer scores with
    many exact ties."""
    w = synth.workload(idx)
    print("case", w.name, rho, levels, flush=True)
    scores = synth.block_scores(w.n_q, w.n_ctx, rho, seed=100 + idx, levels=levels)
    _check(scores, w.n_ctx - w.n_q, w.n_ctx)


def test_select_special_values():
    """NaN (either sign), +-inf, -0.0 next to +0.0, subnormals and runs of equal
    scores, scattered over the rows."""
    n_ctx, n_q = 20000, 700
    rng = np.random.default_rng(5)
    scores = synth.block_scores(n_q, n_ctx, 0.95, seed=6)
    specials = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-42, -1e-42, 1.0, 1.0],
                        np.float32)
    pick = rng.random(scores.shape) < 0.15
    scores[pick] = specials[rng.integers(0, specials.size, size=int(pick.sum()))]
    scores[::7, :] = np.float32(-0.0)      # whole rows of equal (signed) zeros
    scores[3::7, ::2] = np.float32(0.0)
    _check(scores, n_ctx - n_q, n_ctx)


def test_select_dense_to_sparse_positions_and_ragged_counts():
    """Positions from 0 through the first sparse block (own block 32 at p =
    2048) in one call, with a call size that is not a multiple of the four
    positions a work-group handles."""
    n_ctx = 5000
    scores = synth.block_scores(4001, n_ctx, 0.7, seed=8)
    sel, sel_len = _check(scores, 0, n_ctx)
    assert sel_len[:2048].tolist() == list(range(1, 2049))
    _check(scores[:3], 2045, n_ctx)


@pytest.mark.parametrize("n_ctx,n_q", [(262144, 37), (200001, 61), (131072, 45), (70000, 9)])
def test_select_long_contexts(n_ctx, n_q):
    """Contexts up to the entry point's limit (4,096 blocks, the largest slot
    count), positions at the end of the context."""
    print("case", n_ctx, n_q, flush=True)
    scores = synth.block_scores(n_q, n_ctx, 0.3, seed=n_q)
    _check(scores, n_ctx - n_q, n_ctx)


def test_select_larger_row_stride():
    """sel_cap above 2,051: rows keep their stride, padding stays untouched."""
    scores = synth.block_scores(50, 9000, 0.5, seed=9)
    _check(scores, 9000 - 50, 9000, sel_cap=2100)


def test_select_then_union_then_attention():
    """The selection feeds the path: selections from the GPU step, then the
    union and the attention, against the oracle's selection, union and
    attention."""
    w = synth.workload(1)
    print("case chain", w.name, flush=True)
    d = synth.as_problem(synth.generate(w))
    scores = synth.block_scores(w.n_q, w.n_ctx, 0.98, seed=11)
    ref_sel, ref_len = S.select_blocks(scores, w.n_ctx - w.n_q, w.n_ctx)
    sel, sel_len = sa.select_blocks(torch.from_numpy(scores).cuda(), w.n_ctx - w.n_q, w.n_ctx)
    d_gpu = dict(d)
    d_gpu["sel"], d_gpu["sel_len"] = sel.cpu().numpy(), sel_len.cpu().numpy()
    dev = H.to_device(d)
    dev["sel"], dev["sel_len"] = sel, sel_len
    out, cells, mask, length, status = H.run_path(d_gpu, dev)
    assert status == 0
    H.assert_union_equal(cells, mask, length, oracle.union(ref_sel, ref_len, w.n_ctx))
    d_ref = dict(d)
    d_ref["sel"], d_ref["sel_len"] = ref_sel, ref_len
    rows = H.sample_rows(w.n_q, 24, seed=3)
    H.assert_close(out[rows], oracle.attention_of(d_ref, rows=rows), "select+path " + w.name)
