"""CPU oracle for the selection step: block scores -> per-position selection rows.

TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check in __graft_entry__ and
the CPU-baseline leg of bench.py may import it. The HIP path never calls it and
shares no code with it.

Page cited: #2808 "sycl: prompt attention over 8-query selection unions on XMX
(opt-in STRATA_PROMPT_ATTN_UNION=1)". Section What changed lists the selection
(block scores, then top-k) as the step that comes before the prompt attention,
which the page leaves unchanged. The accuracy list in section Summary gives the
selection layout's cap of 2,051 cells. The page does not say how blocks are scored, so the scores
are an input here.

Readings of what the page leaves open:
- A position p selects three sink cells {0, 1, 2}, its own block's causal cells
  [64*floor(p/64), p], and 31 of the full blocks before its own. That is
  3 + 31*64 + 64 = 2,051 cells at most, the cap.
- With at most 31 earlier blocks, it selects them all: the row is [0, p].
- Otherwise the 31 earlier blocks with the highest scores win.
  - Equal scores are ordered by the lower block index first.
  - A NaN score counts as -inf.
  - -0.0 and +0.0 are equal, as the comparison of floats has it.
- A row holds the selected cells once each, in ascending order.

This is the plain definition written out: a stable sort of the earlier blocks
by (score descending, index ascending), a cut at 31, and a sorted set union.
"""
from __future__ import annotations

import numpy as np

PAGE = 64          # cells per block (the page size)
N_SINKS = 3
N_TOP = 31         # blocks chosen besides the position's own
SEL_MAX = N_SINKS + N_TOP * PAGE + PAGE   # 2,051


def chosen_blocks(scores_row: np.ndarray, own: int) -> np.ndarray:
    """The earlier blocks a position with own block `own` selects, ascending."""
    if own <= N_TOP:
        return np.arange(own, dtype=np.int64)
    s = np.asarray(scores_row[:own], dtype=np.float64)
    s = np.where(np.isnan(s), -np.inf, s)
    idx = np.arange(own)
    order = np.lexsort((idx, -s))          # primary: score descending; then index
    return np.sort(order[:N_TOP])


def selection_row(scores_row: np.ndarray, p: int) -> np.ndarray:
    """Sorted selected cells of position p (int32)."""
    own = p // PAGE
    far = chosen_blocks(scores_row, own)
    parts = [np.arange(min(N_SINKS, p + 1)),
             (far[:, None] * PAGE + np.arange(PAGE)[None, :]).ravel(),
             np.arange(own * PAGE, p + 1)]
    return np.unique(np.concatenate(parts)).astype(np.int32)


def select_blocks(scores: np.ndarray, first_pos: int, n_ctx: int, sel_cap: int = SEL_MAX):
    """Selections of positions first_pos .. first_pos + n_q - 1.

    scores: float32 [n_q][ceil(n_ctx/64)]; row j scores the blocks before
    position first_pos + j's own block (later entries are ignored).
    Returns (sel int32 [n_q][sel_cap] padded with -1, sel_len int32 [n_q]).
    """
    n_q = scores.shape[0]
    if first_pos < 0 or first_pos + n_q > n_ctx:
        raise ValueError("positions must lie in [0, n_ctx)")
    if sel_cap < SEL_MAX:
        raise ValueError("sel_cap must hold %d cells" % SEL_MAX)
    sel = np.full((n_q, sel_cap), -1, np.int32)
    sel_len = np.zeros(n_q, np.int32)
    for j in range(n_q):
        row = selection_row(scores[j], first_pos + j)
        sel[j, :row.size] = row
        sel_len[j] = row.size
    return sel, sel_len
