"""Seeded synthetic workloads for prompt-phase selection attention over INT8 paged K/V.

This module only draws inputs: page tables, INT8 K/V pools with per-cell scales,
queries and per-position selection lists. It holds none of the method's
arithmetic (no union, no scores, no softmax), so both the CPU oracle's tests and
the HIP path's tests and benchmark can use it.

Page cited throughout: #2808 "sycl: prompt attention over 8-query selection
unions on XMX (opt-in STRATA_PROMPT_ATTN_UNION=1)".

Shapes the page fixes (the accuracy list in section Summary, the parity
self-test): random INT8
pools behind a shuffled page table, the prompt path's selection layout with a
cap of 2,051 cells, contexts from 1.5K to 40K, ragged last groups, pages that
are not resident. The page measures on a private model and private chats; these
seeded inputs stand in for them.

Readings of what the page leaves open (each is also listed in the design notes):
- A selection is 3 sink cells {0, 1, 2}, the position's own partial block
  [64*floor(p/64), p], and 31 further causal blocks of 64 cells from
  [0, floor(p/64)). While a position has at most 32 causal blocks it selects all
  of its causal cells (at most 2,048 <= cap), and a dense workload always does.
- "Chosen by seeded scores": the first position's 31 blocks are the top 31 of
  seeded uniform scores over its causal blocks, i.e. a uniform random subset.
- "Drift d": from one position to the next every block choice is kept with
  probability 1 - d; the dropped ones are refilled uniformly from the causal
  blocks not already kept. Drift 1.0 draws every position independently.
- Rows are emitted sorted (ascending) unless the workload asks for shuffled
  rows; padding past sel_len is -1.

Memory layout (the library's layout, see include/sel_attn.h):
  k_pool, v_pool  int8    [n_pages][n_kv][page_size][head_dim]
  k_scale, v_scale float32 [n_pages][n_kv][page_size]
  page_table      int32   [ceil(n_ctx / page_size)]  (-1 = page not resident)
  q               float32 [n_q][n_kv * q_per_kv][head_dim]
  sel             int32   [n_q][sel_cap],  sel_len int32 [n_q]
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

SEL_CAP = 2051          # 3 sinks + 32 blocks of 64 cells
PAGE_SIZE = 64
HEAD_DIM = 128
Q_PER_KV = 12
N_SINKS = 3
N_FAR_BLOCKS = 31       # blocks chosen besides the position's own block


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload. Query index j sits at position first_pos + j."""
    name: str
    n_ctx: int
    n_q: int
    n_kv: int
    drift: Optional[float]          # None = dense causal selection
    scale_lo: float = 0.005
    scale_hi: float = 0.02
    shuffle_rows: bool = False
    seed: int = 1000
    n_pages: Optional[int] = None   # physical pool size; default ceil(n_ctx / 64)
    q_per_kv: int = Q_PER_KV
    head_dim: int = HEAD_DIM
    page_size: int = PAGE_SIZE
    sel_cap: int = SEL_CAP

    @property
    def first_pos(self) -> int:
        return self.n_ctx - self.n_q

    @property
    def n_qh(self) -> int:
        return self.n_kv * self.q_per_kv

    @property
    def n_logical_pages(self) -> int:
        return -(-self.n_ctx // self.page_size)

    @property
    def pool_pages(self) -> int:
        return self.n_pages if self.n_pages is not None else self.n_logical_pages

    @property
    def n_groups(self) -> int:
        return -(-self.n_q // 8)


# The five workloads of the parity self-test and the headline measurement.
WORKLOADS = (
    # 1,536 cells, last 250 positions (ragged last group of 2), dense causal.
    Workload("ctx1536_dense", n_ctx=1536, n_q=250, n_kv=1, drift=None, seed=1000),
    # 8,192 cells, last 1,024 positions, drift 0.05.
    Workload("ctx8k_drift005", n_ctx=8192, n_q=1024, n_kv=4, drift=0.05, seed=1001),
    # 32,768 cells, one 8,192-position prompt chunk (24,576..32,767), drift 0.05.
    Workload("ctx32k_drift005", n_ctx=32768, n_q=8192, n_kv=4, drift=0.05, seed=1002),
    # 40,960 cells, 8,190 positions ending at the context end (last group of 6),
    # drift 0.5, rows shuffled.
    Workload("ctx40k_drift05_shuffled", n_ctx=40960, n_q=8190, n_kv=4, drift=0.5,
             shuffle_rows=True, seed=1003),
    # 65,536 cells, last 4,096 positions, independent selections, wider scales.
    Workload("ctx64k_independent", n_ctx=65536, n_q=4096, n_kv=4, drift=1.0,
             scale_lo=0.002, scale_hi=0.05, seed=1004),
)

HEADLINE = 2   # the 32K-context prompt chunk


def workload(index_or_name) -> Workload:
    if isinstance(index_or_name, int):
        return WORKLOADS[index_or_name]
    for w in WORKLOADS:
        if w.name == index_or_name:
            return w
    raise KeyError(index_or_name)


def _selection_rows(rng: np.random.Generator, w: Workload, positions: np.ndarray):
    """Per-position selected cells, as a list of int32 arrays (sorted, unique)."""
    rows = []
    chosen = None                       # block indices chosen besides the own block
    for p in positions:
        p = int(p)
        own = p // w.page_size
        if w.drift is None or own <= N_FAR_BLOCKS:
            rows.append(np.arange(p + 1, dtype=np.int32))
            chosen = None
            continue
        if chosen is None:
            scores = rng.random(own)
            chosen = np.argsort(-scores, kind="stable")[:N_FAR_BLOCKS]
        else:
            kept = chosen[rng.random(chosen.size) >= w.drift]
            free = np.setdiff1d(np.arange(own), kept, assume_unique=False)
            refill = rng.choice(free, N_FAR_BLOCKS - kept.size, replace=False)
            chosen = np.concatenate([kept, refill])
        cells = np.concatenate([
            np.arange(N_SINKS),
            (chosen[:, None] * w.page_size + np.arange(w.page_size)[None, :]).ravel(),
            np.arange(own * w.page_size, p + 1),
        ])
        rows.append(np.unique(cells).astype(np.int32))
    return rows


def generate(w: Workload, with_q: bool = True, with_pools: bool = True,
             with_sel: bool = True) -> dict:
    """Draw every input of one workload from SeedSequence(w.seed).

    Streams, in order: page table, K/V pools, scales, q, selections. Skipping the
    pools, q or the selections (for tests that only need the rest, or a replay
    that brings its own selections) leaves the other streams unchanged because
    each stream is spawned separately.
    """
    ss = np.random.SeedSequence(w.seed).spawn(5)
    r_pt, r_kv, r_sc, r_q, r_sel = (np.random.default_rng(s) for s in ss)
    out = {"workload": w}

    n_lp = w.n_logical_pages
    assert w.pool_pages >= n_lp
    out["page_table"] = r_pt.permutation(w.pool_pages)[:n_lp].astype(np.int32)

    if with_pools:
        shape = (w.pool_pages, w.n_kv, w.page_size, w.head_dim)
        out["k_pool"] = r_kv.integers(-127, 128, size=shape, dtype=np.int8)
        out["v_pool"] = r_kv.integers(-127, 128, size=shape, dtype=np.int8)
        sshape = (w.pool_pages, w.n_kv, w.page_size)
        out["k_scale"] = r_sc.uniform(w.scale_lo, w.scale_hi, size=sshape).astype(np.float32)
        out["v_scale"] = r_sc.uniform(w.scale_lo, w.scale_hi, size=sshape).astype(np.float32)
    if with_q:
        out["q"] = r_q.standard_normal((w.n_q, w.n_qh, w.head_dim), dtype=np.float32)

    positions = np.arange(w.first_pos, w.n_ctx)
    out["positions"] = positions.astype(np.int64)
    out["softmax_scale"] = np.float32(1.0 / math.sqrt(w.head_dim))
    if not with_sel:
        return out
    rows = _selection_rows(r_sel, w, positions)
    sel = np.full((w.n_q, w.sel_cap), -1, dtype=np.int32)
    sel_len = np.zeros(w.n_q, dtype=np.int32)
    for j, cells in enumerate(rows):
        if w.shuffle_rows:
            cells = r_sel.permutation(cells)
        sel[j, :cells.size] = cells
        sel_len[j] = cells.size
    out["sel"] = sel
    out["sel_len"] = sel_len
    return out


def small_random(seed: int, n_ctx: int, n_q: int, n_kv: int, sel_cap: int = SEL_CAP,
                 max_len: Optional[int] = None, shuffle: bool = True,
                 dup_frac: float = 0.0, nonresident_frac: float = 0.0,
                 scale_lo: float = 0.005, scale_hi: float = 0.02,
                 pool_extra: int = 0) -> dict:
    """Small inputs with arbitrary (non block-structured) causal selections.

    Each row draws a random subset of its causal cells [0, p] with a random
    length, optionally with duplicate entries and in random order, and a random
    fraction of logical pages is marked not resident (-1). Used for edge-case
    parity tests at sizes the oracle finishes in moments.
    """
    rng = np.random.default_rng(seed)
    n_lp = -(-n_ctx // PAGE_SIZE)
    n_pages = n_lp + pool_extra
    page_table = rng.permutation(n_pages)[:n_lp].astype(np.int32)
    if nonresident_frac > 0:
        off = rng.random(n_lp) < nonresident_frac
        page_table[off] = -1
    shape = (n_pages, n_kv, PAGE_SIZE, HEAD_DIM)
    k_pool = rng.integers(-127, 128, size=shape, dtype=np.int8)
    v_pool = rng.integers(-127, 128, size=shape, dtype=np.int8)
    k_scale = rng.uniform(scale_lo, scale_hi, size=shape[:3]).astype(np.float32)
    v_scale = rng.uniform(scale_lo, scale_hi, size=shape[:3]).astype(np.float32)
    q = rng.standard_normal((n_q, n_kv * Q_PER_KV, HEAD_DIM), dtype=np.float32)
    positions = np.arange(n_ctx - n_q, n_ctx)
    cap = sel_cap if max_len is None else min(sel_cap, max_len)
    sel = np.full((n_q, sel_cap), -1, dtype=np.int32)
    sel_len = np.zeros(n_q, dtype=np.int32)
    for j, p in enumerate(positions):
        n_causal = int(p) + 1
        n_dup = 0
        length = int(rng.integers(0, min(cap, n_causal) + 1))
        if dup_frac > 0 and length > 0:
            n_dup = min(int(rng.integers(0, int(length * dup_frac) + 1)), cap - length)
        cells = rng.choice(n_causal, size=length, replace=False)
        if n_dup:
            cells = np.concatenate([cells, rng.choice(cells, size=n_dup)])
        if not shuffle:
            cells = np.sort(cells)
        else:
            cells = rng.permutation(cells)
        sel[j, :cells.size] = cells
        sel_len[j] = cells.size
    return dict(page_table=page_table, k_pool=k_pool, v_pool=v_pool, k_scale=k_scale,
                v_scale=v_scale, q=q, sel=sel, sel_len=sel_len, positions=positions,
                softmax_scale=np.float32(1.0 / math.sqrt(HEAD_DIM)), n_ctx=n_ctx,
                n_q=n_q, n_kv=n_kv, n_pages=n_pages, sel_cap=sel_cap)


def as_problem(inputs: dict) -> dict:
    """Flatten a generate() result into the same keys small_random() returns."""
    w = inputs.get("workload")
    if w is None:
        return inputs
    d = dict(inputs)
    d.update(n_ctx=w.n_ctx, n_q=w.n_q, n_kv=w.n_kv, n_pages=w.pool_pages, sel_cap=w.sel_cap)
    return d


def block_scores(n_q: int, n_ctx: int, rho: float, seed: int,
                 levels: Optional[int] = None) -> np.ndarray:
    """Seeded per-position block scores for the selection step.

    float32 [n_q][ceil(n_ctx/64)]. The page does not say how blocks are scored,
    so these stand in for the model's scores:
    - each block's score follows a Gaussian AR(1) walk over the positions,
      s_j = rho * s_(j-1) + sqrt(1 - rho^2) * e_j;
    - rho near 1 gives neighbouring positions nearly the same top blocks,
      while rho = 0 draws every position independently;
    - with `levels`, scores are quantised to the integers 0 .. levels-1,
      which gives many exact ties.
    Row j scores every block; the selection reads only the blocks before the
    position's own block.
    """
    rng = np.random.default_rng(seed)
    nb = -(-n_ctx // PAGE_SIZE)
    out = np.empty((n_q, nb), np.float32)
    s = rng.standard_normal(nb)
    c = math.sqrt(max(0.0, 1.0 - rho * rho))
    for j in range(n_q):
        if j:
            s = rho * s + c * rng.standard_normal(nb)
        out[j] = s
    if levels is not None:
        out = np.floor((out + 3.0) * (levels / 6.0)).clip(0, levels - 1).astype(np.float32)
    return out


# ----------------------------------------------------------------------------
# Recorded selections and partial residency. The page's timing tool replays a
# selection dump and its notes name a partly resident KV pool as untested
# (section What changed, the parity test's arguments; section Extra Notes).
# No dump from a real model is available here, so files are written from the
# generators above; the format is plain arrays that numpy reads without pickle.
# ----------------------------------------------------------------------------
def save_selections(path: str, sel: np.ndarray, sel_len: np.ndarray, n_ctx: int,
                    first_pos: int) -> None:
    """Write selections as an .npz: sel int32 [n_q][cap], sel_len int32 [n_q],
    n_ctx and first_pos (query index j is at position first_pos + j)."""
    np.savez(path, sel=np.ascontiguousarray(sel, np.int32),
             sel_len=np.ascontiguousarray(sel_len, np.int32),
             n_ctx=np.int64(n_ctx), first_pos=np.int64(first_pos))


def load_selections(path: str) -> dict:
    """Read a file written by save_selections (no pickle) and check its shapes
    and ranges: lengths in [0, cap], entries in [0, n_ctx), entries causal."""
    with np.load(path, allow_pickle=False) as f:
        sel = np.ascontiguousarray(f["sel"], np.int32)
        sel_len = np.ascontiguousarray(f["sel_len"], np.int32)
        n_ctx = int(f["n_ctx"])
        first_pos = int(f["first_pos"])
    if sel.ndim != 2 or sel_len.shape != (sel.shape[0],):
        raise ValueError("sel must be [n_q][cap] and sel_len [n_q]")
    n_q, cap = sel.shape
    if first_pos < 0 or first_pos + n_q > n_ctx:
        raise ValueError("positions outside [0, n_ctx)")
    if np.any(sel_len < 0) or np.any(sel_len > cap):
        raise ValueError("a length outside [0, cap]")
    valid = np.arange(cap)[None, :] < sel_len[:, None]
    pos = (first_pos + np.arange(n_q))[:, None]
    if np.any(valid & ((sel < 0) | (sel > pos))):
        raise ValueError("an entry outside [0, p]")
    return {"sel": sel, "sel_len": sel_len, "n_ctx": n_ctx, "first_pos": first_pos}


def drop_pages(page_table: np.ndarray, resident: float, seed: int) -> np.ndarray:
    """A copy of the page table in which a seeded random (1 - resident)
    fraction of the logical pages is marked not resident (-1)."""
    rng = np.random.default_rng(seed)
    out = page_table.copy()
    n_off = int(round((1.0 - resident) * out.size))
    out[rng.choice(out.size, size=n_off, replace=False)] = -1
    return out
