"""CPU oracle for prompt-phase selection attention over INT8 paged K/V.

TEST INFRASTRUCTURE ONLY: tests/, the smoke check in __graft_entry__ and the
CPU-baseline leg of bench.py are the only code allowed to import this package.
The HIP path never calls it, links it or shares code with it.

The arithmetic lives in sel_attn_oracle.c (plain C, FP64, OpenMP over query
positions); this module builds it with gcc and marshals numpy arrays into it.
Page cited: #2808 "sycl: prompt attention over 8-query selection unions on XMX
(opt-in STRATA_PROMPT_ATTN_UNION=1)", sections Summary (with its accuracy list)
and Extra Notes.

Every function here is pinned by tests/test_oracle_pins.py against dense
brute force, closed forms, invariants and hand-worked fixtures; none is
"parity unpinned". union_rows is plain numpy: a definition, not arithmetic
worth a C loop.

The selection step before the path (block scores -> selection rows) lives in
oracle/selection.py (numpy), pinned by tests/test_selection_oracle.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sel_attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_union.argtypes = [i, i, i, p, p, p, p, p]
        lib.oracle_union.restype = i
        lib.oracle_attention.argtypes = [i, i, i, i, i, i, i, i, p, p, p, p, p, p, p, p,
                                         p, i, ctypes.c_float, p, i]
        lib.oracle_attention.restype = i
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = i
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return _load().oracle_max_threads()


def union(sel: np.ndarray, sel_len: np.ndarray, n_ctx: int):
    """Sorted union and chooser masks of every group of 8 query indices.

    Returns (cells int32 [G][8*cap], mask uint8 [G][8*cap], length int32 [G]);
    entries past length[g] are zero. Raises ValueError on a cell outside
    [0, n_ctx) or a length outside [0, cap].
    """
    sel = _c(sel, np.int32)
    sel_len = _c(sel_len, np.int32)
    n_q, cap = sel.shape
    g = (n_q + 7) // 8
    cells = np.zeros((g, 8 * cap), np.int32)
    mask = np.zeros((g, 8 * cap), np.uint8)
    length = np.zeros(g, np.int32)
    rc = _load().oracle_union(n_q, cap, int(n_ctx), _ptr(sel), _ptr(sel_len), _ptr(cells),
                              _ptr(mask), _ptr(length))
    if rc != 0:
        raise ValueError("oracle_union: invalid selection (rc=%d)" % rc)
    return cells, mask, length


PAGE_RANGE = 4   # the status bit union_rows reports for a page-table entry outside [-1, n_pages)


def union_rows(cells: np.ndarray, length: np.ndarray, page_table: np.ndarray, n_kv: int,
               n_pages: int, page_size: int = 64):
    """The pool row, for KV head 0, of every union cell.

    Pools are [n_pages][n_kv][page_size][head_dim] and scales
    [n_pages][n_kv][page_size], so flattened to rows, cell c of physical page
    p = page_table[c // page_size] sits at row (p * n_kv + h) * page_size +
    c % page_size for KV head h: the KV-head-0 row plus h * page_size. A page
    that is not resident (-1) gives -1 (its cells are masked for every
    position: page section Extra Notes); an entry outside [-1, n_pages) gives
    -1 and sets the PAGE_RANGE flag. Entries past length[g] are 0.
    Returns (rows int32 like cells, flags).
    """
    cells = np.asarray(cells, np.int64)
    length = np.asarray(length, np.int64)
    page_table = np.asarray(page_table, np.int64)
    rows = np.zeros(cells.shape, np.int32)
    flags = 0
    for g in range(cells.shape[0]):
        c = cells[g, :length[g]]
        p = page_table[c // page_size]
        bad = (p < -1) | (p >= n_pages)
        if bad.any():
            flags |= PAGE_RANGE
        ok = (p >= 0) & (p < n_pages)
        rows[g, :length[g]] = np.where(ok, p * n_kv * page_size + c % page_size, -1)
    return rows, flags


def attention(q, k_pool, v_pool, k_scale, v_scale, page_table, sel, sel_len,
              softmax_scale: float, n_ctx: int, rows: Optional[Sequence[int]] = None,
              q_per_kv: int = 12, n_threads: int = 0) -> np.ndarray:
    """FP64 per-position selection attention (float64 [n_rows][n_qh][head_dim])."""
    q = _c(q, np.float32)
    k_pool = _c(k_pool, np.int8)
    v_pool = _c(v_pool, np.int8)
    k_scale = _c(k_scale, np.float32)
    v_scale = _c(v_scale, np.float32)
    page_table = _c(page_table, np.int32)
    sel = _c(sel, np.int32)
    sel_len = _c(sel_len, np.int32)
    n_q, n_qh, head_dim = q.shape
    n_pages, n_kv, page_size, hd2 = k_pool.shape
    assert hd2 == head_dim and n_qh == n_kv * q_per_kv
    assert v_pool.shape == k_pool.shape and k_scale.shape == k_pool.shape[:3]
    assert page_table.size >= -(-n_ctx // page_size)
    if rows is None:
        rows_arr = None
        n_rows = n_q
    else:
        rows_arr = _c(rows, np.int32)
        n_rows = rows_arr.size
    out = np.zeros((n_rows, n_qh, head_dim), np.float64)
    rc = _load().oracle_attention(
        n_q, n_kv, q_per_kv, head_dim, page_size, n_pages, int(n_ctx), sel.shape[1],
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(page_table),
        _ptr(sel), _ptr(sel_len), None if rows_arr is None else _ptr(rows_arr), n_rows,
        ctypes.c_float(float(softmax_scale)), _ptr(out), int(n_threads))
    if rc != 0:
        raise ValueError("oracle_attention: invalid input (rc=%d)" % rc)
    return out


def attention_of(problem: dict, rows=None, n_threads: int = 0) -> np.ndarray:
    """attention() over a dict from synth.generate()/synth.small_random()."""
    return attention(problem["q"], problem["k_pool"], problem["v_pool"], problem["k_scale"],
                     problem["v_scale"], problem["page_table"], problem["sel"],
                     problem["sel_len"], problem["softmax_scale"], problem["n_ctx"],
                     rows=rows, n_threads=n_threads)
