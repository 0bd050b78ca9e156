"""Python binding of libselattn.so: prompt-phase selection attention over INT8
paged K/V on gfx950.

Argument marshalling only. Every step of the path runs in the library's HIP
kernels; PyTorch provides device memory and the current stream. There is no
fallback: importing this package fails loudly when libselattn.so is missing,
and every call raises when the library returns an error code.

The functions named like the C entry points (sel_attn_select_blocks,
sel_attn_build_union, sel_attn_prefill, sel_attn_prefill_workspace_bytes,
sel_attn_prefill_split, sel_attn_prefill_positions, sel_attn_decode,
sel_attn_decode_workspace_bytes, sel_attn_decode_noalloc, sel_attn_last_error) take
preallocated device tensors and mirror include/sel_attn.h one to one.
select_blocks(), build_union(), prefill(), prefill_positions(), decode() and
check_status() are conveniences that allocate outputs and read the status word.

Page cited: #2808 "sycl: prompt attention over 8-query selection unions on XMX
(opt-in STRATA_PROMPT_ATTN_UNION=1)", section Summary.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libselattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libselattn.so is not built (%s); run `python sparse_top_selection_amd/build.py`" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

OK = 0
EINVAL = -1
EUNSUPPORTED = -2
ELAUNCH = -3

STATUS_CELL_RANGE = 1
STATUS_SEL_LEN = 2
STATUS_PAGE_RANGE = 4
STATUS_UNION_LEN = 8
STATUS_V_SCALE = 16

HEAD_DIM = 128
PAGE_SIZE = 64
Q_PER_KV = 12
GROUP = 8
SINKS = 3
TOP_BLOCKS = 31
SEL_MAX = 2051
SELECT_MAX_CTX = 262144
POSITIONS_MAX_CAP = 2560
DECODE_MAX_Q = 65535
DECODE_NOALLOC_MAX_BYTES = 8388608

EXPORTED = ("sel_attn_select_blocks", "sel_attn_build_union", "sel_attn_prefill",
            "sel_attn_prefill_workspace_bytes", "sel_attn_prefill_split",
            "sel_attn_prefill_positions", "sel_attn_decode_workspace_bytes", "sel_attn_decode",
            "sel_attn_decode_noalloc", "sel_attn_last_error")


class Dims(ctypes.Structure):
    """sel_attn_dims of include/sel_attn.h."""
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_ctx", "n_q", "n_kv", "q_per_kv", "head_dim", "page_size", "sel_cap",
                 "n_pages")]


def make_dims(n_ctx: int, n_q: int, n_kv: int, n_pages: int, sel_cap: int = 2051,
              q_per_kv: int = Q_PER_KV, head_dim: int = HEAD_DIM,
              page_size: int = PAGE_SIZE) -> Dims:
    return Dims(n_ctx, n_q, n_kv, q_per_kv, head_dim, page_size, sel_cap, n_pages)


_p = ctypes.c_void_p
_lib.sel_attn_select_blocks.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32, _p, _p, _p, _p]
_lib.sel_attn_select_blocks.restype = ctypes.c_int
_lib.sel_attn_build_union.argtypes = [ctypes.POINTER(Dims), _p, _p, _p, _p, _p, _p, _p, _p, _p]
_lib.sel_attn_build_union.restype = ctypes.c_int
_lib.sel_attn_prefill.argtypes = [ctypes.POINTER(Dims), _p, _p, _p, _p, _p, _p, _p, _p,
                                  ctypes.c_float, _p, _p, _p]
_lib.sel_attn_prefill.restype = ctypes.c_int
_lib.sel_attn_prefill_workspace_bytes.argtypes = [ctypes.POINTER(Dims)]
_lib.sel_attn_prefill_workspace_bytes.restype = ctypes.c_size_t
_lib.sel_attn_prefill_split.argtypes = [ctypes.POINTER(Dims), _p, _p, _p, _p, _p, _p, _p, _p,
                                        ctypes.c_float, _p, _p, _p, ctypes.c_size_t, _p]
_lib.sel_attn_prefill_split.restype = ctypes.c_int
_lib.sel_attn_prefill_positions.argtypes = [ctypes.POINTER(Dims), _p, _p, _p, _p, _p, _p, _p, _p,
                                            ctypes.c_float, _p, _p, _p]
_lib.sel_attn_prefill_positions.restype = ctypes.c_int
_lib.sel_attn_decode_workspace_bytes.argtypes = [ctypes.POINTER(Dims)]
_lib.sel_attn_decode_workspace_bytes.restype = ctypes.c_size_t
_lib.sel_attn_decode.argtypes = [ctypes.POINTER(Dims), _p, _p, _p, _p, _p, _p, _p, _p,
                                 ctypes.c_float, _p, _p, ctypes.c_size_t, _p, _p]
_lib.sel_attn_decode.restype = ctypes.c_int
_lib.sel_attn_decode_noalloc.argtypes = [ctypes.POINTER(Dims), _p, _p, _p, _p, _p, _p, _p, _p,
                                         ctypes.c_float, _p, _p, _p]
_lib.sel_attn_decode_noalloc.restype = ctypes.c_int
_lib.sel_attn_last_error.argtypes = []
_lib.sel_attn_last_error.restype = ctypes.c_char_p


class SelAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (code %d)" % (msg, code))
        self.code = code


def sel_attn_last_error() -> str:
    return _lib.sel_attn_last_error().decode()


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int):
    if rc != OK:
        raise SelAttnError(rc, sel_attn_last_error())


def sel_attn_select_blocks(dims: Dims, first_pos: int, block_scores, sel, sel_len,
                           stream=None) -> None:
    """Enqueue the selection step (see include/sel_attn.h). Tensors or raw device pointers."""
    _check(_lib.sel_attn_select_blocks(ctypes.byref(dims), int(first_pos), _ptr(block_scores),
                                       _ptr(sel), _ptr(sel_len), _stream(stream)))


def sel_attn_build_union(dims: Dims, sel, sel_len, page_table, union_cells, union_mask, union_rows,
                         union_len, status, stream=None) -> None:
    """Enqueue the union step (see include/sel_attn.h). Tensors or raw device pointers."""
    _check(_lib.sel_attn_build_union(ctypes.byref(dims), _ptr(sel), _ptr(sel_len),
                                     _ptr(page_table), _ptr(union_cells), _ptr(union_mask),
                                     _ptr(union_rows), _ptr(union_len), _ptr(status),
                                     _stream(stream)))


def sel_attn_prefill(dims: Dims, q, k_pool, v_pool, k_scale, v_scale, union_rows, union_mask,
                     union_len, softmax_scale: float, out, status, stream=None) -> None:
    """Enqueue the attention step (see include/sel_attn.h). Tensors or raw device pointers."""
    _check(_lib.sel_attn_prefill(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                 _ptr(k_scale), _ptr(v_scale), _ptr(union_rows),
                                 _ptr(union_mask), _ptr(union_len),
                                 ctypes.c_float(float(softmax_scale)), _ptr(out), _ptr(status),
                                 _stream(stream)))


def sel_attn_prefill_workspace_bytes(dims: Dims) -> int:
    """Workspace bytes sel_attn_prefill_split needs for these dims (0: it does not split)."""
    return int(_lib.sel_attn_prefill_workspace_bytes(ctypes.byref(dims)))


def sel_attn_prefill_split(dims: Dims, q, k_pool, v_pool, k_scale, v_scale, union_rows,
                           union_mask, union_len, softmax_scale: float, out, status, workspace,
                           workspace_bytes: int, stream=None) -> None:
    """Enqueue the attention step, splitting small grids over the workspace (see
    include/sel_attn.h). Tensors or raw device pointers."""
    _check(_lib.sel_attn_prefill_split(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                       _ptr(k_scale), _ptr(v_scale), _ptr(union_rows),
                                       _ptr(union_mask), _ptr(union_len),
                                       ctypes.c_float(float(softmax_scale)), _ptr(out),
                                       _ptr(status), _ptr(workspace), ctypes.c_size_t(workspace_bytes),
                                       _stream(stream)))


def sel_attn_prefill_positions(dims: Dims, q, k_pool, v_pool, k_scale, v_scale, page_table, sel,
                               sel_len, softmax_scale: float, out, status, stream=None) -> None:
    """Enqueue the per-position attention (see include/sel_attn.h). Tensors or raw device pointers."""
    _check(_lib.sel_attn_prefill_positions(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                           _ptr(k_scale), _ptr(v_scale), _ptr(page_table),
                                           _ptr(sel), _ptr(sel_len),
                                           ctypes.c_float(float(softmax_scale)), _ptr(out),
                                           _ptr(status), _stream(stream)))


def sel_attn_decode_workspace_bytes(dims: Dims) -> int:
    """Workspace bytes sel_attn_decode needs for these dims (0 if they are invalid)."""
    return int(_lib.sel_attn_decode_workspace_bytes(ctypes.byref(dims)))


def sel_attn_decode(dims: Dims, q, k_pool, v_pool, k_scale, v_scale, page_table, sel, sel_len,
                    softmax_scale: float, out, workspace, workspace_bytes: int, status,
                    stream=None) -> None:
    """Enqueue the decode attention (see include/sel_attn.h). Tensors or raw device pointers."""
    _check(_lib.sel_attn_decode(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                _ptr(k_scale), _ptr(v_scale), _ptr(page_table), _ptr(sel),
                                _ptr(sel_len), ctypes.c_float(float(softmax_scale)), _ptr(out),
                                _ptr(workspace), int(workspace_bytes), _ptr(status),
                                _stream(stream)))


def sel_attn_decode_noalloc(dims: Dims, q, k_pool, v_pool, k_scale, v_scale, page_table, sel,
                            sel_len, softmax_scale: float, out, status, stream=None) -> None:
    """Enqueue the decode attention with the library's static scratch instead of
    a workspace (see include/sel_attn.h). Tensors or raw device pointers."""
    _check(_lib.sel_attn_decode_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                        _ptr(k_scale), _ptr(v_scale), _ptr(page_table), _ptr(sel),
                                        _ptr(sel_len), ctypes.c_float(float(softmax_scale)),
                                        _ptr(out), _ptr(status), _stream(stream)))


# --------------------------------------------------------------------------
# conveniences over torch tensors
# --------------------------------------------------------------------------
def _on_gpu(t: torch.Tensor, name: str) -> torch.device:
    """The tensor's device, which must be a GPU: the kernels dereference every
    pointer they are given, so a host tensor must never reach them."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU (got %s)" % (name, t.device))
    return t.device


def _need(t: torch.Tensor, name: str, dtype, ndim: int, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims (got %s)" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s (got %s)" % (name, device, t.device))


def _need_shape(t, name: str, dtype, shape, device):
    """A caller-supplied output: dtype, exact shape, contiguous, on the device."""
    _need(t, name, dtype, len(shape), device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))


def _status_for(status, device) -> torch.Tensor:
    if status is None:
        return new_status(device)
    _need_shape(status, "status", torch.uint32, (1,), device)
    return status


def new_status(device) -> torch.Tensor:
    """A zeroed status word: uint32 [1] on the device, as the header declares it
    (filled as int32 zeros and viewed as uint32: same bytes, no uint32 kernel)."""
    return torch.zeros(1, dtype=torch.int32, device=device).view(torch.uint32)


def status_value(status: torch.Tensor) -> int:
    """Synchronise on a status word and return its bits as an unsigned int
    (read through an int32 view of the same 4 bytes)."""
    return int(status.view(torch.int32).item()) & 0xFFFFFFFF


def check_status(status: torch.Tensor) -> int:
    """Synchronise on the status word and raise on any set bit."""
    v = status_value(status)
    if v:
        names = [n for n, b in (("CELL_RANGE", 1), ("SEL_LEN", 2), ("PAGE_RANGE", 4),
                                ("UNION_LEN", 8), ("V_SCALE", 16)) if v & b]
        raise SelAttnError(v, "device status: " + "|".join(names))
    return v


def select_blocks(block_scores: torch.Tensor, first_pos: int, n_ctx: int,
                  sel_cap: int = SEL_MAX, stream=None, out=None):
    """Selections of positions first_pos .. first_pos + n_q - 1 from block
    scores float32 [n_q][ceil(n_ctx/64)]. Returns (sel, sel_len); entries past
    sel_len are left as allocated (torch.empty) or as they were in `out`."""
    dev = _on_gpu(block_scores, "block_scores")
    _need(block_scores, "block_scores", torch.float32, 2, dev)
    n_q, nb = block_scores.shape
    if nb != -(-n_ctx // PAGE_SIZE):
        raise ValueError("block_scores must be [n_q][ceil(n_ctx/64)]")
    if out is None:
        sel = torch.empty((n_q, sel_cap), dtype=torch.int32, device=dev)
        sel_len = torch.empty(n_q, dtype=torch.int32, device=dev)
    else:
        sel, sel_len = out
        _need(sel, "sel", torch.int32, 2, dev)
        _need_shape(sel_len, "sel_len", torch.int32, (n_q,), dev)
        if sel.shape[0] != n_q:
            raise ValueError("sel must have n_q rows")
        sel_cap = sel.shape[1]
    dims = make_dims(n_ctx, n_q, 1, 1, sel_cap=sel_cap)
    sel_attn_select_blocks(dims, first_pos, block_scores, sel, sel_len, stream)
    return sel, sel_len


def build_union(sel: torch.Tensor, sel_len: torch.Tensor, n_ctx: int, page_table=None,
                n_kv: int = 1, n_pages: int = 1, status=None, stream=None, out=None):
    """Union of every group of 8 query indices, each cell also resolved through
    the page table to its pool row for KV head 0 (pools [n_pages][n_kv][64][128]).
    Without a page table every page counts as not resident (rows -1); the cells
    and masks do not depend on it. Returns (cells, mask, rows, length, status)."""
    dev = _on_gpu(sel, "sel")
    _need(sel, "sel", torch.int32, 2, dev)
    _need(sel_len, "sel_len", torch.int32, 1, dev)
    n_q, cap = sel.shape
    if sel_len.shape[0] != n_q:
        raise ValueError("sel_len must have n_q entries")
    n_lpages = -(-n_ctx // PAGE_SIZE)
    if page_table is None:
        page_table = torch.full((n_lpages,), -1, dtype=torch.int32, device=dev)
    _need(page_table, "page_table", torch.int32, 1, dev)
    if page_table.shape[0] < n_lpages:
        raise ValueError("page_table needs ceil(n_ctx / page_size) entries")
    g = (n_q + 7) // 8
    if out is None:
        cells = torch.empty((g, 8 * cap), dtype=torch.int32, device=dev)
        mask = torch.empty((g, 8 * cap), dtype=torch.uint8, device=dev)
        rows = torch.empty((g, 8 * cap), dtype=torch.int32, device=dev)
        length = torch.empty(g, dtype=torch.int32, device=dev)
    else:
        cells, mask, rows, length = out
        _need_shape(cells, "union_cells", torch.int32, (g, 8 * cap), dev)
        _need_shape(mask, "union_mask", torch.uint8, (g, 8 * cap), dev)
        _need_shape(rows, "union_rows", torch.int32, (g, 8 * cap), dev)
        _need_shape(length, "union_len", torch.int32, (g,), dev)
    status = _status_for(status, dev)
    dims = make_dims(n_ctx, n_q, n_kv, n_pages, sel_cap=cap)
    sel_attn_build_union(dims, sel, sel_len, page_table, cells, mask, rows, length, status, stream)
    return cells, mask, rows, length, status


def prefill(q, k_pool, v_pool, k_scale, v_scale, union_rows, union_mask, union_len,
            softmax_scale: float, n_ctx: int, status=None, stream=None, out=None, split=False,
            workspace=None):
    """Attention over each group's union. With split=True, grids too small for
    the GPU are split over a workspace (uint8 device tensor, allocated when not
    given; see sel_attn_prefill_split). Returns (out, status)."""
    dev = _on_gpu(q, "q")
    _need(q, "q", torch.float32, 3, dev)
    for name, t, dt, nd in (("k_pool", k_pool, torch.int8, 4), ("v_pool", v_pool, torch.int8, 4),
                            ("k_scale", k_scale, torch.float32, 3),
                            ("v_scale", v_scale, torch.float32, 3),
                            ("union_rows", union_rows, torch.int32, 2),
                            ("union_mask", union_mask, torch.uint8, 2),
                            ("union_len", union_len, torch.int32, 1)):
        _need(t, name, dt, nd, dev)
    n_q, n_qh, hd = q.shape
    n_pages, n_kv, ps, hd2 = k_pool.shape
    if v_pool.shape != k_pool.shape or tuple(k_scale.shape) != (n_pages, n_kv, ps) or \
            tuple(v_scale.shape) != (n_pages, n_kv, ps):
        raise ValueError("pool / scale shapes disagree")
    if hd2 != hd or n_qh != n_kv * Q_PER_KV:
        raise ValueError("q is [n_q][n_kv*12][head_dim] with the pools' n_kv and head_dim")
    g = (n_q + 7) // 8
    if union_len.shape[0] != g or union_rows.shape[0] != g or union_rows.shape[1] % 8 != 0 \
            or union_mask.shape != union_rows.shape:
        raise ValueError("union arrays must be [ceil(n_q/8)][8*sel_cap]")
    cap = union_rows.shape[1] // 8
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_shape(out, "out", torch.float32, q.shape, dev)
    status = _status_for(status, dev)
    dims = make_dims(n_ctx, n_q, n_kv, n_pages, sel_cap=cap, head_dim=hd, page_size=ps)
    if not split:
        sel_attn_prefill(dims, q, k_pool, v_pool, k_scale, v_scale, union_rows, union_mask,
                         union_len, softmax_scale, out, status, stream)
        return out, status
    need = sel_attn_prefill_workspace_bytes(dims)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, 1, dev)
    sel_attn_prefill_split(dims, q, k_pool, v_pool, k_scale, v_scale, union_rows, union_mask,
                           union_len, softmax_scale, out, status, workspace,
                           workspace.numel() * workspace.element_size(), stream)
    return out, status


def _positions_dims(q, k_pool, v_pool, k_scale, v_scale, page_table, sel, sel_len, n_ctx):
    dev = _on_gpu(q, "q")
    _need(q, "q", torch.float32, 3, dev)
    for name, t, dt, nd in (("k_pool", k_pool, torch.int8, 4), ("v_pool", v_pool, torch.int8, 4),
                            ("k_scale", k_scale, torch.float32, 3),
                            ("v_scale", v_scale, torch.float32, 3),
                            ("page_table", page_table, torch.int32, 1),
                            ("sel", sel, torch.int32, 2), ("sel_len", sel_len, torch.int32, 1)):
        _need(t, name, dt, nd, dev)
    n_q, n_qh, hd = q.shape
    n_pages, n_kv, ps, hd2 = k_pool.shape
    if v_pool.shape != k_pool.shape or tuple(k_scale.shape) != (n_pages, n_kv, ps) or \
            tuple(v_scale.shape) != (n_pages, n_kv, ps):
        raise ValueError("pool / scale shapes disagree")
    if hd2 != hd or n_qh != n_kv * Q_PER_KV:
        raise ValueError("q is [n_q][n_kv*12][head_dim] with the pools' n_kv and head_dim")
    if page_table.shape[0] < -(-n_ctx // ps):
        raise ValueError("page_table needs ceil(n_ctx / page_size) entries")
    if sel.shape[0] != n_q or sel_len.shape[0] != n_q:
        raise ValueError("sel and sel_len must have n_q rows")
    return make_dims(n_ctx, n_q, n_kv, n_pages, sel_cap=sel.shape[1], head_dim=hd, page_size=ps)


def prefill_positions(q, k_pool, v_pool, k_scale, v_scale, page_table, sel, sel_len,
                      softmax_scale: float, n_ctx: int, status=None, stream=None, out=None):
    """Per-position attention over each position's own selection (no union).
    Returns (out, status)."""
    dims = _positions_dims(q, k_pool, v_pool, k_scale, v_scale, page_table, sel, sel_len, n_ctx)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_shape(out, "out", torch.float32, q.shape, q.device)
    status = _status_for(status, q.device)
    sel_attn_prefill_positions(dims, q, k_pool, v_pool, k_scale, v_scale, page_table, sel, sel_len,
                               softmax_scale, out, status, stream)
    return out, status


def decode(q, k_pool, v_pool, k_scale, v_scale, page_table, sel, sel_len, softmax_scale: float,
           n_ctx: int, status=None, stream=None, out=None, workspace=None):
    """Decode attention for a few positions, split over their cells. The
    workspace (uint8 device tensor) is allocated when not given.
    Returns (out, status)."""
    dims = _positions_dims(q, k_pool, v_pool, k_scale, v_scale, page_table, sel, sel_len, n_ctx)
    need = sel_attn_decode_workspace_bytes(dims)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        _need(workspace, "workspace", torch.uint8, 1, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_shape(out, "out", torch.float32, q.shape, q.device)
    status = _status_for(status, q.device)
    sel_attn_decode(dims, q, k_pool, v_pool, k_scale, v_scale, page_table, sel, sel_len,
                    softmax_scale, out, workspace, workspace.numel() * workspace.element_size(),
                    status, stream)
    return out, status


def attention(q, k_pool, v_pool, k_scale, v_scale, page_table, sel, sel_len,
              softmax_scale: float, n_ctx: int, stream=None, split=False):
    """One pass of the whole path (union, then attention). Returns
    (out, (cells, mask, rows, length), status)."""
    _need(k_pool, "k_pool", torch.int8, 4, _on_gpu(k_pool, "k_pool"))
    n_pages, n_kv = k_pool.shape[0], k_pool.shape[1]
    cells, mask, rows, length, status = build_union(sel, sel_len, n_ctx, page_table, n_kv, n_pages,
                                                    stream=stream)
    out, status = prefill(q, k_pool, v_pool, k_scale, v_scale, rows, mask, length, softmax_scale,
                          n_ctx, status=status, stream=stream, split=split)
    return out, (cells, mask, rows, length), status
