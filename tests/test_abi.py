"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sel_attn.h")
LIB = os.path.join(ROOT, "sparse_top_selection_amd", "libselattn.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sel_attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["sel_attn_build_union", "sel_attn_decode",
                                    "sel_attn_decode_noalloc",
                                    "sel_attn_decode_workspace_bytes", "sel_attn_last_error",
                                    "sel_attn_prefill", "sel_attn_prefill_positions",
                                    "sel_attn_prefill_split",
                                    "sel_attn_prefill_workspace_bytes",
                                    "sel_attn_select_blocks"]


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_names_match_header():
    import sparse_top_selection_amd as sa
    assert sorted(sa.EXPORTED) == declared_functions()
    for name in declared_functions():
        assert callable(getattr(sa, name))


def _dims(**kw):
    import sparse_top_selection_amd as sa
    base = dict(n_ctx=1024, n_q=16, n_kv=2, n_pages=16)
    base.update(kw)
    d = sa.make_dims(base.pop("n_ctx"), base.pop("n_q"), base.pop("n_kv"), base.pop("n_pages"),
                     **base)
    return d


FAKE = 1 << 20   # never dereferenced: every case below fails on the host first


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), -2), (dict(page_size=32), -2), (dict(q_per_kv=8), -2),
    (dict(n_ctx=0), -1), (dict(n_q=-1), -1), (dict(n_kv=0), -1), (dict(sel_cap=0), -1),
    (dict(n_pages=0), -1), (dict(n_pages=1 << 25, n_kv=4), -1),
])
def test_bad_dims_rejected_on_host(kw, code):
    import sparse_top_selection_amd as sa
    with pytest.raises(sa.SelAttnError) as e:
        sa.sel_attn_build_union(_dims(**kw), *(FAKE,) * 8, stream=0)
    assert e.value.code == code
    assert "sel_attn_build_union" in sa.sel_attn_last_error()
    with pytest.raises(sa.SelAttnError) as e:
        sa.sel_attn_prefill(_dims(**kw), *(FAKE,) * 8, 0.1, FAKE, FAKE, stream=0)
    assert e.value.code == code
    with pytest.raises(sa.SelAttnError) as e:
        sa.sel_attn_select_blocks(_dims(sel_cap=2051, **kw) if "sel_cap" not in kw else _dims(**kw),
                                  0, FAKE, FAKE, FAKE, stream=0)
    assert e.value.code == code


@pytest.mark.parametrize("kw,first,code", [
    (dict(sel_cap=2050), 0, -1),                      # cannot hold a full selection
    (dict(sel_cap=2051, n_ctx=1024, n_q=16), 1009, -1),   # last position past n_ctx
    (dict(sel_cap=2051), -1, -1),                     # negative first position
    (dict(sel_cap=2051, n_ctx=262145, n_q=16, n_pages=4200), 0, -2),   # context over the limit
])
def test_select_blocks_rejects_on_host(kw, first, code):
    import sparse_top_selection_amd as sa
    with pytest.raises(sa.SelAttnError) as e:
        sa.sel_attn_select_blocks(_dims(**kw), first, FAKE, FAKE, FAKE, stream=0)
    assert e.value.code == code
    assert "sel_attn_select_blocks" in sa.sel_attn_last_error()
    if code == -1 and kw.get("sel_cap") == 2051 and first >= 0:
        # the same call one position earlier passes the position check and
        # fails only at a NULL pointer
        with pytest.raises(sa.SelAttnError) as e:
            sa.sel_attn_select_blocks(_dims(**kw), first - 1, FAKE, None, FAKE, stream=0)
        assert "NULL" in sa.sel_attn_last_error()


def test_prefill_positions_rejects_on_host():
    import sparse_top_selection_amd as sa
    args = (FAKE,) * 8
    with pytest.raises(sa.SelAttnError) as e:   # row stride over the supported cap
        sa.sel_attn_prefill_positions(_dims(sel_cap=2561), *args, 0.1, FAKE, FAKE, stream=0)
    assert e.value.code == -2 and "sel_attn_prefill_positions" in sa.sel_attn_last_error()
    with pytest.raises(sa.SelAttnError) as e:   # q must be 16-byte aligned
        sa.sel_attn_prefill_positions(_dims(), FAKE + 4, *args[1:], 0.1, FAKE, FAKE, stream=0)
    assert e.value.code == -1
    with pytest.raises(sa.SelAttnError) as e:   # status is required
        sa.sel_attn_prefill_positions(_dims(), *args, 0.1, FAKE, None, stream=0)
    assert e.value.code == -1
    with pytest.raises(sa.SelAttnError) as e:   # a NULL selection
        sa.sel_attn_prefill_positions(_dims(), *args[:6], None, FAKE, 0.1, FAKE, FAKE, stream=0)
    assert e.value.code == -1
    with pytest.raises(sa.SelAttnError) as e:
        sa.sel_attn_prefill_positions(_dims(), *args, float("nan"), FAKE, FAKE, stream=0)
    assert e.value.code == -1
    sa.sel_attn_prefill_positions(_dims(n_q=0), *(None,) * 8, 0.1, None, FAKE, stream=0)
    assert sa.sel_attn_last_error() == ""


def test_decode_rejects_on_host():
    import sparse_top_selection_amd as sa
    d = _dims(n_q=3)
    need = sa.sel_attn_decode_workspace_bytes(d)
    assert need == 3 * 2 * 33 * 6272
    args = (FAKE,) * 8
    for ws, nbytes in ((None, need), (FAKE, need - 1), (FAKE + 8, need)):
        with pytest.raises(sa.SelAttnError) as e:
            sa.sel_attn_decode(d, *args, 0.1, FAKE, ws, nbytes, FAKE, stream=0)
        assert e.value.code == -1 and "workspace" in sa.sel_attn_last_error()
    with pytest.raises(sa.SelAttnError) as e:   # many positions: not a decode call
        big = _dims(n_q=70000)
        sa.sel_attn_decode(big, *args, 0.1, FAKE, FAKE, sa.sel_attn_decode_workspace_bytes(big),
                           FAKE, stream=0)
    assert e.value.code == -1
    with pytest.raises(sa.SelAttnError) as e:
        sa.sel_attn_decode(_dims(sel_cap=2561), *args, 0.1, FAKE, FAKE, 1 << 30, FAKE, stream=0)
    assert e.value.code == -2
    sa.sel_attn_decode(_dims(n_q=0), *(None,) * 8, 0.1, None, None, 0, FAKE, stream=0)
    assert sa.sel_attn_last_error() == ""


def test_decode_noalloc_rejects_on_host():
    """The allocation-free decode refuses dims whose split records exceed its
    static array, and bad arguments, before touching the device."""
    import sparse_top_selection_amd as sa
    args = (FAKE,) * 8
    for n_q, n_kv, cap in ((9, 4, 2560), (1, 34, 2560), (11, 4, 2051)):
        d = _dims(n_q=n_q, n_kv=n_kv, sel_cap=cap, n_pages=16)
        assert sa.sel_attn_decode_workspace_bytes(d) > sa.DECODE_NOALLOC_MAX_BYTES
        with pytest.raises(sa.SelAttnError) as e:
            sa.sel_attn_decode_noalloc(d, *args, 0.1, FAKE, FAKE, stream=0)
        assert e.value.code == -1 and "static scratch" in sa.sel_attn_last_error()
    ok = _dims(n_q=8, n_kv=4, sel_cap=2560)
    assert sa.sel_attn_decode_workspace_bytes(ok) <= sa.DECODE_NOALLOC_MAX_BYTES
    with pytest.raises(sa.SelAttnError) as e:   # fits, but a NULL array pointer
        sa.sel_attn_decode_noalloc(ok, *args[:7], None, 0.1, FAKE, FAKE, stream=0)
    assert e.value.code == -1 and "NULL" in sa.sel_attn_last_error()
    with pytest.raises(sa.SelAttnError) as e:
        sa.sel_attn_decode_noalloc(_dims(sel_cap=2561), *args, 0.1, FAKE, FAKE, stream=0)
    assert e.value.code == -2
    sa.sel_attn_decode_noalloc(_dims(n_q=0), *(None,) * 8, 0.1, None, FAKE, stream=0)
    assert sa.sel_attn_last_error() == ""


def test_null_and_misaligned_pointers_rejected_on_host():
    import sparse_top_selection_amd as sa
    # build_union: dims, sel, sel_len, page_table, cells, mask, rows, len, status
    for bad in (1, 2, 3, 5, 6, 7):   # sel_len, page_table, cells, rows, len, status: NULL
        args = [FAKE] * 8
        args[bad] = None
        with pytest.raises(sa.SelAttnError) as e:
            sa.sel_attn_build_union(_dims(), *args, stream=0)
        assert e.value.code == -1 and "NULL" in sa.sel_attn_last_error()
    for bad in (0, 2, 5):      # sel, page_table, union_rows: 4-byte aligned
        args = [FAKE] * 8
        args[bad] = FAKE + 2
        with pytest.raises(sa.SelAttnError) as e:
            sa.sel_attn_build_union(_dims(), *args, stream=0)
        assert e.value.code == -1 and "aligned" in sa.sel_attn_last_error()
    with pytest.raises(sa.SelAttnError) as e:   # q must be 16-byte aligned
        sa.sel_attn_prefill(_dims(), FAKE + 4, *(FAKE,) * 7, 0.1, FAKE, FAKE, stream=0)
    assert e.value.code == -1
    with pytest.raises(sa.SelAttnError) as e:   # union_rows must be 4-byte aligned
        sa.sel_attn_prefill(_dims(), *(FAKE,) * 5, FAKE + 2, FAKE, FAKE, 0.1, FAKE, FAKE, stream=0)
    assert e.value.code == -1 and "aligned" in sa.sel_attn_last_error()
    with pytest.raises(sa.SelAttnError) as e:   # union_rows is required
        sa.sel_attn_prefill(_dims(), *(FAKE,) * 5, None, FAKE, FAKE, 0.1, FAKE, FAKE, stream=0)
    assert e.value.code == -1 and "NULL" in sa.sel_attn_last_error()
    with pytest.raises(sa.SelAttnError) as e:   # status is required
        sa.sel_attn_prefill(_dims(), *(FAKE,) * 8, 0.1, FAKE, None, stream=0)
    assert e.value.code == -1
    with pytest.raises(sa.SelAttnError) as e:   # non-finite softmax scale
        sa.sel_attn_prefill(_dims(), *(FAKE,) * 8, float("inf"), FAKE, FAKE, stream=0)
    assert e.value.code == -1


def test_empty_query_batch_is_a_no_op():
    import sparse_top_selection_amd as sa
    sa.sel_attn_build_union(_dims(n_q=0), *(None,) * 7, FAKE, stream=0)
    sa.sel_attn_prefill(_dims(n_q=0), *(None,) * 8, 0.1, None, FAKE, stream=0)
    sa.sel_attn_select_blocks(_dims(n_q=0, sel_cap=2051), 5, None, None, None, stream=0)
    assert sa.sel_attn_last_error() == ""
    with pytest.raises(sa.SelAttnError):   # misaligned scores
        sa.sel_attn_select_blocks(_dims(sel_cap=2051), 0, FAKE + 2, FAKE, FAKE, stream=0)


def test_builder_loads_without_the_library():
    # A fresh checkout has no libselattn.so; the build step must still load
    # its builder (the package itself refuses to import until it is built).
    import subprocess
    import sys
    code = ("import sys, __graft_entry__ as g; m = g._load_builder(); "
            "assert 'sparse_top_selection_amd' not in sys.modules; "
            "assert m.sources(), 'no HIP sources'")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def _small_problem(n_q=10, n_kv=1, n_pages=4, cap=7):
    import torch
    return dict(
        q=torch.zeros((n_q, 12 * n_kv, 128), dtype=torch.float32),
        k_pool=torch.zeros((n_pages, n_kv, 64, 128), dtype=torch.int8),
        v_pool=torch.zeros((n_pages, n_kv, 64, 128), dtype=torch.int8),
        k_scale=torch.zeros((n_pages, n_kv, 64), dtype=torch.float32),
        v_scale=torch.zeros((n_pages, n_kv, 64), dtype=torch.float32),
        page_table=torch.zeros(n_pages, dtype=torch.int32),
        sel=torch.zeros((n_q, cap), dtype=torch.int32),
        sel_len=torch.zeros(n_q, dtype=torch.int32),
        cells=torch.zeros(((n_q + 7) // 8, 8 * cap), dtype=torch.int32),
        mask=torch.zeros(((n_q + 7) // 8, 8 * cap), dtype=torch.uint8),
        rows=torch.zeros(((n_q + 7) // 8, 8 * cap), dtype=torch.int32),
        length=torch.zeros((n_q + 7) // 8, dtype=torch.int32))


def test_convenience_outputs_checked_before_the_library(monkeypatch):
    # Caller-supplied outputs and status words of the wrong dtype or shape
    # never reach a kernel: the binding raises first (CPU tensors; the C
    # entry points are replaced by functions that fail the test if called).
    import torch
    import sparse_top_selection_amd as sa

    def never(*a, **k):
        raise AssertionError("reached the library")
    for name in sa.EXPORTED:
        if name not in ("sel_attn_last_error", "sel_attn_decode_workspace_bytes"):
            monkeypatch.setattr(sa, name, never)
    # these CPU tensors stand in for GPU ones: only the shape and dtype checks
    # are under test here (test_host_tensors_never_reach_the_library covers
    # the device check)
    monkeypatch.setattr(sa, "_on_gpu", lambda t, name: t.device)
    p = _small_problem()
    n_ctx = 4 * 64
    pool = (p["q"], p["k_pool"], p["v_pool"], p["k_scale"], p["v_scale"], p["page_table"])
    kv = pool[:5]   # the union call takes rows instead of the page table
    short = torch.zeros((9, 12, 128), dtype=torch.float32)
    wide_status = torch.zeros(2, dtype=torch.int32)
    u32_status = torch.zeros(1, dtype=torch.int64)

    cases = [
        lambda: sa.prefill(*kv, p["rows"], p["mask"], p["length"], 0.1, n_ctx, out=short),
        lambda: sa.prefill(*kv, p["rows"], p["mask"], p["length"], 0.1, n_ctx,
                           out=p["q"].double()),
        lambda: sa.prefill(*kv, p["rows"], p["mask"], p["length"], 0.1, n_ctx,
                           status=wide_status),
        lambda: sa.prefill(*kv, p["rows"], p["mask"], p["length"], 0.1, n_ctx,
                           status=u32_status),
        lambda: sa.prefill(*kv, p["rows"][:, :5], p["mask"], p["length"], 0.1, n_ctx),
        lambda: sa.prefill(*kv, p["cells"].to(torch.int64), p["mask"], p["length"], 0.1, n_ctx),
        lambda: sa.prefill_positions(*pool, p["sel"], p["sel_len"], 0.1, n_ctx, out=short),
        lambda: sa.prefill_positions(*pool, p["sel"], p["sel_len"], 0.1, n_ctx,
                                     status=wide_status),
        lambda: sa.decode(*pool, p["sel"], p["sel_len"], 0.1, n_ctx, out=short),
        lambda: sa.decode(*pool, p["sel"], p["sel_len"], 0.1, n_ctx,
                          workspace=torch.zeros(64, dtype=torch.int32)),
        lambda: sa.build_union(p["sel"], p["sel_len"], n_ctx,
                               out=(p["cells"][:1], p["mask"], p["rows"], p["length"])),
        lambda: sa.build_union(p["sel"], p["sel_len"], n_ctx,
                               out=(p["cells"], p["mask"].to(torch.int8), p["rows"], p["length"])),
        lambda: sa.build_union(p["sel"], p["sel_len"], n_ctx,
                               out=(p["cells"], p["mask"], p["rows"][:1], p["length"])),
        lambda: sa.build_union(p["sel"], p["sel_len"], n_ctx,
                               out=(p["cells"], p["mask"], p["rows"], p["length"][:1])),
        lambda: sa.build_union(p["sel"], p["sel_len"], n_ctx, status=wide_status),
        lambda: sa.build_union(p["sel"], p["sel_len"], n_ctx, p["page_table"][:2]),
        lambda: sa.build_union(p["sel"], p["sel_len"], n_ctx, p["page_table"].to(torch.int64)),
        lambda: sa.select_blocks(torch.zeros((10, 4), dtype=torch.float32), 200, n_ctx,
                                 out=(p["sel"], p["sel_len"][:3])),
    ]
    for i, case in enumerate(cases):
        with pytest.raises((ValueError, TypeError)):
            case()
    # the same calls with valid arguments do reach the library
    with pytest.raises(AssertionError, match="reached the library"):
        sa.prefill(*kv, p["rows"], p["mask"], p["length"], 0.1, n_ctx,
                   out=torch.zeros_like(p["q"]), status=torch.zeros(1, dtype=torch.uint32))
    with pytest.raises(AssertionError, match="reached the library"):
        sa.build_union(p["sel"], p["sel_len"], n_ctx, p["page_table"], 1, 4,
                       out=(p["cells"], p["mask"], p["rows"], p["length"]))


def test_host_tensors_never_reach_the_library(monkeypatch):
    """Every convenience refuses tensors that are not on a GPU before any C
    entry point is called: a kernel handed host pointers would fault."""
    import torch
    import sparse_top_selection_amd as sa

    def never(*a, **k):
        raise AssertionError("reached the library")
    for name in sa.EXPORTED:
        if name not in ("sel_attn_last_error", "sel_attn_decode_workspace_bytes"):
            monkeypatch.setattr(sa, name, never)
    p = _small_problem()
    n_ctx = 4 * 64
    pool = (p["q"], p["k_pool"], p["v_pool"], p["k_scale"], p["v_scale"], p["page_table"])
    cases = [
        lambda: sa.select_blocks(torch.zeros((10, 4), dtype=torch.float32), 200, n_ctx),
        lambda: sa.build_union(p["sel"], p["sel_len"], n_ctx),
        lambda: sa.build_union(p["sel"], p["sel_len"], n_ctx, p["page_table"], 1, 4),
        lambda: sa.prefill(*pool[:5], p["rows"], p["mask"], p["length"], 0.1, n_ctx),
        lambda: sa.prefill_positions(*pool, p["sel"], p["sel_len"], 0.1, n_ctx),
        lambda: sa.decode(*pool, p["sel"], p["sel_len"], 0.1, n_ctx),
        lambda: sa.attention(*pool, p["sel"], p["sel_len"], 0.1, n_ctx),
    ]
    for case in cases:
        with pytest.raises(ValueError, match="must be on a GPU"):
            case()


def test_status_word_is_the_headers_uint32():
    """new_status() gives the header's status type: one zeroed uint32."""
    import torch
    import sparse_top_selection_amd as sa
    st = sa.new_status(torch.device("cpu"))
    assert st.dtype == torch.uint32 and tuple(st.shape) == (1,) and sa.status_value(st) == 0
    assert sa.check_status(st) == 0


def test_prefill_split_workspace_size_and_host_errors():
    """sel_attn_prefill_split needs a workspace only when the grid is small, of
    groups x KV heads x splits records of 49,920 bytes; a missing or short one
    is refused before the device is touched."""
    import sparse_top_selection_amd as sa
    big = _dims(n_ctx=32768, n_q=8192, n_kv=4)
    assert sa.sel_attn_prefill_workspace_bytes(big) == 0      # 4,096 work-groups: no split
    long = _dims(n_ctx=65536, n_q=32, n_kv=4)                 # 16 items: 16 splits each
    assert sa.sel_attn_prefill_workspace_bytes(long) == 16 * 16 * 49920
    mid = _dims(n_ctx=8192, n_q=1024, n_kv=1)                 # 128 items: 4 splits each
    assert sa.sel_attn_prefill_workspace_bytes(mid) == 128 * 4 * 49920
    small = _dims(n_ctx=1536, n_q=250, n_kv=1)                # 32 items, at most 48 chunks: 4 splits
    assert sa.sel_attn_prefill_workspace_bytes(small) == 32 * 4 * 49920
    capped = _dims(n_ctx=65536, n_q=16, n_kv=1, sel_cap=40)   # unions of at most 320 cells: 10 chunks
    assert sa.sel_attn_prefill_workspace_bytes(capped) == 0
    assert sa.sel_attn_prefill_workspace_bytes(_dims(n_ctx=300, n_q=16, n_kv=1)) == 0
    assert sa.sel_attn_prefill_workspace_bytes(_dims(n_q=0)) == 0
    args = (FAKE,) * 8
    for ws, nbytes in ((None, 0), (FAKE, 32 * 4 * 49920 - 1)):
        with pytest.raises(sa.SelAttnError) as e:
            sa.sel_attn_prefill_split(small, *args, 0.1, FAKE, FAKE, ws, nbytes, stream=0)
        assert e.value.code == -1 and "workspace" in sa.sel_attn_last_error()
    with pytest.raises(sa.SelAttnError) as e:
        sa.sel_attn_prefill_split(small, *args, 0.1, FAKE, FAKE, FAKE + 8, 32 * 4 * 49920, stream=0)
    assert e.value.code == -1 and "aligned" in sa.sel_attn_last_error()
    sa.sel_attn_prefill_split(_dims(n_q=0), *(None,) * 8, 0.1, None, FAKE, None, 0, stream=0)
    assert sa.sel_attn_last_error() == ""
