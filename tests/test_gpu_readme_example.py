"""The README's usage sequence (block scores -> selections -> union path; the
per-position call; decode of the last position), run as written on a small
seeded problem and checked against the CPU oracle.

Page cited: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
section What changed (selection, then the prompt attention over the union) and
section Summary (every position attends to exactly its own cells; the accuracy
list against FP64).
"""
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


import gpu_helpers as H  # noqa: E402
import sparse_top_selection_amd as sa  # noqa: E402


def test_readme_sequence():
    n_ctx, n_q = 5000, 37
    first_pos = n_ctx - n_q
    d = synth.small_random(61, n_ctx=n_ctx, n_q=n_q, n_kv=2, nonresident_frac=0.1, pool_extra=3)
    scores = synth.block_scores(n_q, n_ctx, rho=0.95, seed=62)
    g = {k: torch.from_numpy(np.ascontiguousarray(d[k])).cuda()
         for k in ("q", "k_pool", "v_pool", "k_scale", "v_scale", "page_table")}
    q, k_pool, v_pool = g["q"], g["k_pool"], g["v_pool"]
    k_scale, v_scale, page_table = g["k_scale"], g["v_scale"], g["page_table"]
    softmax_scale = float(d["softmax_scale"])
    block_scores = torch.from_numpy(scores).cuda()

    # the README's lines
    sel, sel_len = sa.select_blocks(block_scores, first_pos, n_ctx)
    out, (cells, mask, rows, length), status = sa.attention(
        q, k_pool, v_pool, k_scale, v_scale, page_table, sel, sel_len, softmax_scale, n_ctx)
    assert sa.check_status(status) == 0
    out_pos, status_pos = sa.prefill_positions(q, k_pool, v_pool, k_scale, v_scale, page_table, sel,
                                               sel_len, softmax_scale, n_ctx)
    out_dec, status_dec = sa.decode(q[-1:], k_pool, v_pool, k_scale, v_scale, page_table, sel[-1:],
                                    sel_len[-1:], softmax_scale, n_ctx)
    assert sa.check_status(status_pos) == 0 and sa.check_status(status_dec) == 0

    # the oracle on the selections the GPU produced (themselves bit-exact
    # against the selection oracle in their own tests)
    e = dict(d)
    e["sel"] = sel.cpu().numpy()
    e["sel_len"] = sel_len.cpu().numpy()
    assert np.all(e["sel_len"] > 0)
    ref = oracle.attention_of(e)
    H.assert_close(out.cpu().numpy(), ref, "union path")
    H.assert_close(out_pos.cpu().numpy(), ref, "per-position")
    H.assert_close(out_dec.cpu().numpy(), ref[-1:], "decode")
