"""The v_scale range of the three attention calls, at its edge.

The kernels carry P' = p * v_scale * 2^6 in FP16 (p <= 2^7 under the lazy
stabiliser), so they accept |v_scale| < 4 and flag anything else (including NaN
and infinities) with STATUS_V_SCALE. Below the limit the result must still
match the oracle: the gate of the prompt path (max abs 8e-3 for V values up to
127 * 0.05) is scaled by the V range used here.

Page cited: #2808 "sycl: prompt attention over 8-query selection unions on XMX",
section Summary (P and V enter the product in FP16 with FP32 sums; the accuracy
list against FP64). The limit is this library's, not the page's.
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

BELOW = float(np.nextafter(np.float32(4.0), np.float32(0.0)))   # largest float32 under 4
CALLS = ("union", "positions", "decode")


def _problem(seed: int, call: str) -> dict:
    n_q = 4 if call == "decode" else 21
    return synth.small_random(seed, n_ctx=900, n_q=n_q, n_kv=2, dup_frac=0.2,
                              nonresident_frac=0.1)


def _run(call: str, d: dict, v_scale: np.ndarray):
    dev = H.to_device(d)
    vs = torch.from_numpy(np.ascontiguousarray(v_scale)).cuda()
    args = (dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], vs, dev["page_table"],
            dev["sel"], dev["sel_len"], float(d["softmax_scale"]), int(d["n_ctx"]))
    if call == "union":
        out, _, status = sa.attention(*args)
    elif call == "positions":
        out, status = sa.prefill_positions(*args)
    else:
        out, status = sa.decode(*args)
    torch.cuda.synchronize()
    return out.cpu().numpy(), sa.status_value(status)


@pytest.mark.parametrize("call", CALLS)
def test_v_scales_just_under_the_limit_match_the_oracle(call):
    """Every cell's v_scale drawn from +-[3.9, 4) with the largest float under 4
    on a share of them: no flag, finite outputs, oracle parity at the scaled gate."""
    d = _problem(41, call)
    rng = np.random.default_rng(42)
    vs = rng.uniform(3.9, BELOW, size=d["v_scale"].shape).astype(np.float32)
    vs[rng.random(vs.shape) < 0.3] = BELOW
    vs *= np.where(rng.random(vs.shape) < 0.5, -1.0, 1.0).astype(np.float32)
    d["v_scale"] = vs
    print("case v_scale edge", call, flush=True)
    out, status = _run(call, d, vs)
    assert status == 0, status
    assert np.all(np.isfinite(out))
    ref = oracle.attention_of(d)
    factor = (127 * 4.0) / (127 * 0.05)
    mx, mean = H.error_stats(out, ref)
    print("%s max_abs=%.3e mean_abs=%.3e (gate %.3e / %.3e)" %
          (call, mx, mean, H.MAX_ABS * factor, H.MEAN_ABS * factor), flush=True)
    assert mx <= H.MAX_ABS * factor and mean <= H.MEAN_ABS * factor


@pytest.mark.parametrize("call", CALLS)
@pytest.mark.parametrize("value", [4.0, -4.0, np.inf, -np.inf, np.nan])
def test_v_scale_at_or_past_the_limit_is_flagged(call, value):
    """One chosen resident cell with v_scale 4, -4, +-inf or NaN: STATUS_V_SCALE
    and nothing else, and every output stays finite (that cell's V is dropped)."""
    d = _problem(43, call)
    # a chosen cell on a resident page
    cell = next(int(c) for j in range(d["sel"].shape[0]) for c in d["sel"][j, :d["sel_len"][j]]
                if 0 <= c < d["n_ctx"] and d["page_table"][c // 64] >= 0)
    page = int(d["page_table"][cell // 64])
    vs = d["v_scale"].copy()
    vs[page, :, cell % 64] = value
    print("case v_scale flag", call, value, flush=True)
    out, status = _run(call, d, vs)
    assert status == sa.STATUS_V_SCALE, status
    assert np.all(np.isfinite(out))

