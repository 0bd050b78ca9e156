"""Helpers for the GPU parity tests: move a synthetic problem to the device, run
the HIP path through the C ABI binding, compare with the CPU oracle."""
import numpy as np
import torch

import sparse_top_selection_amd as sa

# Tolerance on the attention output against the FP64 oracle. The products take
# Q, K, V and the probabilities in FP16 and sum in FP32; the pages report
# 2.6e-3 to 5.0e-3 max error against FP64 for such a kernel.
MAX_ABS = 8e-3
MEAN_ABS = 1e-3


def to_device(problem: dict, device="cuda") -> dict:
    out = {}
    for key in ("q", "k_pool", "v_pool", "k_scale", "v_scale", "page_table", "sel", "sel_len"):
        out[key] = torch.from_numpy(np.ascontiguousarray(problem[key])).to(device)
    return out


def run_path(problem: dict, dev: dict = None):
    """One pass: union then attention. Returns numpy (out, cells, mask, length, status)."""
    if dev is None:
        dev = to_device(problem)
    out, (cells, mask, _, length), status = sa.attention(
        dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
        dev["page_table"], dev["sel"], dev["sel_len"], float(problem["softmax_scale"]),
        int(problem["n_ctx"]))
    torch.cuda.synchronize()
    return (out.cpu().numpy(), cells.cpu().numpy(), mask.cpu().numpy(), length.cpu().numpy(),
            sa.status_value(status))


def assert_union_equal(cells, mask, length, ref):
    rc, rm, rl = ref
    assert np.array_equal(length, rl), "union lengths differ"
    valid = np.arange(cells.shape[1])[None, :] < rl[:, None]
    bad = np.argwhere(valid & ((cells != rc) | (mask != rm)))
    assert bad.size == 0, "union differs at (group, index) %s" % (bad[:5].tolist(),)


def assert_union_rows_equal(rows, length, ref_rows):
    valid = np.arange(rows.shape[1])[None, :] < length[:, None]
    bad = np.argwhere(valid & (rows != ref_rows))
    assert bad.size == 0, "union rows differ at (group, index) %s" % (bad[:5].tolist(),)


def error_stats(got: np.ndarray, ref: np.ndarray):
    err = np.abs(got.astype(np.float64) - ref)
    return float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    assert np.all(np.isfinite(got)), "non-finite output " + what
    mx, mean = error_stats(got, ref)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    print("%s max_abs=%.3e mean_abs=%.3e out_rms=%.3e" % (what, mx, mean, rms), flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS, (what, mx, mean)


def sample_rows(n_q: int, n_groups_sampled: int, seed: int = 0) -> np.ndarray:
    """Whole groups of 8: the first, the last (possibly ragged) and random ones."""
    g_total = (n_q + 7) // 8
    rng = np.random.default_rng(seed)
    gs = {0, g_total - 1}
    if g_total > 2:
        gs |= set(rng.choice(np.arange(1, g_total - 1), size=min(n_groups_sampled, g_total - 2),
                             replace=False).tolist())
    rows = [j for g in sorted(gs) for j in range(8 * g, min(8 * g + 8, n_q))]
    return np.array(rows, np.int32)
