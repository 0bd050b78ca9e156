"""Benchmark of prompt-phase selection attention over INT8 paged K/V on one MI355X.

A step is one pass of the whole path over one prompt chunk: the union kernel
then the attention kernel, on inputs already resident in HBM. The default
workload is the 32K-context chunk: 8,192 query positions (24,576..32,767),
4 KV heads x 12 query heads, head_dim 128, INT8 K/V with per-cell scales behind
a shuffled page table of 512 pages, selections of 3 sinks + own block + 31
drifting blocks (drift 0.05), cap 2,051.

Prints ONE JSON line: the metric (selected query-head-cells per second; prompt
positions per second beside it), the roofline of the dominant kernel measured
with HIP events on its own stream, and the CPU oracle timed on a bounded sample
of the same workload on this host's cores.

`--op select` measures the step before the path instead: block scores -> the
selection rows (top 31 earlier blocks + 3 sinks + own block) of the same
chunk's positions, one kernel launch per step. It prints its own JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense FP16 matrix
# algorithmic bytes per union cell per (group, KV head) workgroup:
#   K row 128 + V row 128 + k_scale 4 + v_scale 4 (the union K/V bytes: 264)
#   + union pool row 4 + chooser byte 1
UNION_KV_BYTES = 264
UNION_CELL_BYTES = UNION_KV_BYTES + 4 + 1   # + union pool row and chooser byte
RIDGE_FLOP_PER_BYTE = F16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
ROW_BYTES = 128 * 4 * 2        # q in + out, per (query position, query head)
FLOP_PER_CELL_ROW = 4 * 128    # QK^T and PV, per (union cell, row)
SELECT_RHO = 0.99              # AR(1) correlation of the block scores across positions
# the kernel each op's roofline and counter summary is about
SPLIT_CALL = ("sel_attn_prefill_split_kernel", "prefill_merge_kernel")   # sel_attn_prefill_split's launches
OP_KERNELS = {"path": ("sel_attn_prefill_kernel", "union_build_kernel") + SPLIT_CALL,
              "select": ("select_blocks_kernel",),
              "positions": ("prefill_positions_kernel",),
              "decode": ("decode_split_kernel", "decode_merge_kernel")}
DEFAULT_WORKLOAD = {"path": "ctx32k_drift005", "select": "ctx32k_drift005",
                    "positions": "ctx64k_independent", "decode": "ctx64k_independent"}
# algorithmic bytes of the per-position kernel: per (position, KV head, listed
# cell) its K and V rows and two scales; per listed cell of a position its
# selection entry and page-table entry; q and out as for the path
POS_CELL_BYTES = 128 + 128 + 4 + 4
POS_ENTRY_BYTES = 4 + 4
# Untimed back-to-back steps before the warm-up steps. The GPU idles while the
# host builds the inputs, and its shader clock then needs tens of milliseconds of
# load to climb back: after a 5-step warm-up the 32K prefill timed 0.736-0.740 ms,
# after 50 or 200 steps 0.703-0.705 ms (one machine, same build).
SETTLE_MS = 100.0
SETTLE_WHY = ("untimed back-to-back steps until the GPU has run them for %.0f ms, before the warm-up "
              "steps: the shader clock climbs back from the idle of the input set-up" % SETTLE_MS)


def settle(step, min_ms: float = SETTLE_MS, max_steps: int = 20000) -> dict:
    """Run `step` untimed, ten at a time, until min_ms of wall time have passed
    (or max_steps); returns what was run, for the JSON line."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < max_steps:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            break
    return {"steps": n, "ms": round((time.perf_counter() - t0) * 1e3, 1), "why": SETTLE_WHY}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="default: ctx32k_drift005 (ctx64k_independent for --op positions)")
    ap.add_argument("--op", choices=("path", "select", "positions", "decode"), default="path",
                    help="path: union + attention (the default); select: the selection step; "
                         "positions: the per-position attention (no union); decode: the last "
                         "--decode-positions positions of the workload, split over their cells")
    ap.add_argument("--decode-positions", type=int, default=1, metavar="N",
                    help="positions per decode call (1 = decode, 5 = a verify window of 4 drafts)")
    ap.add_argument("--sel", metavar="FILE",
                    help="replay recorded selections (.npz from synth.save_selections) instead of "
                         "the workload's own; n_ctx and n_q come from the file")
    ap.add_argument("--ctx", type=int, default=None, metavar="N",
                    help="timing mode: a workload of N context cells built from the arguments "
                         "(with --queries and --drift; the last Q positions, 4 KV heads) instead "
                         "of a named one")
    ap.add_argument("--queries", type=int, default=8192, metavar="Q",
                    help="timing mode: query positions (the last Q of the context)")
    ap.add_argument("--drift", type=float, default=0.05, metavar="F",
                    help="timing mode: share of far-block choices redrawn from one position to "
                         "the next (1.0 = independent selections)")
    ap.add_argument("--kv-heads", type=int, default=4, metavar="H", help="timing mode: KV heads")
    ap.add_argument("--seed", type=int, default=TIMING_SEED, help="timing mode: input seed")
    ap.add_argument("--kv-resident", type=float, default=1.0, metavar="F",
                    help="fraction of logical pages resident; the rest are marked -1 (seeded)")
    ap.add_argument("--cpu-rows", type=int, default=-1,
                    help="query positions of the oracle's timed sample (-1 = all of the chunk, 0 = skip)")
    ap.add_argument("--profile", action="store_true",
                    help="short run for rocprofv3: no CPU leg, plus a 512 MiB copy for counter calibration")
    ap.add_argument("--summarize", metavar="DIR",
                    help="no GPU: turn the rocprofv3 output that profile.sh left in DIR into the "
                         "summaries under profiles/")
    return ap.parse_args(argv)


# the kernel sources behind each op's counters
OP_SOURCES = {"path": ("union_build.hip", "sel_attn_prefill.hip", "sel_attn_prefill_dev.h",
                       "sel_attn_prefill_split.hip"),
              "select": ("select_blocks.hip",),
              "positions": ("prefill_positions.hip",),
              "decode": ("prefill_positions.hip",)}


def _cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def source_hash(op: str = "path") -> str:
    """Hash of the op's kernel sources and the shared argument header: counters
    taken on other bytes are not used."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_top_selection_amd", "csrc")
    for name in sorted(OP_SOURCES[op] + ("sel_attn_internal.h",)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def _profile_names(workload: str, op: str):
    """(stats text, counter json) file names under profiles/ for an op."""
    if op == "path":
        return "kernels_%s_stats.txt" % workload, "prefill_%s_counters.json" % workload
    return "kernels_%s_%s_stats.txt" % (op, workload), "%s_%s_counters.json" % (op, workload)


def counter_record(workload_name: str, op: str = "path"):
    """The committed counter summary of the op on this workload, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", _profile_names(workload_name, op)[1])
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(op):
        return None
    return rec


def counter_traffic(workload_name: str, op: str = "path"):
    """HBM bytes per launch of the op's main kernel from the committed counter
    summary, if it was taken on the current kernel sources; else None."""
    rec = counter_record(workload_name, op)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def measured_limiter(rec, kernels, alg_bytes: float, sec: float):
    """What the counters say bounds the call's kernels (the first is the main
    one): HBM traffic against their algorithmic bytes and against what HBM
    could carry in the measured time, and how busy the matrix cores were."""
    if rec is None or not all(k in rec["kernels"] for k in kernels):
        return None
    traffic = sum(rec["kernels"][k]["hbm_bytes"] for k in kernels)
    hbm_frac = traffic / sec / 1e9 / HBM_PEAK_GBS
    out = {"hbm_traffic_over_algorithmic_bytes": traffic / alg_bytes,
           "hbm_traffic_frac_of_peak": hbm_frac}
    sq = rec.get("sq", {}).get(kernels[0])
    if sq:
        d = sq["derived"]
        out["matrix_core_busy_frac"] = d.get("matrix-core busy / (4 x CU busy cycles)")
        out["valu_beside_matrix_core_frac"] = d.get("VALU beside matrix core / matrix-core busy")
    if out["hbm_traffic_over_algorithmic_bytes"] < 0.5:
        out["verdict"] = ("cache-fed: HBM carries %.2fx the algorithmic bytes, so the kernel is bound by "
                          "instruction issue on the CUs (VALU, LDS and MFMA together), not by HBM"
                          % out["hbm_traffic_over_algorithmic_bytes"])
    elif hbm_frac < 0.3:
        out["verdict"] = ("latency-bound: HBM carries %.2fx the algorithmic bytes but at %.0f%% of its peak, "
                          "so too few work-groups or dependent memory round trips set the time, not "
                          "bandwidth" % (out["hbm_traffic_over_algorithmic_bytes"], 100 * hbm_frac))
    else:
        out["verdict"] = ("HBM carries %.2fx the algorithmic bytes at %.0f%% of its peak: bandwidth-bound"
                          % (out["hbm_traffic_over_algorithmic_bytes"], 100 * hbm_frac))
    return out


COPY_BYTES = 512 << 20         # the calibration copy of --profile: bytes read, and bytes written


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    return name.split("(")[0].split("<")[0].split("::")[-1]


def _sq_summary(d: str, kernels):
    """Mean per dispatch of every SQ counter that the sq1..sq3 passes of
    profile.sh took for each kernel, plus ratios of them: matrix-core busy
    cycles per SIMD-cycle of busy CUs (4 SIMDs per CU), the share of those in
    which VALU work ran beside the matrix core, and instruction counts per
    wave."""
    out = {}
    for sub in ("sq1", "sq2", "sq3"):
        path = os.path.join(d, sub, "pmc_counter_collection.csv")
        if not os.path.exists(path):
            return None
        for r in _csv_rows(path):
            k = _short(r["Kernel_Name"])
            if k not in kernels:
                continue
            acc = out.setdefault(k, {}).setdefault(r["Counter_Name"], {})
            acc[r["Dispatch_Id"]] = acc.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    res = {}
    for k, counters in out.items():
        c = {name: float(np.mean(list(v.values()))) for name, v in counters.items()}
        waves = c.get("SQ_WAVES", 0.0)
        derived = {}
        if c.get("SQ_BUSY_CU_CYCLES"):
            derived["matrix-core busy / (4 x CU busy cycles)"] = \
                c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4.0 * c["SQ_BUSY_CU_CYCLES"])
        if c.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            derived["VALU beside matrix core / matrix-core busy"] = \
                c.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / c["SQ_VALU_MFMA_BUSY_CYCLES"]
        if waves:
            for name in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VALU_TRANS_F32"):
                if name in c:
                    derived[name + " per wave"] = c[name] / waves
        if c.get("SQ_ACTIVE_INST_LDS"):
            derived["LDS bank-conflict cycles / LDS active cycles"] = \
                c.get("SQ_LDS_BANK_CONFLICT", 0.0) / c["SQ_ACTIVE_INST_LDS"]
        res[k] = {"counters": c, "derived": derived}
    return res


def summarize(d: str, workload: str, op: str = "path"):
    """Summaries of a profile.sh run: the kernel-trace statistics as text, and the
    HBM bytes per launch of the op's kernels from FETCH_SIZE / WRITE_SIZE, each
    counter scaled by what it reads for a copy of COPY_BYTES (the copy kernel
    with the largest grid in the run)."""
    stats_name, counters_name = _profile_names(workload, op)
    kernels = OP_KERNELS[op]
    with open(os.path.join(d, "commands.txt")) as f:
        commands = f.read().strip().splitlines()
    stats = _csv_rows(os.path.join(d, "trace", "run_kernel_stats.csv"))
    lines = ["rocprofv3 --kernel-trace --stats summary, workload %s%s" % (
                 workload, "" if op == "path" else ", op " + op),
             "command: " + commands[0], "",
             "%-30s %6s %12s %12s %12s %12s" % ("kernel", "calls", "avg_us", "min_us", "max_us", "total_%")]
    for r in stats:
        lines.append("%-30s %6s %12.2f %12.2f %12.2f %12.2f" % (
            _short(r["Name"])[:30], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", stats_name), "w") as f:
        f.write("\n".join(lines) + "\n")

    rec = {"workload": workload, "source_hash": source_hash(op), "commands": commands[1:3],
           "copy_bytes": COPY_BYTES, "kernels": {}}
    for counter, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        rows = [r for r in _csv_rows(os.path.join(d, sub, "pmc_counter_collection.csv"))
                if r["Counter_Name"] == counter]
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"] or "copy" in _short(r["Kernel_Name"]).lower()]
        big = max(int(r["Grid_Size"]) for r in copies)
        copy_kib = np.mean([float(r["Counter_Value"]) for r in copies if int(r["Grid_Size"]) == big])
        factor = COPY_BYTES / (copy_kib * 1024.0)
        rec[counter] = {"copy_KiB": copy_kib, "factor": factor}
        for k in kernels:
            v = [float(r["Counter_Value"]) for r in rows if _short(r["Kernel_Name"]) == k]
            if not v:   # not launched by this workload (the merge of a split prefill)
                continue
            ent = rec["kernels"].setdefault(k, {})
            ent[counter + "_KiB_per_dispatch"] = float(np.mean(v))
            ent[counter.split("_")[0].lower() + "_bytes"] = float(np.mean(v)) * 1024.0 * factor
    for ent in rec["kernels"].values():
        ent["hbm_bytes"] = ent["fetch_bytes"] + ent["write_bytes"]
    # the op's call: its first kernel, or for a split attention call its two launches
    main = SPLIT_CALL if op == "path" and kernels[0] not in rec["kernels"] else kernels[:1]
    rec["hbm_bytes_per_launch"] = sum(rec["kernels"][k]["hbm_bytes"] for k in main)
    with open(os.path.join(ROOT, "profiles", counters_name), "w") as f:
        json.dump(rec, f, indent=1)
    lines += ["", "HBM bytes per dispatch from counters (two --pmc runs, one counter each):"]
    lines += ["command: " + c for c in commands[1:3]]
    lines.append("calibration: a %d MiB device copy reads FETCH_SIZE %.0f KiB (factor %.4f) and "
                 "WRITE_SIZE %.0f KiB (factor %.4f)" % (
                     COPY_BYTES >> 20, rec["FETCH_SIZE"]["copy_KiB"], rec["FETCH_SIZE"]["factor"],
                     rec["WRITE_SIZE"]["copy_KiB"], rec["WRITE_SIZE"]["factor"]))
    for k, ent in rec["kernels"].items():
        lines.append("%-30s FETCH %.0f KiB -> %.1f MB, WRITE %.0f KiB -> %.1f MB, total %.1f MB" % (
            k, ent["FETCH_SIZE_KiB_per_dispatch"], ent["fetch_bytes"] / 1e6,
            ent["WRITE_SIZE_KiB_per_dispatch"], ent["write_bytes"] / 1e6, ent["hbm_bytes"] / 1e6))
    sq = _sq_summary(d, kernels)
    if sq:
        rec["sq"] = sq
        lines += ["", "SQ counters per dispatch (three --pmc runs of at most 8 SQ counters each):"]
        lines += ["command: " + c for c in commands[3:6]]
        for k, ent in sq.items():
            lines.append("%s:" % k)
            for name in sorted(ent["counters"]):
                lines.append("  %-28s %16.6g" % (name, ent["counters"][name]))
            for name, v in ent["derived"].items():
                lines.append("  %-44s %10.4g" % (name, v))
        with open(os.path.join(ROOT, "profiles", counters_name), "w") as f:
            json.dump(rec, f, indent=1)
    lines.append("kernel sources: sha256 prefix %s (the benchmark uses these bytes only while it "
                 "matches)" % rec["source_hash"])
    extra = ("" if op == "path" else " --op " + op) + \
        ("" if workload == DEFAULT_WORKLOAD[op] else " --workload " + workload)
    lines.append("made by: bash profile.sh OUTDIR%s; python3 bench.py --summarize OUTDIR%s" % (
        extra, extra))
    with open(os.path.join(ROOT, "profiles", stats_name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(open(os.path.join(ROOT, "profiles", stats_name)).read())
    print(json.dumps(rec, indent=1))


TIMING_SEED = 2000   # the timing mode's default input seed


def timing_workload(args):
    """The workload of the timing mode: the 32K chunk's recipe (INT8 pools with
    per-cell scales behind a shuffled page table, 3 sinks + own block + 31 far
    blocks) at the context, position count, drift and KV-head count given."""
    import synth
    if not (0 < args.queries <= args.ctx):
        raise SystemExit("--queries must be in [1, --ctx]")
    if not (0.0 <= args.drift <= 1.0):
        raise SystemExit("--drift must be in [0, 1]")
    name = "ctx%d_q%d_drift%g_kv%d" % (args.ctx, args.queries, args.drift, args.kv_heads)
    if args.seed != TIMING_SEED:
        name += "_seed%d" % args.seed
    return dataclasses.replace(synth.workload(synth.HEADLINE), name=name, n_ctx=args.ctx,
                               n_q=args.queries, n_kv=args.kv_heads, drift=args.drift,
                               seed=args.seed, n_pages=None)


def measured_workload_name(args) -> str:
    """The name of the workload a run with these arguments measures (the timing
    mode's, else --workload's): profile summaries and counter records use it."""
    return timing_workload(args).name if args.ctx else args.workload


def main():
    args = parse()
    if args.workload is None:
        args.workload = DEFAULT_WORKLOAD[args.op]
    if args.summarize:
        summarize(args.summarize, measured_workload_name(args), args.op)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this path is measured on a single MI355X "
              "(the work units are independent; see the sharding notes). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import sparse_top_selection_amd as sa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.op == "select":
        bench_select(args)
        return
    if args.op == "decode":
        bench_decode(args)
        return
    dev = torch.device("cuda:0")
    w = timing_workload(args) if args.ctx else synth.workload(args.workload)
    label = w.name
    if args.sel:
        rec = synth.load_selections(args.sel)
        w = dataclasses.replace(w, n_ctx=rec["n_ctx"], n_q=rec["sel"].shape[0],
                                sel_cap=rec["sel"].shape[1])
        inp = synth.generate(w, with_sel=False)
        inp["sel"], inp["sel_len"] = rec["sel"], rec["sel_len"]
        label = "replay:%s (pools of %s)" % (os.path.basename(args.sel), label)
    else:
        inp = synth.generate(w)
    inp = synth.as_problem(inp)
    if args.kv_resident < 1.0:
        inp["page_table"] = synth.drop_pages(inp["page_table"], args.kv_resident, seed=w.seed)
        label += " resident %.2f" % args.kv_resident

    # work counts of this input
    sel, sel_len, pt = inp["sel"], inp["sel_len"], inp["page_table"]
    resident_cells = 0
    for j in range(w.n_q):
        row = np.unique(sel[j, :sel_len[j]])
        resident_cells += int(np.count_nonzero(pt[row // 64] >= 0))
    q_head_cells = resident_cells * w.n_qh

    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
         for k in ("q", "k_pool", "v_pool", "k_scale", "v_scale", "page_table", "sel", "sel_len")}
    g = w.n_groups
    cap = w.sel_cap
    cells = torch.empty((g, 8 * cap), dtype=torch.int32, device=dev)
    mask = torch.empty((g, 8 * cap), dtype=torch.uint8, device=dev)
    rows = torch.empty((g, 8 * cap), dtype=torch.int32, device=dev)
    length = torch.empty(g, dtype=torch.int32, device=dev)
    out = torch.empty_like(t["q"])
    status = sa.new_status(dev)
    dims = sa.make_dims(w.n_ctx, w.n_q, w.n_kv, w.pool_pages, sel_cap=cap)
    scale = float(inp["softmax_scale"])
    stream = torch.cuda.current_stream(dev)

    positions = args.op == "positions"
    # grids too small to fill the GPU take the split call (workspace allocated here,
    # outside the timed steps); the others the plain call, which is the same kernel
    split_bytes = 0 if positions else sa.sel_attn_prefill_workspace_bytes(dims)
    workspace = torch.empty(max(split_bytes, 16), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if not positions:
            sa.sel_attn_build_union(dims, t["sel"], t["sel_len"], t["page_table"], cells, mask,
                                    rows, length, status, stream)
        if ev is not None:
            ev[1].record(stream)
        if positions:
            sa.sel_attn_prefill_positions(dims, t["q"], t["k_pool"], t["v_pool"], t["k_scale"],
                                          t["v_scale"], t["page_table"], t["sel"], t["sel_len"],
                                          scale, out, status, stream)
        elif split_bytes:
            sa.sel_attn_prefill_split(dims, t["q"], t["k_pool"], t["v_pool"], t["k_scale"],
                                      t["v_scale"], rows, mask, length, scale, out, status,
                                      workspace, split_bytes, stream)
        else:
            sa.sel_attn_prefill(dims, t["q"], t["k_pool"], t["v_pool"], t["k_scale"],
                                t["v_scale"], rows, mask, length, scale, out, status, stream)
        if ev is not None:
            ev[2].record(stream)

    settled = None if args.profile else settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    sa.check_status(status)

    steps = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sa.check_status(status)
    union_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    prefill_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms_per_step = wall / steps * 1e3

    if positions:
        # every (position, KV head) gathers its own resident cells
        alg_bytes = resident_cells * (w.n_kv * POS_CELL_BYTES + POS_ENTRY_BYTES) + \
            w.n_q * w.n_qh * ROW_BYTES
        kv_bytes = resident_cells * w.n_kv * UNION_KV_BYTES
        flops = q_head_cells * FLOP_PER_CELL_ROW
    else:
        lens = length.cpu().numpy().astype(np.int64)
        union_cells = int(lens.sum())
        alg_bytes = union_cells * w.n_kv * UNION_CELL_BYTES + w.n_q * w.n_qh * ROW_BYTES
        kv_bytes = union_cells * w.n_kv * UNION_KV_BYTES
        flops = union_cells * w.n_kv * 96 * FLOP_PER_CELL_ROW
    sec = prefill_ms * 1e-3
    # the committed counters were taken on the workload's own inputs (a timing-mode
    # workload's name holds every argument that shapes its inputs)
    custom = bool(args.sel or args.kv_resident < 1.0)
    rec = None if custom else counter_record(w.name, args.op)
    # the kernels of the timed attention call (a split call: its two launches)
    call_kernels = (("prefill_positions_kernel",) if positions else
                    SPLIT_CALL if split_bytes else ("sel_attn_prefill_kernel",))
    kernel = " + ".join(call_kernels)
    traffic = None
    if rec is not None and all(k in rec["kernels"] for k in call_kernels):
        traffic = sum(rec["kernels"][k]["hbm_bytes"] for k in call_kernels)
    kv_gbps = kv_bytes / sec / 1e9
    if positions:
        # The gathered rows (every listed cell of every position) are mostly
        # re-reads that the L2 and the last-level cache serve, so their rate
        # exceeds what HBM alone delivers; the roofline line is stated on the
        # bytes HBM actually carried (counters), which it can meet.
        roofline = {
            "kernel": kernel, "bound": "hbm",
            "basis": "HBM bytes per launch from the FETCH_SIZE / WRITE_SIZE counters",
            "achieved": None if traffic is None else traffic / sec / 1e9,
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": None if traffic is None else traffic / sec / 1e9 / HBM_PEAK_GBS,
            "traffic": traffic,
            "gathered_bytes": {"bytes_per_launch": alg_bytes, "effective_GBps": alg_bytes / sec / 1e9,
                               "note": "every gathered row counted; most are cache hits"},
        }
    else:
        intensity = flops / kv_bytes
        roofline = {
            "kernel": kernel,
            # by arithmetic intensity against the MI355X ridge (2.5 PFLOP/s / 8 TB/s)
            "bound": "hbm" if intensity < RIDGE_FLOP_PER_BYTE else "mfma",
            "basis": "union K/V bytes: 264 B per union cell and KV head (K and V rows, two fp32 scales)",
            "achieved": kv_gbps, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": kv_gbps / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes,
            "intensity_flop_per_byte": intensity,
            "ridge_flop_per_byte": RIDGE_FLOP_PER_BYTE,
            "with_indices_and_q_out": {
                "basis": "+ 5 B of union pool row and chooser byte per union cell and KV head, "
                         "+ 98,304 B of q in and out per work-group",
                "bytes_per_launch": alg_bytes, "achieved": alg_bytes / sec / 1e9,
                "frac": alg_bytes / sec / 1e9 / HBM_PEAK_GBS},
            "mfma": {"achieved_tflops": flops / sec / 1e12, "peak_tflops": F16_MFMA_PEAK_TFLOPS,
                     "frac": flops / sec / 1e12 / F16_MFMA_PEAK_TFLOPS},
            "measured_limiter": measured_limiter(rec, call_kernels, kv_bytes, sec),
        }

    if args.profile:
        # plain copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    result = {
        "metric": ("selected query-head-cells/s (per-position attention, %s)" % w.name if positions
                   else "selected query-head-cells/s (32K-context prompt chunk)"
                   if w.name == synth.workload(synth.HEADLINE).name
                   else "selected query-head-cells/s (%s)" % w.name),
        "value": q_head_cells / (ms_per_step * 1e-3),
        "unit": "query-head-cells/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup, "settle": settled,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 K/V, fp16 products, fp32 softmax and sums",
        "data": "synthetic (seeded; shapes of the pages' parity self-test)",
        "config": {
            "workload": label,
            "n_ctx": w.n_ctx, "query_positions": w.n_q, "first_position": w.first_pos,
            "kv_heads": w.n_kv, "q_heads_per_kv": w.q_per_kv, "head_dim": w.head_dim,
            "page_size": w.page_size, "pool_pages": w.pool_pages, "sel_cap": w.sel_cap,
            "drift": w.drift, "parallelism": "single GPU",
        },
        "prompt_positions_per_s": w.n_q / (ms_per_step * 1e-3),
        "kernels_ms": ({"prefill_positions": prefill_ms} if positions
                       else {"union_build": union_ms, "prefill": prefill_ms}),
        "kv_GBps": kv_gbps,
        "kv_frac_of_hbm_peak": kv_gbps / HBM_PEAK_GBS,
        "mfma_frac_of_f16_peak": flops / sec / 1e12 / F16_MFMA_PEAK_TFLOPS,
        "roofline": roofline,
        "source_hash": source_hash(args.op),
    }
    if not positions:
        result["union"] = {"cells": union_cells, "mean_per_group": union_cells / g,
                           "ratio_to_mean_selection": (union_cells / g) / float(sel_len.mean())}
        result["prefill_call"] = ("sel_attn_prefill_split (%d work-groups per (group, KV head), "
                                  "then the merge)" % (split_bytes // (g * w.n_kv * 49920))
                                  if split_bytes else "sel_attn_prefill")

    if args.cpu_rows != 0 and not args.profile:
        import oracle
        n_rows = w.n_q if args.cpu_rows < 0 else min(args.cpu_rows, w.n_q)
        rows = np.arange(n_rows, dtype=np.int32)
        cores = oracle.max_threads()
        c0 = time.perf_counter()
        ref = oracle.attention_of(inp, rows=rows, n_threads=cores)
        cpu_s = time.perf_counter() - c0
        sample_cells = 0
        for j in rows:
            row = np.unique(sel[j, :sel_len[j]])
            sample_cells += int(np.count_nonzero(pt[row // 64] >= 0))
        got = out[:n_rows].cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        result["cpu_baseline"] = {
            "value": sample_cells * w.n_qh / cpu_s,
            "unit": "query-head-cells/s",
            "cores": cores,
            "kind": "oracle",
            "sample": "query positions 0..%d of the same chunk (%d of %d), FP64 per-position "
                      "gather, %.1f s" % (n_rows - 1, n_rows, w.n_q, cpu_s),
            "positions_per_s": n_rows / cpu_s,
            "cpu_model": _cpu_model(),
        }
        # the same oracle on one thread, over a sixteenth of the sample
        n1 = max(1, min(n_rows, n_rows // 16))
        c0 = time.perf_counter()
        oracle.attention_of(inp, rows=rows[:n1], n_threads=1)
        one_s = time.perf_counter() - c0
        one_cells = 0
        for j in rows[:n1]:
            row = np.unique(sel[j, :sel_len[j]])
            one_cells += int(np.count_nonzero(pt[row // 64] >= 0))
        result["cpu_baseline"]["one_core"] = {
            "value": one_cells * w.n_qh / one_s, "positions_per_s": n1 / one_s,
            "sample": "query positions 0..%d, %.1f s" % (n1 - 1, one_s)}
        result["parity_on_cpu_sample"] = {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
                                          "out_rms": float(np.sqrt(np.mean(ref ** 2)))}
    print(json.dumps(result), flush=True)


def bench_decode(args):
    """The decode call on the workload's last N positions (its pools, q and
    selections): one call per step, timed like the selection step (one event
    pair around K back-to-back calls queued behind device copies)."""
    import torch
    import synth
    import sparse_top_selection_amd as sa

    dev = torch.device("cuda:0")
    w = synth.workload(args.workload)
    nd = args.decode_positions
    inp = synth.as_problem(synth.generate(w))
    for k in ("q", "sel", "sel_len"):
        inp[k] = np.ascontiguousarray(inp[k][-nd:])
    inp["n_q"] = nd
    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
         for k in ("q", "k_pool", "v_pool", "k_scale", "v_scale", "page_table", "sel", "sel_len")}
    out = torch.empty_like(t["q"])
    status = sa.new_status(dev)
    dims = sa.make_dims(w.n_ctx, nd, w.n_kv, w.pool_pages, sel_cap=w.sel_cap)
    ws_bytes = sa.sel_attn_decode_workspace_bytes(dims)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    scale = float(inp["softmax_scale"])
    stream = torch.cuda.current_stream(dev)

    def launch():
        sa.sel_attn_decode(dims, t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"],
                           t["page_table"], t["sel"], t["sel_len"], scale, out, ws, ws_bytes,
                           status, stream)

    settled = None if args.profile else settle(launch)
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    sa.check_status(status)
    steps = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if not args.profile:
        busy_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        busy_dst = torch.empty_like(busy_src)
        torch.cuda.synchronize()
        for _ in range(8 + steps // 4):   # ~0.2 ms each; enqueueing a call takes ~50 us
            busy_dst.copy_(busy_src)
    e0.record(stream)
    for _ in range(steps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    sa.check_status(status)
    us = e0.elapsed_time(e1) / steps * 1e3

    pt = inp["page_table"]
    cells = 0
    for j in range(nd):
        row = np.unique(inp["sel"][j, :inp["sel_len"][j]])
        cells += int(np.count_nonzero(pt[row // 64] >= 0))
    alg_bytes = cells * (w.n_kv * POS_CELL_BYTES + POS_ENTRY_BYTES) + nd * w.n_qh * ROW_BYTES
    achieved = alg_bytes / (us * 1e-6) / 1e9
    if args.profile:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    result = {
        "metric": "decode attention latency (%d position%s at the end of %s)" % (
            nd, "" if nd == 1 else "s", w.name),
        "value": us, "unit": "us", "n_gpus": 1, "steps": steps, "warmup": args.warmup, "settle": settled,
        "ms_per_step": us * 1e-3, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8 K/V, fp16 products, fp32 softmax and sums",
        "data": "synthetic (seeded; the workload's last positions)",
        "config": {"workload": "decode%d_%s" % (nd, w.name), "n_ctx": w.n_ctx, "positions": nd,
                   "kv_heads": w.n_kv, "cells": cells, "splits": (w.sel_cap + 63) // 64,
                   "parallelism": "single GPU"},
        "timing": "one HIP event pair around K back-to-back calls queued behind device copies",
        "roofline": {"kernel": "decode_split_kernel + decode_merge_kernel", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": alg_bytes},
        "source_hash": source_hash("decode"),
    }
    if args.cpu_rows != 0 and not args.profile:
        import oracle
        cores = oracle.max_threads()
        c0 = time.perf_counter()
        reps = 0
        while True:
            ref = oracle.attention_of(inp, n_threads=cores)
            reps += 1
            if time.perf_counter() - c0 > 1.0:
                break
        cpu_s = (time.perf_counter() - c0) / reps
        err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
        result["cpu_baseline"] = {"value": cpu_s * 1e6, "unit": "us", "cores": cores,
                                  "kind": "oracle", "cpu_model": _cpu_model(),
                                  "sample": "the same %d position(s), FP64, %d repeats" % (nd, reps)}
        result["parity_on_cpu_sample"] = {"max_abs": float(err.max()), "mean_abs": float(err.mean())}
    print(json.dumps(result), flush=True)


def bench_select(args):
    """The selection step on the chunk's positions: one launch per step.

    A launch takes about as long as the host needs to enqueue it, so the timed
    launches are queued behind device copies that outlast the enqueueing. One pair of HIP events
    on the launch stream then brackets all K launches, which run back to back,
    and the average launch time is their span divided by K.
    """
    import torch
    import synth
    import sparse_top_selection_amd as sa

    dev = torch.device("cuda:0")
    w = synth.workload(args.workload)
    first = w.n_ctx - w.n_q
    scores_np = synth.block_scores(w.n_q, w.n_ctx, SELECT_RHO, seed=w.seed)
    scores = torch.from_numpy(scores_np).to(dev)
    sel = torch.empty((w.n_q, w.sel_cap), dtype=torch.int32, device=dev)
    sel_len = torch.empty(w.n_q, dtype=torch.int32, device=dev)
    dims = sa.make_dims(w.n_ctx, w.n_q, 1, 1, sel_cap=w.sel_cap)
    stream = torch.cuda.current_stream(dev)

    def launch():
        sa.sel_attn_select_blocks(dims, first, scores, sel, sel_len, stream)

    settled = None if args.profile else settle(launch)
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    steps = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if not args.profile:   # the counter runs calibrate on the one copy size below
        busy_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        busy_dst = torch.empty_like(busy_src)
        torch.cuda.synchronize()
        for _ in range(8 + steps // 8):   # ~0.2 ms each; enqueueing a launch takes ~25 us
            busy_dst.copy_(busy_src)
    e0.record(stream)
    for _ in range(steps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    kern_ms = e0.elapsed_time(e1) / steps

    lens = sel_len.cpu().numpy().astype(np.int64)
    own = np.arange(first, w.n_ctx) // 64
    read_bytes = 4 * int(np.where(own > 31, own, 0).sum())   # the scores the kernel reads
    write_bytes = 4 * int(lens.sum()) + 4 * w.n_q            # rows and lengths
    alg_bytes = read_bytes + write_bytes
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9

    if args.profile:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    result = {
        "metric": "selection rows/s (positions of the 32K-context prompt chunk, from block scores)",
        "value": w.n_q / (kern_ms * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup, "settle": settled,
        "ms_per_step": kern_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 scores, int32 cells",
        "data": "synthetic (seeded AR(1) block scores, rho %.2f)" % SELECT_RHO,
        "config": {"workload": "select_" + w.name, "n_ctx": w.n_ctx, "query_positions": w.n_q,
                   "first_position": first, "blocks": -(-w.n_ctx // 64), "sel_cap": w.sel_cap,
                   "parallelism": "single GPU"},
        "timing": "one HIP event pair around K back-to-back launches queued behind device copies",
        "mean_sel_len": float(lens.mean()),
        "roofline": {
            "kernel": "select_blocks_kernel",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": counter_traffic(w.name, "select"),
            "algorithmic_bytes_per_launch": alg_bytes,
        },
        "source_hash": source_hash("select"),
    }
    if args.cpu_rows != 0 and not args.profile:
        from oracle import selection as S
        n_rows = w.n_q if args.cpu_rows < 0 else min(args.cpu_rows, w.n_q)
        c0 = time.perf_counter()
        ref, ref_len = S.select_blocks(scores_np[:n_rows], first, w.n_ctx, w.sel_cap)
        cpu_s = time.perf_counter() - c0
        got = sel[:n_rows].cpu().numpy()
        valid = np.arange(w.sel_cap)[None, :] < ref_len[:, None]
        same = bool(np.array_equal(lens[:n_rows], ref_len) and np.array_equal(got[valid], ref[valid]))
        result["cpu_baseline"] = {
            "value": n_rows / cpu_s, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": "positions %d..%d (%d rows), numpy per-row sort, %.1f s" % (
                first, first + n_rows - 1, n_rows, cpu_s)}
        result["parity_on_cpu_sample"] = {"rows_bit_exact": same}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
