"""Host-side logic of bench.py that needs no GPU: the one-GPU refusal, the
counter summaries' source-hash guard and the recorded command lines."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stdout + res.stderr


def test_counter_traffic_only_for_matching_sources(monkeypatch):
    for op, workload in (("path", "ctx32k_drift005"), ("select", "ctx32k_drift005"),
                         ("positions", "ctx64k_independent")):
        path = os.path.join(ROOT, "profiles", bench._profile_names(workload, op)[1])
        with open(path) as f:
            rec = json.load(f)
        monkeypatch.setattr(bench, "source_hash", lambda o, h=rec["source_hash"]: h)
        assert bench.counter_traffic(workload, op) == rec["hbm_bytes_per_launch"] > 0
        monkeypatch.setattr(bench, "source_hash", lambda o: "0" * 16)
        assert bench.counter_traffic(workload, op) is None


def test_source_hash_covers_each_ops_sources():
    hashes = {op: bench.source_hash(op) for op in bench.OP_SOURCES}
    assert all(len(h) == 16 for h in hashes.values())
    assert len({hashes["path"], hashes["select"], hashes["positions"]}) == 3
    for op, names in bench.OP_SOURCES.items():
        for name in names:
            assert os.path.exists(os.path.join(ROOT, "sparse_top_selection_amd", "csrc", name))


def test_profile_summaries_name_their_commands():
    # every committed stats summary records the rocprofv3 command that made it,
    # and those commands run committed files only
    pdir = os.path.join(ROOT, "profiles")
    stats = [n for n in os.listdir(pdir) if n.endswith("_stats.txt")]
    assert stats
    for name in stats:
        text = open(os.path.join(pdir, name)).read()
        cmds = [l for l in text.splitlines() if l.startswith("command: rocprofv3")]
        assert cmds, name
        for c in cmds:
            assert "_work" not in c, c
            assert "$REPO/bench.py" in c, c


def test_summaries_are_named_after_the_measured_workload():
    args = bench.parse(["--summarize", "X", "--ctx", "32768", "--queries", "8192", "--drift", "0.76"])
    args.workload = args.workload or bench.DEFAULT_WORKLOAD[args.op]
    name = bench.measured_workload_name(args)
    assert name == "ctx32768_q8192_drift0.76_kv4"
    assert bench._profile_names(name, "path")[0] == "kernels_ctx32768_q8192_drift0.76_kv4_stats.txt"
    args = bench.parse(["--summarize", "X", "--ctx", "32768", "--seed", "7"])
    assert bench.measured_workload_name(args).endswith("_seed7")
    args = bench.parse(["--summarize", "X"])
    args.workload = bench.DEFAULT_WORKLOAD[args.op]
    assert bench.measured_workload_name(args) == "ctx32k_drift005"


def test_measured_limiter_verdicts():
    # cache-fed (HBM carries well under the algorithmic bytes), latency-bound
    # (more than the algorithmic bytes, far below the HBM peak: records of a
    # split call on a small grid) and bandwidth-bound; a call's launches add up
    rec = {"kernels": {"k": {"hbm_bytes": 1.0e9}, "split": {"hbm_bytes": 15e6},
                       "merge": {"hbm_bytes": 5e6}, "stream": {"hbm_bytes": 6.0e9}}}
    v = bench.measured_limiter(rec, ("k",), 3.0e9, 0.72e-3)
    assert v["verdict"].startswith("cache-fed")
    v = bench.measured_limiter(rec, ("split", "merge"), 12e6, 23e-6)
    assert abs(v["hbm_traffic_over_algorithmic_bytes"] - 20 / 12) < 1e-9
    assert v["verdict"].startswith("latency-bound")
    v = bench.measured_limiter(rec, ("stream",), 6.0e9, 1.0e-3)
    assert v["verdict"].endswith("bandwidth-bound") and v["hbm_traffic_frac_of_peak"] == 0.75
    assert bench.measured_limiter(rec, ("k", "absent"), 1.0, 1.0) is None
    assert bench.measured_limiter(None, ("k",), 1.0, 1.0) is None
