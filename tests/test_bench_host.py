"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the per-step time
spread, and the HBM traffic lookup keyed on the kernel source."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


class _Event:
    """Stand-in for a timing event: elapsed_time is the difference of two stamps (ms)."""

    def __init__(self, t):
        self.t = t

    def elapsed_time(self, other):
        return other.t - self.t


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""   # no result line


def test_step_spread_takes_first_to_last_event():
    # 21 steps of 2.0, 2.1, ..., 4.0 ms between their first and last events, in
    # scrambled order; a middle event that would shorten them is ignored.
    times = [2.0 + 0.1 * i for i in range(21)]
    order = [(8 * i) % 21 for i in range(21)]   # a permutation (8 and 21 coprime)
    events = [[_Event(10.0), _Event(10.5), _Event(10.0 + times[i])] for i in order]
    s = bench.step_spread(events)
    assert s == {"median": 3.0, "p10": 2.2, "p90": 3.8}


def test_traffic_is_reported_only_for_the_profiled_source():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    entry = t[bench.DOMINANT]
    workload, rec = next(iter(entry.items()))
    if rec["source_sha"] == bench.source_sha():
        assert bench.load_traffic(workload) == rec["hbm_bytes_per_launch"]
    else:
        assert bench.load_traffic(workload) is None
    assert bench.load_traffic("no-such-workload") is None


def test_kernel_names_match_the_committed_traces():
    """bench.py labels each step with the kernel the launchers pick
    (kernel_name); every profiles/<workload>.md kernel trace, taken from a run of
    the library, must list exactly those kernels for the forward, dK/dV and dQ
    steps."""
    import re
    import workloads
    names = dict(workloads.BY_NAME)
    names.update(workloads.VARLEN_BY_NAME)
    checked = 0
    for fn in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        wname = fn[:-3]
        if not fn.endswith(".md") or wname not in names:
            continue
        text = open(os.path.join(ROOT, "profiles", fn)).read()
        traced = set(re.findall(r"^\| `(\w+_kernel)` \|", text, re.M))
        w = names[wname]
        for step in ("fwd", "dkdv", "dq"):
            assert bench.kernel_name(step, w) in traced, (wname, step, traced)
        checked += 1
    assert checked >= 6
