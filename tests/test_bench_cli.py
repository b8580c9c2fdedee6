"""Host-side checks of bench.py (no GPU): the one-GPU scope, the kernel-source
hash that ties the committed counter summaries to the kernel, and the
summaries themselves."""
import os
import re
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
WORKLOADS = ["long-mha", "gqa-32k", "paged", "short-batch", "long-mha-fp8", "paged-fp8", "paged-spec4"]


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_kernel_hash_ignores_comments_and_blank_space(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int a; // note\n/* block\n comment */ int  b;\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    h = bench.kernel_source_hash()
    src.write_text("int a;\n\n int b; // another note\n")
    assert bench.kernel_source_hash() == h
    src.write_text("int a; int c;\n")
    assert bench.kernel_source_hash() != h


@pytest.mark.parametrize("workload", WORKLOADS)
def test_counter_summaries_are_complete(workload):
    """Each bench workload has a trace summary and an HBM-counter summary
    under profiles/, each naming the command that made it (committed files
    only; for the default workload, the trace is of plain `bench.py`) and
    the kernel-source hash it was taken with; the traffic figure is within
    2 % of the algorithmic K+V bytes it states."""
    trace = open(os.path.join(ROOT, "profiles", f"fd_kernels_{workload}_trace.md")).read()
    counters = open(os.path.join(ROOT, "profiles", f"fd_partial_{workload}_counters.md")).read()
    # The default workload's trace is of the default command itself.
    assert f"bench.py --workload {workload}" in counters
    assert f"bench.py --workload {workload}" in trace or (workload == "long-mha" and "-- python3 bench.py\n" in trace)
    for text in (trace, counters):
        assert "rocprofv3 " in text and "_work" not in text
        assert re.search(r"kernel_source_sha256[^:]*:\s*[0-9a-f]{16}", text)
    traffic = float(re.search(rf"traffic_bytes_per_launch\[{re.escape(workload)}\]:\s*([0-9.eE+]+)", counters).group(1))
    alg = int(re.search(r"algorithmic K\+V bytes per launch: (\d+)", counters).group(1))
    assert 1.0 <= traffic / alg <= 1.02
