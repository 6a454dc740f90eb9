"""bench.py host logic (CPU only): the one-GPU guard and the source hash that
decides whether stored HBM traffic still describes the kernels."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_code_only_ignores_comments_and_blank_lines():
    a = "int x; // one\n\n/* two\n three */ int y;\n"
    b = "int x;   // another\n/* - */ int y;\n\n"
    assert bench._code_only(a) == bench._code_only(b) == "int x;\n int y;"
    assert bench._code_only("int x;") != bench._code_only("int z;")


def test_stored_traffic_file_has_what_bench_reads():
    # profiles/traffic.json is written together with the rocprofv3 summaries;
    # bench.py reports roofline.traffic only while its hash matches the
    # sources (after a kernel change it reports null until re-measured).
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        t = json.load(f)
    assert len(t["kernel_source_hash"]) == len(bench.kernel_source_hash()) == 64
    assert t["fetch_factor"] > 0 and t["write_factor"] > 0
    assert "dense_8192" in t["workloads"]
