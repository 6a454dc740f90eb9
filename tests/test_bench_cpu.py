"""bench.py host logic (CPU only): the one-GPU guard, the source hash that
decides whether stored counters still describe the kernels, and the parsing
of rocprofv3's CSV output in --profile mode (on synthetic files)."""
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


def test_stored_counters_file_has_what_bench_reads():
    # profiles/counters.json is written by --profile together with the
    # summaries; bench.py reports roofline.traffic and the counters only
    # while its hash matches the sources (after a kernel change: null until
    # measured again).
    with open(os.path.join(ROOT, "profiles", "counters.json")) as f:
        t = json.load(f)
    assert len(t["kernel_source_hash"]) == len(bench.kernel_source_hash()) == 64
    assert t["fetch_factor"] > 0 and t["write_factor"] > 0
    w = t["workloads"]["dense_8192"]
    for k in ("kernel_ns", "clock_ghz", "bytes", "mfma_busy", "lds_bank_conflict_cycles",
              "mops_x512_equals_2mnk"):
        assert k in w, k


def _write_csv(path, header, rows):
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(str(x) for x in r) + "\n")


def test_profile_csv_parsing(tmp_path):
    d = tmp_path / "pass" / "host" / "1234"
    d.mkdir(parents=True)
    k1 = '"void sg::pingpong16_gemm_kernel<true, 16, false, false, true>(sg::DenseParams)"'
    k2 = '"void at::native::fill_kernel<float>(...)"'
    rows = [(i, k1, 1000 * i, 1000 * i + 700 + i) for i in range(1, 6)] + [(9, k2, 0, 50)]
    _write_csv(d / "trace_kernel_trace.csv",
               ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    trace = bench._csv_rows(str(tmp_path), "kernel_trace.csv")
    name, durs = bench._dominant(trace)
    assert name.startswith("void sg::pingpong16_gemm_kernel") and durs == [701, 702, 703, 704, 705]
    assert bench._short(name) == "pingpong16_gemm_kernel"
    # counters: two dimensions of one dispatch are summed, dispatches averaged
    crow = []
    for did in range(1, 6):
        crow += [(did, k1, "SQ_WAVES", 4), (did, k1, "SQ_WAVES", 4),
                 (did, k1, "SQ_LDS_BANK_CONFLICT", did)]
    crow += [(7, k2, "SQ_WAVES", 99)]
    _write_csv(d / "sq_counter_collection.csv",
               ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], crow)
    c = bench._counter_means(bench._csv_rows(str(tmp_path), "counter_collection.csv"), name, 1, 3)
    assert c == {"SQ_WAVES": 8.0, "SQ_LDS_BANK_CONFLICT": 3.0}   # dispatches 2, 3, 4


def test_profile_keys():
    assert bench.profile_key("dense_8192", None) == "dense_8192"
    assert bench.profile_key("dense_8192", ("io", 16, 0)) == "dense_8192@io16_0"
    assert bench.profile_key("dense_8192", (256, 8)) == "dense_8192@layout256_8"
    assert bench._flops_of({"config": {"M": 2, "N": 3, "K": 4}}) == 48.0
    assert bench._flops_of({"config": {"m_sizes": [1, 2], "N": 3, "K": 4}}) == 72.0
