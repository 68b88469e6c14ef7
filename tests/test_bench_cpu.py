"""Host-side checks of bench.py's bookkeeping (no GPU): a committed HBM
traffic record is attached only to the workload its counters were read on,
and only while the GEMM source is the one they were read on."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM_SRC = os.path.join(ROOT, "float8linear_tensorwise_amax_amd", "csrc", "gemm.hip")


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _records():
    import json
    return json.load(open(os.path.join(ROOT, "profiles", "gemm_traffic.json")))["records"]


def test_traffic_records_are_consistent():
    """Each record's HBM bytes are its two counters times the copy calibration."""
    for name, rec in _records().items():
        scale = rec["copy_calibration"]
        want = rec["fetch_size_kib_per_launch"] * 1024 * scale["fetch_scale"] + \
            rec["write_size_kib_per_launch"] * 1024 * scale["write_scale"]
        assert abs(rec["hbm_bytes_per_launch"] - want) <= 1024, name
        assert rec["workload_name"] == name


def test_traffic_record_is_attached_only_to_its_workload_and_source():
    b = _bench()
    recs = _records()
    current = b.sha256_of(GEMM_SRC)
    for w in ("gpt1p5b_block_t12288_delayed", "linear4096_m16", "llama3_8b_layer_t8192", "linear4096_m4096",
              "linear4096_m65536_outliers"):
        got = b.load_traffic(GEMM_SRC, w)
        rec = recs.get(w)
        if rec is not None and rec["source_sha256"] == current:
            assert got is rec or got == rec
        else:
            assert got is None, w


def test_more_than_one_gpu_is_refused_with_a_message():
    import json
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]
