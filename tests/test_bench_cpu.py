"""Host-side checks of bench.py's bookkeeping (no GPU): the committed HBM
traffic record belongs to the current GEMM source and only to the workload
its counters were read on."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM_SRC = os.path.join(ROOT, "float8linear_tensorwise_amax_amd", "csrc", "gemm.hip")


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_record_matches_the_gemm_source():
    rec = _bench().load_traffic(GEMM_SRC, "linear4096_m4096")
    assert rec is not None, "profiles/gemm_traffic.json was taken on another gemm.hip: re-read the counters"
    scale = rec["copy_calibration"]
    want = rec["fetch_size_kib_per_launch"] * 1024 * scale["fetch_scale"] + \
        rec["write_size_kib_per_launch"] * 1024 * scale["write_scale"]
    assert abs(rec["hbm_bytes_per_launch"] - want) <= 1024


def test_traffic_record_is_not_attached_to_other_workloads():
    b = _bench()
    for w in ("gpt1p5b_block_t12288_delayed", "linear4096_m16", "llama3_8b_layer_t8192"):
        assert b.load_traffic(GEMM_SRC, w) is None


def test_more_than_one_gpu_is_refused_with_a_message():
    import json
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]
