"""Host logic of bench.py that runs without a GPU: the multi-GPU refusal and the HBM
traffic record, which is reported only while the GEMM source is the one the counters
were taken on."""
import hashlib
import importlib.util
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_follows_the_gemm_source(tmp_path):
    bench = _load_bench()
    prof = os.path.join(ROOT, "profiles", "gate_up_gemm_hbm_counters.md")
    src = os.path.join(ROOT, "bitwise_consistent_rl_amd", "csrc", "gemm.hip")
    rec = bench.gate_up_traffic()
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if f"sha256={digest}" in open(prof).read():
        # the committed counters belong to the committed kernel: bytes per launch at
        # M = 16384, at least the launch's algorithmic bytes (A, W and C once)
        assert rec is not None and rec["m"] == 16384
        algorithmic = (16384 * 2048 + 12288 * 2048 + 16384 * 6144) * 2
        assert rec["bytes_per_launch"] >= algorithmic
    else:
        assert rec is None
    # a copy of the tree whose gemm.hip differs by one byte: no traffic figure
    (tmp_path / "profiles").mkdir()
    (tmp_path / "bitwise_consistent_rl_amd" / "csrc").mkdir(parents=True)
    shutil.copy(prof, tmp_path / "profiles")
    data = open(src, "rb").read() + b"\n"
    (tmp_path / "bitwise_consistent_rl_amd" / "csrc" / "gemm.hip").write_bytes(data)
    bench.ROOT = str(tmp_path)
    assert bench.gate_up_traffic() is None
    # and the same copy with the original bytes: the record again
    (tmp_path / "bitwise_consistent_rl_amd" / "csrc" / "gemm.hip").write_bytes(open(src, "rb").read())
    assert bench.gate_up_traffic() == rec
