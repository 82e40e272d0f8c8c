"""Host-side behaviour of bench.py that needs no GPU: the one-GPU message,
the training mode's workload check, and the key of its traffic table."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args):
    return subprocess.run([sys.executable, BENCH, *args], cwd=ROOT, capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_training_mode_refuses_a_multi_layer_workload():
    r = _run("--backward", "--workload", "effnet_b0_mbconv", "--no-cpu-baseline")
    assert r.returncode == 2
    assert "not a single-layer workload" in r.stderr


def test_traffic_table_is_keyed_to_the_current_kernel_sources():
    """The HBM counters in the traffic table were taken on the fused kernel
    built from the sources bench.py hashes; bench.py reports traffic only
    while that hash matches, so the table and the sources must agree."""
    spec = importlib.util.spec_from_file_location("bench_mod", BENCH)
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    assert all(os.path.exists(f) for f in bench.KERNEL_SOURCES)
    sha = bench.source_sha()
    assert len(sha) == 16
    assert bench.TRAFFIC["resnet50_3x3"]["source_sha"] == sha
