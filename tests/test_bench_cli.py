"""bench.py's command line without a GPU: it measures one GPU only and says so for more."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    for n in ("2", "8"):
        res = run_bench("--gpus", n)
        assert res.returncode == 2, res
        assert "one GPU" in res.stderr, res.stderr
        assert res.stdout == ""  # no JSON line


def test_help_lists_the_contract_flags():
    res = run_bench("--help")
    assert res.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--kernel", "--partition"):
        assert flag in res.stdout


def test_block_size_must_be_a_multiple_of_16():
    for bs in ("8", "24"):
        res = run_bench("--block-size", bs)
        assert res.returncode == 2, res
        assert "multiple of 16" in res.stderr, res.stderr
        assert res.stdout == ""

