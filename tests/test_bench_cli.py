"""bench.py's command-line contract on the CPU: the cases it must refuse
before touching a GPU (more than one GPU, a bucket size where none applies)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("n", ["2", "8"])
def test_bench_refuses_more_than_one_gpu(n):
    r = _run("--gpus", n)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("args", [["--workload", "tiny", "--bucket-numel", "1024"],
                                  ["--workload", "rs_ag", "--bucket-numel", "1024"],
                                  ["--bucket-numel", "-5"]])
def test_bench_refuses_bucket_size_where_none_applies(args):
    r = _run(*args)
    assert r.returncode == 2
    assert "--bucket-numel" in r.stderr and r.stdout == ""
