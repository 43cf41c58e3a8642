"""Host-side contract checks (no GPU): the binding has no fallback when the
library is missing, and the bench refuses more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

from sparse_long_context_ekv_amd import ekv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_binding_raises_without_library(tmp_path):
    with pytest.raises(FileNotFoundError):
        ekv.load(str(tmp_path / "libekv.so"))


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_bench_refuses_several_gpus(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == int(gpus)
