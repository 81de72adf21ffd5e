"""Host-side contract checks that need no GPU: the product path has no CPU
fallback (a missing library or host tensors raise), and bench.py refuses a
GPU count other than one with a message, before touching a device."""
import os
import subprocess
import sys

import pytest
import torch

import sparse_long_context_piattn_amd as pa
from sparse_long_context_piattn_amd import binding

ROOT = os.path.join(os.path.dirname(__file__), "..")


def test_missing_library_raises(monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libpiattn.so"))
    with pytest.raises(RuntimeError, match="not built"):
        binding.lib()


def test_host_tensors_are_refused():
    q = torch.zeros((1, 1, 8, 32), dtype=torch.float32)
    g = torch.zeros((1, 1, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        pa.fwd(q, q, q, g, window_k=2, period_pi=4, num_skips=1)


@pytest.mark.parametrize("n", [2, 8])
def test_bench_refuses_more_than_one_gpu(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout.strip() == ""
