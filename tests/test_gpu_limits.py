"""Maximum sizes: the split prefill path addresses rows with 32-bit byte
offsets and accepts a call when (n + 16 pi + d) times the largest token
stride, in bytes, stays below 2^31.  With token-major [1, n, H, d] storage
(token stride H d = 1024 elements at H = 16, d = 64) that allows n up to
1,046,463 with pi = 128, 2.1 GB per tensor.  At that n the split path must
run and match the oracle on the rows with the largest offsets; one token
more, it must refuse and the default dispatch must take another kernel (the
residue-tiled one, whose own bound is n d H 2 bytes) that still matches.
Rows checked: the first and last 300 and 2000 seeded ones of one head,
against the oracle on that head's slice.
"""
import os

import numpy as np
import pytest
import torch

import sparse_long_context_piattn_amd as pa
from sparse_long_context_piattn_amd import workloads as wl

from helpers import max_err, oracle_dense_fwd

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
H, D, K, PI, M = 16, 64, 64, 128, 16
N_MAX = (1 << 31) // (2 * H * D) - 16 * PI - D - 1      # 1,046,463
BF16_TOL = 2e-2


def _inputs(n, seed):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    t = [torch.randn((1, n, H, D), generator=gen, device=DEV, dtype=torch.bfloat16) for _ in range(3)]
    g = torch.randn((1, n, H), generator=gen, device=DEV, dtype=torch.float32)
    return {"q": t[0].permute(0, 2, 1, 3), "k": t[1].permute(0, 2, 1, 3), "v": t[2].permute(0, 2, 1, 3),
            "g": g.permute(0, 2, 1)}


def _fwd(x, kernel=None):
    old = os.environ.get("PIATTN_FWD_KERNEL")
    if kernel:
        os.environ["PIATTN_FWD_KERNEL"] = kernel
    try:
        return pa.fwd(x["q"], x["k"], x["v"], x["g"], window_k=K, period_pi=PI, num_skips=M)
    finally:
        if old is None:
            os.environ.pop("PIATTN_FWD_KERNEL", None)
        else:
            os.environ["PIATTN_FWD_KERNEL"] = old


def _check(x, out, n, tag):
    w = wl.Workload("limit", "fwd", "bf16", B=1, H=1, n=n, d=D, k=K, pi=PI, M=M, seed=0)
    h = 7
    rng = np.random.default_rng(61)
    rows = np.unique(np.concatenate([np.arange(300), rng.integers(0, n, 2000), np.arange(n - 300, n)]))
    sl = {k_: x[k_][:, h:h + 1] for k_ in ("q", "k", "v", "g")}
    ref = oracle_dense_fwd(sl, w, rows=rows)
    got = out[0, h].index_select(0, torch.from_numpy(rows).to(DEV))
    assert max_err(got, ref, tag) <= BF16_TOL


def test_split_path_at_its_largest_n():
    x = _inputs(N_MAX, 60)
    print("limit: split at n=%d" % N_MAX, flush=True)
    out = _fwd(x, "split")
    torch.cuda.synchronize()
    _check(x, out, N_MAX, "split n=%d" % N_MAX)


def test_one_token_more_leaves_the_split_path():
    n = N_MAX + 1
    x = _inputs(n, 62)
    print("limit: n=%d" % n, flush=True)
    with pytest.raises(pa.PiattnError) as e:
        _fwd(x, "split")
    assert e.value.code == 2
    out = _fwd(x)
    torch.cuda.synchronize()
    _check(x, out, n, "default dispatch n=%d" % n)
