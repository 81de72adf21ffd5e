"""Seeded random sweep of patterns through the GPU paths, against the oracle.

Each of 48 forward and 32 backward cases (PIATTN_SWEEP_FWD / PIATTN_SWEEP_BWD
widen the seed ranges) draws a window k, period pi, skip count M, direction, head dim,
ragged length and (sometimes) a skip schedule of up to three levels, within
the bounds the library accepts; the prefill runs on every kernel that takes
the pattern (split, resid, gather, f32mfma; pa.forced_kernels), and the backward on
both paths.  Tolerances as in the other parity tests: 1e-5 (fp32) / 2e-2
(bf16) for the forward, 1e-5 / 3e-2 relative to the gradient's scale for
the backward.
"""

import os

import numpy as np
import pytest
import torch

import sparse_long_context_piattn_amd as pa
from sparse_long_context_piattn_amd import workloads as wl

import oracle
from helpers import max_err, oracle_dense_fwd, packed, tol_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _case(seed):
    rng = np.random.default_rng(9000 + seed)
    d = int(rng.choice([32, 64, 64, 128]))
    dt = "f32" if d == 32 and rng.random() < 0.5 else "bf16"
    k = int(rng.integers(0, 90))
    pi = int(rng.integers(1, 200))
    M = int(rng.integers(0, 40))
    bidir = bool(rng.random() < 0.4)
    n = int(rng.integers(1, 1500))
    levels = ()
    if rng.random() < 0.35:
        base = int(rng.integers(1, 40))
        levels = tuple((base * int(rng.integers(1, 5)), int(rng.integers(0, 8))) for _ in range(rng.integers(1, 4)))
        pi = base * int(rng.integers(1, 4))
        M = int(rng.integers(0, 10))
    H = int(rng.integers(1, 4))
    return wl.Workload("sweep%d" % seed, "fwd", dt, B=1, H=H, n=n, d=d, k=k, pi=pi, M=M, bidir=bidir,
                       levels=levels, seed=seed)


def _forced(which, kernel, fn):
    with pa.forced_kernels(**{which: kernel}):
        return fn()


@pytest.mark.parametrize("seed", range(int(os.environ.get("PIATTN_SWEEP_FWD", "48"))))
def test_sweep_fwd_every_kernel(seed):
    w = _case(seed)
    x = wl.make_fwd_inputs(w, device=DEV)
    ref = oracle_dense_fwd(x, w)
    ran = 0
    for kern in ("split", "resid", "gather", "f32mfma"):
        print("sweep fwd seed %d %s: %s" % (seed, kern, w), flush=True)
        try:
            out = _forced("fwd", kern, lambda: pa.fwd(
                x["q"], x["k"], x["v"], x["g"], window_k=w.k, period_pi=w.pi, num_skips=w.M,
                bidirectional=w.bidir, levels=w.levels))
        except pa.PiattnError as e:
            if e.code == 2:                        # this kernel (or the schedule) is not supported
                continue
            raise
        torch.cuda.synchronize()
        assert max_err(out, ref, "sweep fwd %d %s" % (seed, kern)) <= tol_for(w), kern
        ran += 1
    assert ran >= 1 or w.levels


@pytest.mark.parametrize("seed", range(int(os.environ.get("PIATTN_SWEEP_BWD", "32"))))
def test_sweep_bwd_both_paths(seed):
    w = _case(100 + seed)
    if w.n > 900:
        w = wl.Workload(w.name, "fwd", w.dtype, B=1, H=w.H, n=900, d=w.d, k=w.k, pi=w.pi, M=w.M,
                        bidir=w.bidir, levels=w.levels, seed=w.seed)
    x = wl.make_fwd_inputs(w, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(w.seed + 7)
    dout = torch.randn(x["q"].shape, generator=gen, device=DEV).to(x["q"].dtype)
    kw = dict(window_k=w.k, period_pi=w.pi, num_skips=w.M, bidirectional=w.bidir, levels=w.levels)
    lse = torch.empty_like(x["g"])
    try:
        out = pa.fwd(x["q"], x["k"], x["v"], x["g"], lse=lse, **kw)
    except pa.PiattnError as e:
        assert e.code == 2 and w.levels
        pytest.skip("schedule beyond 127 multiples of its gcd")
    B, H, n, d = x["q"].shape
    gg = x["g"].detach().cpu().permute(0, 2, 1).reshape(B * n, H).double().numpy()
    ref = oracle.bwd(packed(x["q"]), packed(x["k"]), packed(x["v"]), gg, packed(dout), [0, n], w.k, w.pi,
                     w.M, w.bidir, w.scale, levels=w.levels)
    back = lambda t: t.reshape(B, n, H, d).transpose(0, 2, 1, 3)
    refs = (back(ref[0]), back(ref[1]), back(ref[2]), ref[3].reshape(B, n, H).transpose(0, 2, 1))
    tol = 1e-5 if w.dtype == "f32" else 3e-2
    for path in ("band", "gather"):
        print("sweep bwd seed %d %s: %s" % (seed, path, w), flush=True)
        try:
            grads = _forced("bwd", path, lambda: pa.bwd(
                x["q"], x["k"], x["v"], x["g"], out, dout, lse=lse if path == "band" else None, **kw))
        except pa.PiattnError as e:
            if e.code == 2 and path == "band":     # fp32 or d = 32
                continue
            raise
        torch.cuda.synchronize()
        for got, r, nm in zip(grads, refs, ("dq", "dk", "dv", "dg")):
            scale = max(1.0, float(np.abs(r).max()))
            assert max_err(got, r, "sweep bwd %d %s %s" % (seed, path, nm)) / scale <= tol, (path, nm)
