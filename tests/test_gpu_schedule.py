"""GPU parity for skip schedules (the union of several levels' skip sets).

The library reduces a schedule to its base period g (gcd of the periods) and
the set of skip multiples of g, held as a mask; these tests check every GPU
path that takes a pattern against the oracle's schedule functions
(oracle/piattn_oracle.c, the *_levels entry points, pinned in
test_oracle_pins.py): the neighbour dump bit for bit, the prefill kernels
(split on MFMA, gather), decode (linear and rolling caches) and both
backward paths, to the tolerances of the single-period tests.
"""
import zlib

import numpy as np
import pytest
import torch

import sparse_long_context_piattn_amd as pa
from sparse_long_context_piattn_amd import workloads as wl

import oracle
from helpers import LSE_TOL_BF16, LSE_TOL_F32, host_array, lse_tol_for, max_err, oracle_dense_fwd, packed, tol_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"

# name, k, pi, M, levels, bidir
SCHEDS = [
    # distances {4, 8, 12, 16, 32}: multiples {1, 2, 3, 4, 8} of 4 (a mask)
    ("g4_mask", 3, 8, 2, ((4, 3), (16, 2)), False),
    ("g4_mask_bidir", 3, 8, 2, ((4, 3), (16, 2)), True),
    # the hierarchical workload's pattern: multiples 1..16, 18..32/2, 36..64/4 of 128
    ("doubling", 64, 128, 16, ((256, 16), (512, 16)), False),
    ("doubling_bidir", 20, 32, 8, ((64, 8), (128, 8)), True),
    # distances {12, 24, 36} u {8, 16, 24, 32}: multiples {2, 3, 4, 6, 8, 9} of 4
    ("mixed_bidir", 5, 12, 3, ((8, 4),), True),
    # distances {6, 12} u {9}: multiples {2, 3, 4} of 3, contiguous but not from 1
    ("contig_from_2", 2, 6, 2, ((9, 1),), False),
    # gcd 1: distances 12 and 15 beyond the window
    ("gcd1", 10, 3, 5, ((5, 3),), False),
]


def _w(name, dt, B, H, n, d, k, pi, M, levels, bidir):
    seed = zlib.crc32(name.encode()) % 1000
    return wl.Workload(name, "fwd", dt, B=B, H=H, n=n, d=d, k=k, pi=pi, M=M, bidir=bidir,
                       levels=tuple(levels), seed=seed)


def _forced(which, kernel, fn):
    with pa.forced_kernels(**{which: kernel}):
        return fn()


@pytest.mark.parametrize("case", SCHEDS, ids=[c[0] for c in SCHEDS])
def test_schedule_neighbors_bit_exact(case):
    name, k, pi, M, levels, bidir = case
    n = 700
    idx, kind, cnt = pa.neighbors(n, window_k=k, period_pi=pi, num_skips=M, bidirectional=bidir,
                                  levels=levels)
    torch.cuda.synchronize()
    cap = idx.shape[1]
    ridx, rkind, rcnt = oracle.neighbor_table(n, k, pi, M, bidir, cap=cap, levels=levels)
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(kind.cpu().numpy(), rkind)


FWD = [(c, dt, d, kern) for c in SCHEDS for dt, d, kern in
       (("bf16", 64, "split"), ("bf16", 128, "split"), ("f32", 32, "gather"), ("bf16", 64, "gather"),
        ("f32", 32, "f32mfma"), ("f32", 64, "f32mfma"))]


@pytest.mark.parametrize("case,dt,d,kernel", FWD,
                         ids=["%s-%s%d-%s" % (c[0], dt, d, kern) for c, dt, d, kern in FWD])
def test_schedule_fwd_matches_oracle(case, dt, d, kernel):
    name, k, pi, M, levels, bidir = case
    n = 1500 if name.startswith("doubling") else 900
    w = _w(name, dt, 2, 2, n, d, k, pi, M, levels, bidir)
    x = wl.make_fwd_inputs(w, device=DEV)
    lse = torch.empty_like(x["g"])
    print("schedule fwd %s %s d%d %s" % (name, dt, d, kernel), flush=True)
    out = _forced("fwd", kernel, lambda: pa.fwd(
        x["q"], x["k"], x["v"], x["g"], window_k=k, period_pi=pi, num_skips=M, bidirectional=bidir,
        levels=levels, lse=lse))
    torch.cuda.synchronize()
    ref, rlse = oracle_dense_fwd(x, w, want_lse=True)
    assert max_err(out, ref, "sched fwd %s %s%d %s" % (name, dt, d, kernel)) <= tol_for(w)
    assert max_err(lse, rlse) <= (LSE_TOL_F32 if dt == "f32" else LSE_TOL_BF16)


def test_schedule_workload_every_row():
    """prefill_8k_sched (B4 H16 n8192 d64, k64, levels (128,16) (256,16)
    (512,16)): every row of the full-size call, with its lse, and every
    gradient row of its backward on the band kernels."""
    w = wl.WORKLOADS["prefill_8k_sched"]
    x = wl.make_fwd_inputs(w, device=DEV)
    print("schedule workload prefill_8k_sched", flush=True)
    kw = dict(window_k=w.k, period_pi=w.pi, num_skips=w.M, levels=w.levels)
    lse = torch.empty_like(x["g"])
    out = pa.fwd(x["q"], x["k"], x["v"], x["g"], lse=lse, **kw)
    torch.cuda.synchronize()
    ref, rlse = oracle_dense_fwd(x, w, want_lse=True)
    assert max_err(out, ref, "sched prefill_8k_sched all rows") <= tol_for(w)
    assert max_err(lse, rlse, "sched lse prefill_8k_sched all rows") <= lse_tol_for(w)
    gen = torch.Generator(device=DEV).manual_seed(w.seed + 3)
    dout = torch.randn(x["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    grads = _forced("bwd", "band", lambda: pa.bwd(x["q"], x["k"], x["v"], x["g"], out, dout, lse=lse, **kw))
    torch.cuda.synchronize()
    B, H, n, d = x["q"].shape
    gg = x["g"].detach().cpu().permute(0, 2, 1).reshape(B * n, H).double().numpy()
    rg = oracle.bwd(packed(x["q"]), packed(x["k"]), packed(x["v"]), gg, packed(dout), np.arange(B + 1) * n,
                    w.k, w.pi, w.M, w.bidir, w.scale, levels=w.levels)
    back = lambda t: t.reshape(B, n, H, d).transpose(0, 2, 1, 3)
    refs = (back(rg[0]), back(rg[1]), back(rg[2]), rg[3].reshape(B, n, H).transpose(0, 2, 1))
    for got, r, nm in zip(grads, refs, ("dq", "dk", "dv", "dg")):
        scale = max(1.0, float(np.abs(r).max()))
        assert max_err(got, r, "sched bwd prefill_8k_sched %s" % nm) / scale <= 3e-2, nm


@pytest.mark.parametrize("rolling", [False, True])
def test_schedule_decode_matches_oracle(rolling):
    k, pi, M, levels = 20, 32, 8, ((64, 8), (128, 8))
    S, H, d = 3, 2, 128
    slots = pa.rolling_slots(k, pi, M, levels=levels)
    assert slots == 128 * 8 + 1
    L = slots if rolling else 1400
    lens_lin = [1400, 700, 1]
    w = wl.Workload("sched_dec", "decode", "bf16", B=S, H=H, n=1400, d=d, k=k, pi=pi, M=M,
                    levels=levels, seed=81)
    x = wl.make_decode_inputs(w, device=DEV, lens=lens_lin)
    ref = oracle.decode(host_array(x["q"]), host_array(x["k_cache"]), host_array(x["v_cache"]),
                        lens_lin, x["g"].cpu().double().numpy(), k, pi, M, w.scale, levels=levels)
    kc, vc = x["k_cache"], x["v_cache"]
    if rolling:                                  # position j in row j mod slots
        kr = torch.empty((S, H, L, d), dtype=kc.dtype, device=DEV)
        vr = torch.empty_like(kr)
        for s, n in enumerate(lens_lin):
            for j in range(max(0, n - L), n):
                kr[s, :, j % L] = kc[s, :, j]
                vr[s, :, j % L] = vc[s, :, j]
        kc, vc = kr, vr
    print("schedule decode rolling=%d" % rolling, flush=True)
    out = pa.decode(x["q"], kc, vc, x["lens"], x["g"], window_k=k, period_pi=pi, num_skips=M,
                    levels=levels, rolling=rolling)
    torch.cuda.synchronize()
    assert max_err(out, ref, "sched decode rolling=%d" % rolling) <= 2e-2


BWD = [(c, path) for c in SCHEDS for path in ("band", "gather")]


@pytest.mark.parametrize("case,path", BWD, ids=["%s-%s" % (c[0], p) for c, p in BWD])
def test_schedule_bwd_matches_oracle(case, path):
    name, k, pi, M, levels, bidir = case
    n = 1100 if name.startswith("doubling") else 600
    w = _w(name, "bf16", 1, 2, n, 64, k, pi, M, levels, bidir)
    x = wl.make_fwd_inputs(w, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(w.seed + 1)
    dout = torch.randn(x["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    kw = dict(window_k=k, period_pi=pi, num_skips=M, bidirectional=bidir, levels=levels)
    lse = torch.empty_like(x["g"]) if path == "band" else None
    out = pa.fwd(x["q"], x["k"], x["v"], x["g"], lse=lse, **kw)
    print("schedule bwd %s %s" % (name, path), flush=True)
    grads = _forced("bwd", path,
                    lambda: pa.bwd(x["q"], x["k"], x["v"], x["g"], out, dout, lse=lse, **kw))
    torch.cuda.synchronize()
    B, H, n_, d = x["q"].shape
    gg = x["g"].detach().cpu().permute(0, 2, 1).reshape(B * n_, H).double().numpy()
    ref = oracle.bwd(packed(x["q"]), packed(x["k"]), packed(x["v"]), gg, packed(dout), [0, n_], k, pi,
                     M, bidir, w.scale, levels=levels)
    back = lambda t: t.reshape(B, n_, H, d).transpose(0, 2, 1, 3)
    refs = (back(ref[0]), back(ref[1]), back(ref[2]), ref[3].reshape(B, n_, H).transpose(0, 2, 1))
    for got, r, nm in zip(grads, refs, ("dq", "dk", "dv", "dg")):
        scale = max(1.0, float(np.abs(r).max()))
        assert max_err(got, r, "sched bwd %s %s %s" % (path, nm, name)) / scale <= 3e-2, nm
