"""GPU parity of the backward (piattn_bwd) against the fp64 oracle's
gradients (oracle.bwd, pinned to finite differences of the forward).

Two GPU paths: "gather" (no lse given: each row's softmax recomputed in
fp32) and "band" (bf16, d 64 / 128, the forward's lse given: MFMA kernels,
P and dS rounded to bf16 as MFMA operands, the skip part of dq, dk, dv held
as bf16 between its two passes).  Both take D_i = <dout_i, out_i> from the
forward output they are given; the oracle recomputes everything in fp64
from the same inputs.  Errors are judged relative to the gradient's scale:
max|got - ref| <= tol * max(1, max|ref|), tol 1e-5 for fp32 and 3e-2 for
bf16 (bf16 outputs, the bf16 forward output in D, fp32 sums over up to a
few hundred keys).
"""
import zlib

import numpy as np
import pytest
import torch

import sparse_long_context_piattn_amd as pa
from sparse_long_context_piattn_amd import workloads as wl

import oracle
from helpers import host_array, max_err, packed

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
TOL = {"f32": 1e-5, "bf16": 3e-2}


def _rel(got, ref, tag):
    ref = np.asarray(ref)
    scale = max(1.0, float(np.abs(ref).max()))
    err = max_err(got, ref, tag)
    return err / scale


def run(x, w, dout, path="gather"):
    """Forward, then the backward on `path`: gather (no lse) or band (the
    forward's lse, with the band kernels forced so that a call the MFMA
    kernels cannot take fails instead of falling back)."""
    kw = dict(window_k=w.k, period_pi=w.pi, num_skips=w.M, bidirectional=w.bidir,
              cu_seqlens=x.get("cu_seqlens"))
    lse = torch.empty_like(x["g"]) if path == "band" else None
    out = pa.fwd(x["q"], x["k"], x["v"], x["g"], lse=lse, **kw)
    with pa.forced_kernels(bwd=path):
        return out, pa.bwd(x["q"], x["k"], x["v"], x["g"], out, dout, lse=lse, **kw)


def oracle_grads_dense(x, w, dout):
    q, k, v, g = x["q"], x["k"], x["v"], x["g"]
    B, H, n, d = q.shape
    gg = g.detach().cpu().permute(0, 2, 1).reshape(B * n, H).double().numpy()
    res = oracle.bwd(packed(q), packed(k), packed(v), gg, packed(dout), np.arange(B + 1) * n,
                     w.k, w.pi, w.M, w.bidir, w.scale)
    dq, dk, dv, dg = res
    back = lambda t: t.reshape(B, n, H, d).transpose(0, 2, 1, 3)
    return back(dq), back(dk), back(dv), dg.reshape(B, n, H).transpose(0, 2, 1)


CASES = [
    # name, dtype, B, H, n, d, k, pi, M, bidir
    ("f32_d32", "f32", 2, 2, 300, 32, 8, 16, 4, False),
    ("f32_d64_bidir", "f32", 1, 2, 257, 64, 10, 24, 3, True),
    ("f32_d128", "f32", 1, 1, 200, 128, 16, 20, 5, False),
    ("bf16_d64", "bf16", 2, 2, 700, 64, 20, 64, 8, False),
    ("bf16_d128_bidir", "bf16", 1, 2, 600, 128, 30, 64, 6, True),
    ("bf16_d32", "bf16", 1, 3, 333, 32, 12, 16, 9, False),
    ("bf16_pi_le_k", "bf16", 1, 2, 400, 64, 40, 16, 5, False),
    ("bf16_no_skips", "bf16", 1, 2, 300, 64, 20, 64, 0, True),
    ("bf16_k0", "bf16", 1, 2, 300, 64, 0, 8, 6, False),
    ("bf16_n1", "bf16", 1, 2, 1, 64, 4, 8, 2, False),
    ("bf16_pi1", "bf16", 1, 1, 120, 64, 3, 1, 7, True),
    # shapes for the band kernels: several view tiles per residue (short pi),
    # skip bands longer than a tile (M > 64), windows wider than a tile,
    # residues shorter than a tile, and ragged tails everywhere
    ("bf16_d64_long_res", "bf16", 1, 2, 1500, 64, 5, 8, 70, False),
    ("bf16_d64_bidir_long_res", "bf16", 1, 1, 1300, 64, 6, 8, 70, True),
    ("bf16_d128_wide_win", "bf16", 1, 2, 777, 128, 150, 200, 3, False),
    ("bf16_d128_bidir_wide", "bf16", 1, 1, 650, 128, 100, 101, 5, True),
    ("bf16_d64_bidir_pi_le_k", "bf16", 1, 2, 500, 64, 20, 6, 12, True),
    ("bf16_d128_M1", "bf16", 2, 1, 300, 128, 10, 64, 1, False),
    ("bf16_d64_n63", "bf16", 1, 2, 63, 64, 7, 9, 6, True),
    ("bf16_d64_k200_pi3", "bf16", 1, 1, 400, 64, 200, 3, 100, False),
    # either side of the length at which the band skip pass forms the row
    # records itself (every residue view one 64-row tile: n <= 64 pi) instead
    # of reading them from the record kernel
    ("bf16_d64_views_one_tile", "bf16", 1, 2, 448, 64, 5, 7, 9, False),
    ("bf16_d64_views_one_row_more", "bf16", 1, 2, 449, 64, 5, 7, 9, False),
    ("bf16_d64_bidir_views_one_tile", "bf16", 1, 2, 448, 64, 5, 7, 9, True),
    ("bf16_d64_bidir_views_one_row_more", "bf16", 1, 2, 449, 64, 5, 7, 9, True),
    ("bf16_d128_views_one_tile", "bf16", 1, 2, 320, 128, 4, 5, 7, False),
    ("bf16_d128_views_one_row_more", "bf16", 1, 2, 321, 128, 4, 5, 7, False),
    ("bf16_d128_bidir_views_one_tile", "bf16", 1, 2, 320, 128, 4, 5, 7, True),
    ("bf16_d128_bidir_views_one_row_more", "bf16", 1, 2, 321, 128, 4, 5, 7, True),
]

# bf16_d64_k200_pi3 (causal, first skip multiple 67) gives the skip pass a
# first tile without keys, whose first stage is a query tile with its records.
BAND = [c for c in CASES if c[1] == "bf16" and c[5] in (64, 128)]
BAND_IDS = [c[0] for c in BAND]


def _check_case(case, path):
    name, dt, B, H, n, d, k, pi, M, bidir = case
    seed = zlib.crc32(name.encode()) % 1000
    w = wl.Workload(name, "fwd", dt, B=B, H=H, n=n, d=d, k=k, pi=pi, M=M, bidir=bidir, seed=seed)
    x = wl.make_fwd_inputs(w, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(seed + 1)
    dout = torch.randn(x["q"].shape, generator=gen, device=DEV).to(x["q"].dtype)
    print("bwd case %s path %s" % (name, path), flush=True)
    out, (dq, dk, dv, dg) = run(x, w, dout, path)
    torch.cuda.synchronize()
    ref = oracle_grads_dense(x, w, dout)
    for got, r, nm in zip((dq, dk, dv, dg), ref, ("dq", "dk", "dv", "dg")):
        assert _rel(got, r, "bwd %s %s %s" % (path, nm, name)) <= TOL[dt], nm


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_matches_oracle(case):
    _check_case(case, "gather")


@pytest.mark.parametrize("case", BAND, ids=BAND_IDS)
def test_bwd_band_matches_oracle(case):
    _check_case(case, "band")


@pytest.mark.parametrize("path", ["gather", "band"])
def test_bwd_varlen_matches_oracle(path):
    for bidir in (False, True):
        w = wl.Workload("vlb", "fwd", "bf16", H=3, d=64, k=12, pi=32, M=5, bidir=bidir, nseq=5,
                        len_lo=1, len_hi=600, seed=51)
        x = wl.make_fwd_inputs(w, device=DEV, lengths=[1, 600, 37, 0, 255])
        gen = torch.Generator(device=DEV).manual_seed(52)
        dout = torch.randn(x["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
        print("bwd varlen bidir=%d path %s" % (bidir, path), flush=True)
        out, grads = run(x, w, dout, path)
        torch.cuda.synchronize()
        cu = x["cu_seqlens"].cpu().numpy().astype(np.int64)
        ref = oracle.bwd(host_array(x["q"]), host_array(x["k"]), host_array(x["v"]),
                         x["g"].detach().cpu().double().numpy(), host_array(dout), cu, w.k, w.pi, w.M,
                         w.bidir, w.scale)
        for got, r, nm in zip(grads, ref, ("dq", "dk", "dv", "dg")):
            assert _rel(got, r, "bwd %s varlen %s bidir=%d" % (path, nm, bidir)) <= TOL["bf16"], (nm, bidir)


@pytest.mark.parametrize("path", ["gather", "band"])
def test_bwd_prefill_8k_every_row(path):
    """The full prefill_8k shape (B4 H16 n8192 d64, k64 pi128 M16): every
    gradient row of every (sequence, head), half a million rows, against the
    oracle on the same inputs."""
    w = wl.WORKLOADS["prefill_8k"]
    x = wl.make_fwd_inputs(w, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(53)
    dout = torch.randn(x["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    print("bwd prefill_8k path %s" % path, flush=True)
    out, grads = run(x, w, dout, path)
    torch.cuda.synchronize()
    ref = oracle_grads_dense(x, w, dout)
    for got, r, nm in zip(grads, ref, ("dq", "dk", "dv", "dg")):
        assert _rel(got, r, "bwd %s prefill_8k %s" % (path, nm)) <= TOL["bf16"], nm


def test_bwd_band_prefill_128k_every_row():
    """The full prefill_128k shape (B1 H32 n131072 d128, k128 pi256 M64) on
    the band kernels: every gradient row of every head (about 4.2 million
    rows) against the oracle, which runs its (sequence, head) pairs in
    parallel."""
    w = wl.WORKLOADS["prefill_128k"]
    x = wl.make_fwd_inputs(w, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(57)
    dout = torch.randn(x["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    print("bwd prefill_128k band", flush=True)
    out, grads = run(x, w, dout, "band")
    torch.cuda.synchronize()
    ref = oracle_grads_dense(x, w, dout)
    for got, r, nm in zip(grads, ref, ("dq", "dk", "dv", "dg")):
        assert _rel(got, r, "bwd band prefill_128k %s" % nm) <= TOL["bf16"], nm


def test_bwd_band_bidir_varlen_every_row():
    """The full bidir_varlen shape (8 packed sequences of 4096..32768 tokens,
    H16 d64, k32 pi64 M32 per direction) on the band kernels: every gradient
    row (about 3 million) against the oracle on the same packed batch."""
    w = wl.WORKLOADS["bidir_varlen"]
    lengths = wl.varlen_lengths(w)
    x = wl.make_fwd_inputs(w, device=DEV, lengths=lengths)
    gen = torch.Generator(device=DEV).manual_seed(55)
    dout = torch.randn(x["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    print("bwd bidir_varlen band", flush=True)
    out, grads = run(x, w, dout, "band")
    torch.cuda.synchronize()
    cu = x["cu_seqlens"].cpu().numpy().astype(np.int64)
    ref = oracle.bwd(host_array(x["q"]), host_array(x["k"]), host_array(x["v"]),
                     x["g"].detach().cpu().double().numpy(), host_array(dout), cu, w.k, w.pi, w.M,
                     w.bidir, w.scale)
    for got, r, nm in zip(grads, ref, ("dq", "dk", "dv", "dg")):
        assert _rel(got, r, "bwd band bidir_varlen %s" % nm) <= TOL["bf16"], nm


@pytest.mark.parametrize("with_lse", [False, True])
def test_bwd_deterministic_and_workspace_checked(with_lse):
    w = wl.Workload("det", "fwd", "bf16", B=1, H=2, n=500, d=64, k=16, pi=32, M=4, seed=54)
    x = wl.make_fwd_inputs(w, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(56)
    dout = torch.randn(x["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    kw = dict(window_k=w.k, period_pi=w.pi, num_skips=w.M)
    lse = torch.empty_like(x["g"]) if with_lse else None
    out = pa.fwd(x["q"], x["k"], x["v"], x["g"], lse=lse, **kw)
    a = pa.bwd(x["q"], x["k"], x["v"], x["g"], out, dout, lse=lse, **kw)
    b = pa.bwd(x["q"], x["k"], x["v"], x["g"], out, dout, lse=lse, **kw)
    torch.cuda.synchronize()
    assert all(torch.equal(u, v) for u, v in zip(a, b))
    short = torch.empty(16 * 500 * 2 - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(pa.PiattnError) as e:
        pa.bwd(x["q"], x["k"], x["v"], x["g"], out, dout, lse=lse, workspace=short, **kw)
    assert e.value.code == 3


def test_bwd_band_and_gather_agree():
    """The two GPU paths on one input: equal to within the bf16 rounding of
    their different summation orders and operand roundings."""
    w = wl.Workload("agree", "fwd", "bf16", B=2, H=2, n=900, d=128, k=40, pi=48, M=9, seed=57)
    x = wl.make_fwd_inputs(w, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(58)
    dout = torch.randn(x["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    _, ga = run(x, w, dout, "gather")
    _, gb = run(x, w, dout, "band")
    torch.cuda.synchronize()
    for u, v, nm in zip(ga, gb, ("dq", "dk", "dv", "dg")):
        scale = max(1.0, float(u.float().abs().max()))
        assert float((u.float() - v.float()).abs().max()) / scale <= TOL["bf16"], nm


def test_bwd_band_refuses_what_it_cannot_take():
    """The forced band backward without lse, or for fp32, is EUNSUPPORTED
    (refused on the host, before any launch)."""
    w = wl.Workload("ref", "fwd", "bf16", B=1, H=1, n=64, d=64, k=4, pi=8, M=2, seed=59)
    x = wl.make_fwd_inputs(w, device=DEV)
    lse = torch.empty_like(x["g"])
    kw = dict(window_k=4, period_pi=8, num_skips=2)
    out = pa.fwd(x["q"], x["k"], x["v"], x["g"], lse=lse, **kw)
    xf = {k_: v_.float() if v_.dtype == torch.bfloat16 else v_ for k_, v_ in x.items()}
    outf = out.float()
    with pa.forced_kernels(bwd="band"):
        for args, use_lse in (((x["q"], x["k"], x["v"], x["g"], out, torch.ones_like(out)), False),
                              ((xf["q"], xf["k"], xf["v"], xf["g"], outf, torch.ones_like(outf)), True)):
            with pytest.raises(pa.PiattnError) as e:
                pa.bwd(*args, lse=lse if use_lse else None, **kw)
            assert e.value.code == 2