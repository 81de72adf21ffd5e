"""GPU parity of the backward (piattn_bwd) against the fp64 oracle's
gradients (oracle.bwd, pinned to finite differences of the forward).

The GPU recomputes each row's softmax in fp32 and takes D_i = <dout_i,
out_i> from the forward output it is given; the oracle recomputes
everything in fp64 from the same inputs.  Errors are judged relative to the
gradient's scale: max|got - ref| <= tol * max(1, max|ref|), tol 1e-5 for
fp32 and 3e-2 for bf16 (bf16 outputs, the bf16 forward output in D, fp32
sums over up to ~150 keys).
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


def run(x, w, dout):
    kw = dict(window_k=w.k, period_pi=w.pi, num_skips=w.M, bidirectional=w.bidir,
              cu_seqlens=x.get("cu_seqlens"))
    out = pa.fwd(x["q"], x["k"], x["v"], x["g"], **kw)
    return out, pa.bwd(x["q"], x["k"], x["v"], x["g"], out, dout, **kw)


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
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_matches_oracle(case):
    name, dt, B, H, n, d, k, pi, M, bidir = case
    seed = zlib.crc32(name.encode()) % 1000
    w = wl.Workload(name, "fwd", dt, B=B, H=H, n=n, d=d, k=k, pi=pi, M=M, bidir=bidir, seed=seed)
    x = wl.make_fwd_inputs(w, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(seed + 1)
    dout = torch.randn(x["q"].shape, generator=gen, device=DEV).to(x["q"].dtype)
    out, (dq, dk, dv, dg) = run(x, w, dout)
    torch.cuda.synchronize()
    ref = oracle_grads_dense(x, w, dout)
    for got, r, nm in zip((dq, dk, dv, dg), ref, ("dq", "dk", "dv", "dg")):
        assert _rel(got, r, "bwd %s %s" % (nm, name)) <= TOL[dt], nm


def test_bwd_varlen_matches_oracle_and_dense():
    for bidir in (False, True):
        w = wl.Workload("vlb", "fwd", "bf16", H=3, d=64, k=12, pi=32, M=5, bidir=bidir, nseq=5,
                        len_lo=1, len_hi=600, seed=51)
        x = wl.make_fwd_inputs(w, device=DEV, lengths=[1, 600, 37, 0, 255])
        gen = torch.Generator(device=DEV).manual_seed(52)
        dout = torch.randn(x["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
        out, grads = run(x, w, dout)
        torch.cuda.synchronize()
        cu = x["cu_seqlens"].cpu().numpy().astype(np.int64)
        ref = oracle.bwd(host_array(x["q"]), host_array(x["k"]), host_array(x["v"]),
                         x["g"].detach().cpu().double().numpy(), host_array(dout), cu, w.k, w.pi, w.M,
                         w.bidir, w.scale)
        for got, r, nm in zip(grads, ref, ("dq", "dk", "dv", "dg")):
            assert _rel(got, r, "bwd varlen %s bidir=%d" % (nm, bidir)) <= TOL["bf16"], (nm, bidir)


def test_bwd_prefill_8k_one_head_every_row():
    """The prefill_8k shape (B4 H16 n8192 d64, k64 pi128 M16): the gradients of
    sequence 1, head 5 (every row; the oracle on that slice alone, since the
    heads are independent) against the full-size GPU run."""
    w = wl.WORKLOADS["prefill_8k"]
    x = wl.make_fwd_inputs(w, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(53)
    dout = torch.randn(x["q"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    out, grads = run(x, w, dout)
    torch.cuda.synchronize()
    b, h = 1, 5
    xs = {k_: v_[b:b + 1, h:h + 1] for k_, v_ in x.items()}
    ref = oracle_grads_dense(xs, w, dout[b:b + 1, h:h + 1])
    for got, r, nm in zip(grads, ref, ("dq", "dk", "dv", "dg")):
        g1 = got[b:b + 1, h:h + 1]
        assert _rel(g1, r, "bwd prefill_8k %s" % nm) <= TOL["bf16"], nm


def test_bwd_deterministic_and_workspace_checked():
    w = wl.Workload("det", "fwd", "bf16", B=1, H=2, n=500, d=64, k=16, pi=32, M=4, seed=54)
    x = wl.make_fwd_inputs(w, device=DEV)
    dout = torch.ones_like(x["q"])
    kw = dict(window_k=w.k, period_pi=w.pi, num_skips=w.M)
    out = pa.fwd(x["q"], x["k"], x["v"], x["g"], **kw)
    a = pa.bwd(x["q"], x["k"], x["v"], x["g"], out, dout, **kw)
    b = pa.bwd(x["q"], x["k"], x["v"], x["g"], out, dout, **kw)
    torch.cuda.synchronize()
    assert all(torch.equal(u, v) for u, v in zip(a, b))
    short = torch.empty(8 * 500 * 2 - 8, dtype=torch.uint8, device=DEV)
    with pytest.raises(pa.PiattnError) as e:
        pa.bwd(x["q"], x["k"], x["v"], x["g"], out, dout, workspace=short, **kw)
    assert e.value.code == 3
