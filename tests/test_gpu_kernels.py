"""GPU parity of every prefill kernel, each forced through pa.forced_kernels.

The default dispatch runs one kernel per call shape; these tests pin each
kernel (split, residue-layout, gather) to the fp64 oracle on
the cases it accepts, so that a kernel the dispatch does not pick for the
headline shapes stays covered.  Tolerances as in test_gpu_parity.
"""
import zlib

import numpy as np
import pytest
import torch

import sparse_long_context_piattn_amd as pa
from sparse_long_context_piattn_amd import workloads as wl

from helpers import BF16_TOL, LSE_TOL_BF16, lse_tol_for, max_err, oracle_dense_fwd, \
    oracle_varlen_fwd, tol_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
KERNELS = ["split", "resid", "gather"]


def run_fwd(x, w, kernel, **kw):
    try:
        with pa.forced_kernels(fwd=kernel):
            return pa.fwd(x["q"], x["k"], x["v"], x["g"], window_k=w.k, period_pi=w.pi,
                          num_skips=w.M, bidirectional=w.bidir, cu_seqlens=x.get("cu_seqlens"), **kw)
    except pa.PiattnError as e:
        if "cannot take this call" in str(e):
            pytest.skip("%s does not take this shape" % kernel)
        raise


CASES = [
    # name, B, H, n, d, k, pi, M, bidir
    ("d64_pi64", 2, 3, 3000, 64, 20, 64, 10, False),
    ("d64_pi128_k64", 2, 2, 4096 + 77, 64, 64, 128, 16, False),
    ("d64_pi_le_k", 1, 2, 2000, 64, 70, 64, 5, False),
    ("d64_no_skips", 1, 2, 1500, 64, 64, 128, 0, False),
    ("d64_k0", 1, 2, 1500, 64, 0, 64, 7, False),
    ("d64_short_n", 2, 2, 37, 64, 8, 64, 3, False),
    ("d64_n1", 1, 2, 1, 64, 8, 64, 3, False),
    ("d64_odd_pi", 1, 2, 2500, 64, 24, 40, 9, False),
    ("d64_big_M", 1, 1, 4000, 64, 16, 64, 100, False),
    ("d64_bidir", 1, 3, 2900, 64, 32, 64, 6, True),
    ("d64_bidir_pi_le_k", 1, 2, 2500, 64, 80, 64, 6, True),
    ("d64_bidir_wide", 1, 1, 3333, 64, 100, 192, 8, True),
    ("d64_bidir_M32", 1, 2, 5000, 64, 32, 64, 32, True),
    ("d128_k128_pi256", 1, 2, 9000, 128, 128, 256, 20, False),
    ("d128_pi128", 2, 2, 3000, 128, 40, 128, 9, False),
    ("d128_odd_pi", 1, 2, 2222, 128, 30, 100, 13, False),
    ("d128_bidir", 1, 2, 3000, 128, 24, 128, 9, True),
    ("d128_no_skips", 1, 2, 1000, 128, 50, 128, 0, False),
    ("d128_short_n", 1, 2, 50, 128, 10, 16, 4, False),
    ("d128_M40", 1, 2, 6000, 128, 64, 64, 40, False),
    ("d128_M64_pi256", 1, 1, 20000, 128, 128, 256, 64, False),
    ("d128_bidir_M30", 1, 2, 4000, 128, 40, 64, 30, True),
    ("d128_bidir_M12", 1, 2, 3100, 128, 20, 96, 12, True),
    # bands of more than five key blocks: the skip pass without the register ring
    ("d128_big_M", 1, 1, 6000, 128, 16, 32, 90, False),
    ("d128_bidir_M40", 1, 1, 5000, 128, 24, 64, 40, True),
    ("d64_bidir_M50", 1, 2, 4000, 64, 16, 48, 50, True),
]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forced_kernel_matches_oracle(case, kernel):
    name, B, H, n, d, k, pi, M, bidir = case
    w = wl.Workload(name, "fwd", "bf16", B=B, H=H, n=n, d=d, k=k, pi=pi, M=M, bidir=bidir,
                    seed=zlib.crc32(name.encode()) % 1000)
    x = wl.make_fwd_inputs(w, device=DEV)
    lse = torch.empty_like(x["g"])
    out = run_fwd(x, w, kernel, lse=lse)
    torch.cuda.synchronize()
    ref, rlse = oracle_dense_fwd(x, w, want_lse=True)
    tag = "%s %s" % (kernel, name)
    assert max_err(out, ref, "fwd " + tag) <= tol_for(w)
    assert max_err(lse, rlse, "lse " + tag) <= lse_tol_for(w)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_f32mfma_matches_oracle(case):
    """The fp32 MFMA kernel on the same shapes in fp32 (its own dtype)."""
    name, B, H, n, d, k, pi, M, bidir = case
    w = wl.Workload(name + "_f32", "fwd", "f32", B=B, H=H, n=n, d=d, k=k, pi=pi, M=M, bidir=bidir,
                    seed=zlib.crc32(name.encode()) % 1000)
    x = wl.make_fwd_inputs(w, device=DEV)
    lse = torch.empty_like(x["g"])
    out = run_fwd(x, w, "f32mfma", lse=lse)
    torch.cuda.synchronize()
    ref, rlse = oracle_dense_fwd(x, w, want_lse=True)
    tag = "f32mfma %s" % name
    assert max_err(out, ref, "fwd " + tag) <= tol_for(w)
    assert max_err(lse, rlse, "lse " + tag) <= lse_tol_for(w)


def test_f32mfma_tiny_fp32_every_row():
    """The fp32 workload (B1 H2 n256 d32, k8 pi16 M4) on the fp32 MFMA kernel, every row."""
    w = wl.WORKLOADS["tiny_fp32"]
    x = wl.make_fwd_inputs(w, device=DEV)
    lse = torch.empty_like(x["g"])
    out = run_fwd(x, w, "f32mfma", lse=lse)
    torch.cuda.synchronize()
    ref, rlse = oracle_dense_fwd(x, w, want_lse=True)
    assert max_err(out, ref, "fwd f32mfma tiny_fp32") <= tol_for(w)
    assert max_err(lse, rlse, "lse f32mfma tiny_fp32") <= lse_tol_for(w)


def test_f32mfma_varlen_every_row():
    for bidir in (True, False):
        w = wl.Workload("vl32", "fwd", "f32", H=3, d=32, k=12, pi=20, M=5, bidir=bidir, nseq=6,
                        len_lo=1, len_hi=900, seed=29)
        x = wl.make_fwd_inputs(w, device=DEV, lengths=[0, 1, 700, 33, 899, 64])
        lse = torch.empty_like(x["g"])
        out = run_fwd(x, w, "f32mfma", lse=lse)
        torch.cuda.synchronize()
        ref, rlse = oracle_varlen_fwd(x, w, want_lse=True)
        T = x["q"].shape[0]
        tag = "f32mfma varlen bidir=%d" % bidir
        assert max_err(out.reshape(T * w.H, w.d), ref, "fwd " + tag) <= tol_for(w)
        assert max_err(lse.reshape(-1), rlse, "lse " + tag) <= lse_tol_for(w)


@pytest.mark.parametrize("kernel", ["resid", "split"])
def test_forced_kernel_varlen_every_row(kernel):
    for bidir in (True, False):
        w = wl.Workload("vl", "fwd", "bf16", H=3, d=64, k=12, pi=64, M=5, bidir=bidir, nseq=6,
                        len_lo=1, len_hi=900, seed=23)
        x = wl.make_fwd_inputs(w, device=DEV, lengths=[0, 1, 700, 33, 899, 64])
        lse = torch.empty_like(x["g"])
        out = run_fwd(x, w, kernel, lse=lse)
        torch.cuda.synchronize()
        ref, rlse = oracle_varlen_fwd(x, w, want_lse=True)
        T = x["q"].shape[0]
        tag = "%s varlen bidir=%d" % (kernel, bidir)
        assert max_err(out.reshape(T * w.H, w.d), ref, "fwd " + tag) <= BF16_TOL
        assert max_err(lse.reshape(-1), rlse, "lse " + tag) <= LSE_TOL_BF16


def test_split_prefill_8k_every_row():
    w = wl.WORKLOADS["prefill_8k"]
    x = wl.make_fwd_inputs(w, device=DEV)
    out = run_fwd(x, w, "split")
    torch.cuda.synchronize()
    ref = oracle_dense_fwd(x, w)
    assert max_err(out, ref, "fwd split prefill_8k all rows") <= BF16_TOL


def test_split_bidir_varlen_sampled_rows():
    w = wl.WORKLOADS["bidir_varlen"]
    x = wl.make_fwd_inputs(w, device=DEV)
    out = run_fwd(x, w, "split")
    torch.cuda.synchronize()
    cu = x["cu_seqlens"].cpu().numpy()
    T = int(cu[-1])
    rng = np.random.default_rng(5)
    toks = [np.arange(cu[s], min(cu[s] + 150, cu[s + 1])) for s in range(len(cu) - 1)]
    toks += [np.arange(max(cu[s], cu[s + 1] - 150), cu[s + 1]) for s in range(len(cu) - 1)]
    toks.append(rng.integers(0, T, 3000))
    toks = np.unique(np.concatenate(toks))
    heads = rng.integers(0, w.H, toks.size)
    rows = toks * w.H + heads
    ref = oracle_varlen_fwd(x, w, rows=rows)
    got = out.reshape(T * w.H, w.d).index_select(0, torch.from_numpy(rows).to(DEV))
    assert max_err(got, ref, "fwd split bidir_varlen sampled") <= BF16_TOL


def test_split_and_resid_agree_on_prefill_8k():
    w = wl.WORKLOADS["prefill_8k"]
    x = wl.make_fwd_inputs(w, device=DEV)
    a = run_fwd(x, w, "resid")
    b = run_fwd(x, w, "split")
    torch.cuda.synchronize()
    assert (a.float() - b.float()).abs().max().item() <= 2 * BF16_TOL


def test_split_workspace_reused_and_checked():
    """One caller workspace serves consecutive calls on a stream; a short one is refused."""
    w = wl.Workload("ws", "fwd", "bf16", B=2, H=3, n=1500, d=64, k=20, pi=64, M=10, bidir=False, seed=7)
    x1 = wl.make_fwd_inputs(w, device=DEV)
    x2 = wl.make_fwd_inputs(w, device=DEV, seed=8)
    kw = dict(window_k=w.k, period_pi=w.pi, num_skips=w.M, bidirectional=w.bidir)
    need = pa.fwd_workspace_bytes(1, w.B, w.H, w.n, w.d, pa.make_pattern(w.k, w.pi, w.M))
    assert need == 8 * w.B * w.H * w.n
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    a1 = pa.fwd(x1["q"], x1["k"], x1["v"], x1["g"], workspace=ws, **kw)
    a2 = pa.fwd(x2["q"], x2["k"], x2["v"], x2["g"], workspace=ws, **kw)
    b1 = pa.fwd(x1["q"], x1["k"], x1["v"], x1["g"], **kw)
    b2 = pa.fwd(x2["q"], x2["k"], x2["v"], x2["g"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(a1, b1) and torch.equal(a2, b2)
    assert max_err(a2, oracle_dense_fwd(x2, w), "fwd workspace reuse") <= BF16_TOL
    with pytest.raises(pa.PiattnError) as e:
        pa.fwd(x1["q"], x1["k"], x1["v"], x1["g"], workspace=ws[: need - 8], **kw)
    assert e.value.code == 3
