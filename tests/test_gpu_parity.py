"""GPU parity: libpiattn (through its C ABI) against the fp64 CPU oracle.

Index work is compared bit-exactly; floating point within max-abs 1e-5 (fp32)
and 2e-2 (bf16 inputs/outputs, fp32 accumulation).  Inputs come from the
seeded generators in sparse_long_context_piattn_amd.workloads.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import sparse_long_context_piattn_amd as pa
from sparse_long_context_piattn_amd import workloads as wl

from helpers import (BF16_TOL, F32_TOL, LSE_TOL_BF16, host_array, lse_tol_for, max_err,
                     oracle_dense_fwd, oracle_varlen_fwd, tol_for)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def run_fwd(x, w, **kw):
    return pa.fwd(x["q"], x["k"], x["v"], x["g"], window_k=w.k, period_pi=w.pi, num_skips=w.M,
                  bidirectional=w.bidir, cu_seqlens=x.get("cu_seqlens"), **kw)


# ------------------------------------------------------------------ neighbours

NEIGHBOR_CASES = [
    (16, 3, 1, 0, False), (16, 15, 1, 0, False), (1, 0, 1, 0, False), (1, 4, 3, 2, True),
    (50, 0, 1, 5, False), (50, 2, 7, 4, False), (50, 9, 3, 6, False), (50, 9, 3, 6, True),
    (97, 4, 16, 10, True), (300, 8, 16, 4, False), (64, 70, 5, 3, True), (33, 5, 5, 40, False),
]


@pytest.mark.parametrize("n,k,pi,M,bidir", NEIGHBOR_CASES)
def test_neighbors_small_bit_exact(n, k, pi, M, bidir):
    idx, kind, cnt = pa.neighbors(n, window_k=k, period_pi=pi, num_skips=M, bidirectional=bidir,
                                  device=DEV)
    cap = idx.shape[1]
    ri, rk, rc = oracle.neighbor_table(n, k, pi, M, bidir, cap=cap)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(kind.cpu().numpy(), rk)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)


def test_neighbors_partial_range_and_wide_cap():
    idx, kind, cnt = pa.neighbors(1000, window_k=5, period_pi=11, num_skips=9, q_begin=123,
                                  q_count=400, cap=40, device=DEV)
    ri, rk, rc = oracle.neighbor_table(1000, 5, 11, 9, False, q_begin=123, q_count=400, cap=40)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(kind.cpu().numpy(), rk)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)


@pytest.mark.parametrize("name", ["tiny_fp32", "prefill_8k", "prefill_128k", "decode_32k"])
def test_neighbors_every_row_of_workload(name):
    w = wl.WORKLOADS[name]
    idx, kind, cnt = pa.neighbors(w.n, window_k=w.k, period_pi=w.pi, num_skips=w.M,
                                  bidirectional=w.bidir, device=DEV)
    ri, rk, rc = oracle.neighbor_table(w.n, w.k, w.pi, w.M, w.bidir, cap=idx.shape[1])
    assert np.array_equal(cnt.cpu().numpy(), rc)
    assert np.array_equal(idx.cpu().numpy(), ri)
    assert np.array_equal(kind.cpu().numpy(), rk)


def test_neighbors_every_row_bidir_varlen_lengths():
    w = wl.WORKLOADS["bidir_varlen"]
    for n in sorted(set(wl.varlen_lengths(w))):
        idx, kind, cnt = pa.neighbors(n, window_k=w.k, period_pi=w.pi, num_skips=w.M,
                                      bidirectional=True, device=DEV)
        ri, rk, rc = oracle.neighbor_table(n, w.k, w.pi, w.M, True, cap=idx.shape[1])
        assert np.array_equal(idx.cpu().numpy(), ri), n
        assert np.array_equal(kind.cpu().numpy(), rk), n
        assert np.array_equal(cnt.cpu().numpy(), rc), n


# ------------------------------------------------------------------ prefill

def test_fwd_tiny_fp32_full_with_lse():
    w = wl.WORKLOADS["tiny_fp32"]
    x = wl.make_fwd_inputs(w, device=DEV)
    lse = torch.empty_like(x["g"])
    out = run_fwd(x, w, lse=lse)
    torch.cuda.synchronize()
    ref, rlse = oracle_dense_fwd(x, w, want_lse=True)
    assert max_err(out, ref, "fwd tiny_fp32 all rows") <= F32_TOL
    assert max_err(lse, rlse, "lse tiny_fp32 all rows") <= 1e-5


SMALL = [
    # name, dtype, B, H, n, d, k, pi, M, bidir
    ("ragged_d64", "bf16", 2, 3, 1000, 64, 20, 32, 6, False),
    ("ragged_d128", "bf16", 1, 2, 777, 128, 40, 64, 5, False),
    ("d32_bf16", "bf16", 1, 2, 300, 32, 8, 16, 4, False),
    ("pi_le_k", "bf16", 1, 2, 500, 64, 37, 16, 7, False),
    ("no_skips", "bf16", 1, 2, 400, 64, 30, 32, 0, False),
    ("k0", "bf16", 1, 2, 400, 64, 0, 16, 9, False),
    ("pi1", "bf16", 1, 1, 200, 64, 3, 1, 50, False),
    ("n1", "bf16", 3, 2, 1, 64, 5, 16, 3, False),
    ("k_ge_n", "bf16", 1, 2, 90, 64, 200, 16, 3, False),
    ("bidir_d64", "bf16", 1, 3, 900, 64, 32, 64, 6, True),
    ("bidir_pi_le_k", "bf16", 1, 2, 333, 64, 20, 8, 9, True),
    ("f32_d64", "f32", 1, 2, 600, 64, 16, 32, 8, False),
    ("f32_d128_bidir", "f32", 1, 2, 300, 128, 10, 16, 5, True),
    ("tiles_d64_pi128", "bf16", 2, 2, 4096 + 77, 64, 64, 128, 16, False),
    ("tiles_d128_pi256", "bf16", 1, 2, 9000, 128, 128, 256, 20, False),
    ("tiles_bidir_pi64", "bf16", 1, 2, 5000, 64, 32, 64, 32, True),
    # larger shapes: several MFMA tiles, chunks and ragged tails
    ("tiled_pi64_d64", "bf16", 2, 3, 3000, 64, 20, 64, 10, False),
    ("tiled_pi_le_k", "bf16", 1, 2, 2000, 64, 70, 64, 5, False),
    ("tiled_no_skips", "bf16", 1, 2, 1500, 64, 64, 128, 0, False),
    ("tiled_k0", "bf16", 1, 2, 1500, 64, 0, 64, 7, False),
    ("tiled_short_n", "bf16", 2, 2, 37, 64, 8, 64, 3, False),
    ("tiled_n1", "bf16", 1, 2, 1, 64, 8, 64, 3, False),
    ("tiled_bidir_d128", "bf16", 1, 2, 3000, 128, 24, 128, 9, True),
    ("tiled_bidir_pi_le_k", "bf16", 1, 2, 2500, 64, 80, 64, 6, True),
    ("tiled_big_M", "bf16", 1, 1, 4000, 64, 16, 64, 100, False),
    ("tiled_d128_k128", "bf16", 1, 1, 5000, 128, 128, 256, 30, False),
    ("tiled_bidir_d64_wide", "bf16", 1, 1, 3333, 64, 100, 192, 8, True),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_fwd_small_cases_full(case):
    name, dt, B, H, n, d, k, pi, M, bidir = case
    w = wl.Workload(name, "fwd", dt, B=B, H=H, n=n, d=d, k=k, pi=pi, M=M, bidir=bidir,
                    seed=zlib.crc32(name.encode()) % 1000)
    x = wl.make_fwd_inputs(w, device=DEV)
    lse = torch.empty_like(x["g"])
    out = run_fwd(x, w, lse=lse)
    torch.cuda.synchronize()
    ref, rlse = oracle_dense_fwd(x, w, want_lse=True)
    assert max_err(out, ref, "fwd " + name) <= tol_for(w)
    assert max_err(lse, rlse, "lse " + name) <= lse_tol_for(w)


@pytest.mark.parametrize("pi", [32, 64])
def test_fwd_bnhd_layout_matches_bhnd(pi):
    w = wl.Workload("layout", "fwd", "bf16", B=2, H=4, n=1640, d=64, k=16, pi=pi, M=6, seed=11)
    x = wl.make_fwd_inputs(w, device=DEV, layout="bnhd")        # [B, n, H, d] storage
    view = dict(q=x["q"].transpose(1, 2), k=x["k"].transpose(1, 2), v=x["v"].transpose(1, 2),
                g=x["g"])
    out = torch.empty_like(x["q"]).transpose(1, 2)
    run_fwd(view, w, out=out)
    dense = {k: v.contiguous() for k, v in view.items()}
    out2 = run_fwd(dense, w)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    ref = oracle_dense_fwd(dense, w)
    assert max_err(out2, ref) <= BF16_TOL


@pytest.mark.parametrize("pi", [32, 64])
@pytest.mark.parametrize("gval", [float("inf"), float("-inf"), 60.0, -60.0])
def test_fwd_gate_limits(gval, pi):
    w = wl.Workload("gate", "fwd", "bf16", B=1, H=2, n=1700, d=64, k=10, pi=pi, M=8, seed=5)
    x = wl.make_fwd_inputs(w, device=DEV)
    x["g"].fill_(gval)
    out = run_fwd(x, w)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    ref = oracle_dense_fwd(x, w)
    assert max_err(out, ref) <= BF16_TOL


def test_fwd_empty_input_is_a_no_op():
    q = torch.empty((0, 2, 16, 64), dtype=torch.bfloat16, device=DEV)
    g = torch.empty((0, 2, 16), dtype=torch.float32, device=DEV)
    out = pa.fwd(q, q, q, g, window_k=4, period_pi=8, num_skips=2)
    assert out.shape == q.shape


def test_fwd_deterministic():
    w = wl.WORKLOADS["prefill_8k"]
    x = wl.make_fwd_inputs(w, device=DEV)
    a = run_fwd(x, w)
    b = run_fwd(x, w)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_fwd_prefill_8k_every_row():
    w = wl.WORKLOADS["prefill_8k"]
    x = wl.make_fwd_inputs(w, device=DEV)
    lse = torch.empty_like(x["g"])
    out = run_fwd(x, w, lse=lse)
    torch.cuda.synchronize()
    ref, rlse = oracle_dense_fwd(x, w, want_lse=True)
    assert max_err(out, ref, "fwd prefill_8k all rows") <= BF16_TOL
    assert max_err(lse, rlse, "lse prefill_8k all rows") <= LSE_TOL_BF16


def _sampled_rows(n, count, seed, edge=300):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(min(edge, n)), rng.integers(0, n, count),
                           np.arange(max(0, n - edge), n)])
    return np.unique(rows)


def test_fwd_prefill_128k_every_row():
    """Every row of the full prefill_128k call (B1 H32 n131072 d128: about 4.2
    million rows), with its lse, against the oracle; eight heads at a time
    (the heads are independent), which bounds the host memory of the fp64
    reference to about 1 GB per group."""
    w = wl.WORKLOADS["prefill_128k"]
    x = wl.make_fwd_inputs(w, device=DEV)
    lse = torch.empty_like(x["g"])
    out = run_fwd(x, w, lse=lse)
    torch.cuda.synchronize()
    for h0 in range(0, w.H, 8):
        print("fwd prefill_128k heads %d..%d" % (h0, h0 + 7), flush=True)
        sl = {k: x[k][:, h0:h0 + 8] for k in ("q", "k", "v", "g")}
        ref, rlse = oracle_dense_fwd(sl, w, want_lse=True)
        assert max_err(out[:, h0:h0 + 8], ref, "fwd prefill_128k heads %d.. all rows" % h0) <= BF16_TOL, h0
        assert max_err(lse[:, h0:h0 + 8], rlse, "lse prefill_128k heads %d.. all rows" % h0) <= LSE_TOL_BF16, h0
        del ref, rlse


def test_fwd_bidir_varlen_every_row():
    """Every row (token, head) of the full bidir_varlen workload: 8 packed
    sequences, about 3 million rows, against the C oracle."""
    w = wl.WORKLOADS["bidir_varlen"]
    x = wl.make_fwd_inputs(w, device=DEV)
    lse = torch.empty_like(x["g"])
    out = run_fwd(x, w, lse=lse)
    torch.cuda.synchronize()
    T = x["q"].shape[0]
    ref, rlse = oracle_varlen_fwd(x, w, want_lse=True)
    assert max_err(out.reshape(T * w.H, w.d), ref, "fwd bidir_varlen all rows") <= BF16_TOL
    assert max_err(lse.reshape(-1), rlse, "lse bidir_varlen all rows") <= LSE_TOL_BF16


@pytest.mark.parametrize("pi", [32, 64])
def test_fwd_small_varlen_every_row(pi):
    w = wl.Workload("vl", "fwd", "bf16", H=3, d=64, k=12, pi=pi, M=5, bidir=True, nseq=5,
                    len_lo=1, len_hi=900, seed=21)
    for bidir in (True, False):
        w2 = wl.Workload("vl", "fwd", "bf16", H=3, d=64, k=12, pi=pi, M=5, bidir=bidir, nseq=5,
                         len_lo=1, len_hi=900, seed=21)
        x = wl.make_fwd_inputs(w2, device=DEV, lengths=[0, 1, 700, 33, 899])
        lse = torch.empty_like(x["g"])
        out = run_fwd(x, w2, lse=lse)
        torch.cuda.synchronize()
        ref, rlse = oracle_varlen_fwd(x, w2, want_lse=True)
        T = x["q"].shape[0]
        tag = "varlen pi=%d bidir=%d" % (pi, bidir)
        assert max_err(out.reshape(T * w.H, w.d), ref, "fwd " + tag) <= BF16_TOL
        assert max_err(lse.reshape(-1), rlse, "lse " + tag) <= LSE_TOL_BF16


# ------------------------------------------------------------------ decode

def run_decode(x, w, **kw):
    return pa.decode(x["q"], x["k_cache"], x["v_cache"], x["lens"], x["g"], window_k=w.k,
                     period_pi=w.pi, num_skips=w.M, **kw)


def oracle_decode(x, w):
    return oracle.decode(host_array(x["q"]), host_array(x["k_cache"]), host_array(x["v_cache"]),
                         x["lens"].cpu().numpy(), x["g"].cpu().double().numpy(), w.k, w.pi, w.M,
                         w.scale)


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("bf16", 32)])
def test_decode_small_ragged_lengths_all_split_counts(dt, d):
    w = wl.Workload("dec", "decode", dt, B=6, H=3, n=3000, d=d, k=100, pi=128, M=20, seed=31)
    lens = [3000, 1, 101, 129, 2500, 777]
    x = wl.make_decode_inputs(w, device=DEV, lens=lens)
    ref = oracle_decode(x, w)
    outs = []
    for splits in (1, 0, 2, 7, 64):
        o = run_decode(x, w, num_splits=splits)
        torch.cuda.synchronize()
        assert max_err(o, ref, "decode %s d=%d splits=%d" % (dt, d, splits)) <= tol_for(w), splits
        outs.append(o)
    assert torch.equal(outs[0], run_decode(x, w, num_splits=1))


def test_decode_bad_length_rows_are_nan():
    w = wl.Workload("dec", "decode", "bf16", B=3, H=2, n=500, d=64, k=10, pi=32, M=4, seed=32)
    x = wl.make_decode_inputs(w, device=DEV, lens=[500, 1, 1])
    x["lens"][1] = 0
    x["lens"][2] = 501
    for splits in (1, 3):
        o = run_decode(x, w, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.isnan(o[1].float()).all() and torch.isnan(o[2].float()).all()
        assert torch.isfinite(o[0].float()).all()


def test_decode_equals_prefill_last_row():
    w = wl.Workload("dec", "fwd", "bf16", B=2, H=4, n=2048, d=128, k=64, pi=128, M=15, seed=33)
    x = wl.make_fwd_inputs(w, device=DEV)
    out = run_fwd(x, w)
    d = dict(q=x["q"][:, :, -1].contiguous(), k_cache=x["k"], v_cache=x["v"],
             lens=torch.full((2,), 2048, dtype=torch.int32, device=DEV),
             g=x["g"][:, :, -1].contiguous())
    o = pa.decode(d["q"], d["k_cache"], d["v_cache"], d["lens"], d["g"], window_k=w.k,
                  period_pi=w.pi, num_skips=w.M)
    torch.cuda.synchronize()
    assert (o.float() - out[:, :, -1].float()).abs().max().item() <= BF16_TOL


def test_decode_32k_every_row():
    """Every (sequence, head) row of the full 128 x 32 decode call against the
    oracle.  The whole cache is 68.7 GB, so only the key and value rows the
    query reads -- the oracle's own neighbour list of position len-1 -- are
    gathered on the GPU and copied to the host (about 671 MB), then placed
    at their positions in a zeroed full-length host cache of one (sequence,
    head) for each oracle call.  Were that list wrong, the oracle would read
    zero rows and the comparison would fail."""
    w = wl.WORKLOADS["decode_32k"]
    x = wl.make_decode_inputs(w, device=DEV)
    out = run_decode(x, w)
    torch.cuda.synchronize()
    lens = x["lens"].cpu().numpy()
    S, H, L, d = x["k_cache"].shape
    got = out.float().cpu().numpy()
    qh = host_array(x["q"])
    gh = x["g"].cpu().double().numpy()
    kbuf = np.zeros((1, 1, L, d), np.uint16)
    vbuf = np.zeros((1, 1, L, d), np.uint16)
    worst = 0.0
    for ln in sorted(set(int(v) for v in lens)):
        seqs = np.nonzero(lens == ln)[0]
        pos, _ = oracle.neighbors(ln, w.k, w.pi, w.M, False, ln - 1)
        assert pos.size == min(ln - 1, w.k) + 1 + min(w.M, (ln - 1) // w.pi)
        pidx = torch.from_numpy(pos.astype(np.int64)).to(DEV)
        sidx = torch.from_numpy(seqs.astype(np.int64)).to(DEV)
        kr = host_array(x["k_cache"].index_select(0, sidx).index_select(2, pidx))   # [s, H, |N|, d]
        vr = host_array(x["v_cache"].index_select(0, sidx).index_select(2, pidx))
        for a, s in enumerate(seqs):
            for h in range(H):
                kbuf[0, 0, pos] = kr[a, h]
                vbuf[0, 0, pos] = vr[a, h]
                ref = oracle.decode(qh[s:s + 1, h:h + 1], kbuf, vbuf, np.array([ln], np.int32),
                                    gh[s:s + 1, h:h + 1], w.k, w.pi, w.M, w.scale)
                err = float(np.abs(got[s, h] - ref[0, 0]).max())
                worst = max(worst, err)
                assert err <= BF16_TOL, (s, h, err)
    max_err(torch.zeros(1), np.array([worst]), "decode_32k every row")
    del x
    torch.cuda.empty_cache()
