"""Bit-exact index sets of the compute kernels, read back through their outputs.

The neighbour dump (piattn_neighbors) is checked bit-exactly elsewhere, but
the MFMA kernels build their own band masks.  A key dropped from (or added
to) a row with a small weight would stay inside the value tolerance, so
these tests read each kernel's membership matrix out of its results and
compare it bit-exactly with the oracle's neighbour table
(oracle.neighbor_table: L(i) and S(i) by membership tests; gist.science,
"pi-Attention ...", section 2, "Ring-Local Attention" and "pi-Skip
Attention").

Forward probe.  Head h of a batch probes key j0 = h: every query is e_0,
k_{j0} = C e_0 with scale*C ~ 32 and every other key 0, v_{j0} = all ones and
every other value 0.  Row i's output is then ~1 when j0 is one of its keys
(its weight is ~1) and 0 when not.  A gate logit of +40 adds -40 to skip
logits, so j0 then shows only where it is a local key; -40 shows it only
where it is a skip key.  A row without skip keys gets no prior (it would be a
constant shift), so there every key shows in both runs.  A threshold of 0.5
separates the two outcomes with a wide margin: a suppressed key keeps a
weight below e^-8.

Backward probes (exact zeros; gate logits +inf / -inf give the suppressed
kind a weight of exactly 0):
  * key side (dk, dv): head h probes query row i0 = h, dout is zero except
    on that row, q, k, v are random.  dv_j = P_{i0 j} dout_{i0} is nonzero
    exactly for the keys j of row i0, and so is dk_j = scale dS_{i0 j} q_{i0},
    except when row i0 has a single key: P = 1 there, so dS vanishes up to
    rounding, and only the absence of every other key is checked.
  * query side (dq): head h probes key j0 = h as in the forward probe, with
    logit 1 for it and 0 for the rest, v_{j0} = e_0, dout = e_0 everywhere.
    dq_i = scale dS_{i j0} k_{j0} is nonzero exactly when j0 is a key of row i,
    except on rows with a single key, where the softmax gradient vanishes up
    to rounding (P = 1); there only the absence of other keys is checked.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_long_context_piattn_amd as pa

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"

# name, n, d, k, pi, M, bidir, levels
CASES = [
    ("causal", 300, 64, 8, 16, 5, False, ()),
    ("k0", 300, 64, 0, 16, 9, False, ()),
    ("pi_le_k", 300, 64, 20, 8, 10, False, ()),
    ("no_skips", 257, 64, 16, 32, 0, False, ()),
    ("long_band", 200, 64, 5, 7, 30, False, ()),
    ("pi64", 300, 64, 20, 64, 3, False, ()),
    ("short_n", 37, 64, 8, 16, 2, False, ()),
    ("n1", 1, 64, 3, 4, 2, False, ()),
    ("bidir", 300, 64, 12, 16, 6, True, ()),
    ("bidir_pi_le_k", 300, 64, 20, 8, 9, True, ()),
    ("bidir_pi64", 300, 64, 20, 64, 2, True, ()),
    ("d128", 300, 128, 10, 16, 8, False, ()),
    ("d128_bidir", 240, 128, 6, 16, 4, True, ()),
    ("schedule", 300, 64, 6, 8, 4, False, ((24, 3), (40, 2))),
    ("schedule_bidir", 260, 64, 3, 8, 2, True, ((32, 3),)),
]


def kind_matrix(n, k, pi, M, bidir, levels):
    """[n, n] int8: 1 if j is a local key of row i, 2 if a skip key, else 0."""
    idx, kind, _ = oracle.neighbor_table(n, k, pi, M, bidir, levels=levels)
    K = np.zeros((n, n), np.int8)
    rows = np.repeat(np.arange(n), idx.shape[1])
    flat = idx.reshape(-1)
    ok = flat >= 0
    K[rows[ok], flat[ok]] = kind.reshape(-1)[ok]
    return K


def expected_shows(K):
    """(shown with gate +big, shown with gate -big): [i, j] booleans."""
    has_skip = (K == 2).any(axis=1, keepdims=True)
    local, skip = K == 1, K == 2
    return local, skip | (local & ~has_skip)


def _scale_c(d):
    # k_{j0} entry with scale * C ~ 32 (exact in bf16)
    return {32: 192.0, 64: 256.0, 128: 384.0}[d]


def fwd_probe(n, d, k, pi, M, bidir, levels, kernel, dtype=torch.bfloat16):
    """Membership matrices [i, j] read from the forward kernel `kernel`."""
    H = n
    q = torch.zeros((1, H, n, d), dtype=dtype, device=DEV)
    q[..., 0] = 1
    kk = torch.zeros_like(q)
    vv = torch.zeros_like(q)
    hh = torch.arange(H, device=DEV)
    kk[0, hh, hh, 0] = _scale_c(d)
    vv[0, hh, hh, :] = 1
    shows = []
    for gval in (40.0, -40.0):
        g = torch.full((1, H, n), gval, dtype=torch.float32, device=DEV)
        try:
            with pa.forced_kernels(fwd=kernel):
                out = pa.fwd(q, kk, vv, g, window_k=k, period_pi=pi, num_skips=M,
                             bidirectional=bidir, levels=levels)
        except pa.PiattnError as e:
            if e.code == 2:
                pytest.skip("%s does not take this shape" % kernel)
            raise
        torch.cuda.synchronize()
        o = out[0, :, :, :].float()                   # [j0 = h, i, d]
        assert torch.isfinite(o).all()
        # every column carries the same marker
        assert torch.equal(o.min(dim=2).values > 0.5, o.max(dim=2).values > 0.5)
        shows.append((o[:, :, 0] > 0.5).cpu().numpy().T)   # [i, j0]
    return shows


@pytest.mark.parametrize("kernel", ["split", "resid", "gather"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_membership_bit_exact(case, kernel):
    name, n, d, k, pi, M, bidir, levels = case
    K = kind_matrix(n, k, pi, M, bidir, levels)
    exp_local, exp_skip = expected_shows(K)
    got_local, got_skip = fwd_probe(n, d, k, pi, M, bidir, levels, kernel)
    assert np.array_equal(got_local, exp_local), (name, kernel, np.argwhere(got_local != exp_local)[:8])
    assert np.array_equal(got_skip, exp_skip), (name, kernel, np.argwhere(got_skip != exp_skip)[:8])


@pytest.mark.parametrize("kernel", ["gather", "f32mfma"])
@pytest.mark.parametrize("n,d,k,pi,M,levels", [(200, 32, 6, 16, 5, ()), (150, 64, 20, 7, 9, ()),
                                                (130, 32, 0, 3, 30, ()), (90, 128, 40, 16, 0, ()),
                                                (240, 32, 4, 8, 3, ((16, 4), (32, 2)))])
def test_forward_membership_fp32(kernel, n, d, k, pi, M, levels):
    for bidir in (False, True):
        K = kind_matrix(n, k, pi, M, bidir, levels)
        exp_local, exp_skip = expected_shows(K)
        got_local, got_skip = fwd_probe(n, d, k, pi, M, bidir, levels, kernel, dtype=torch.float32)
        assert np.array_equal(got_local, exp_local), (kernel, bidir)
        assert np.array_equal(got_skip, exp_skip), (kernel, bidir)


@pytest.mark.parametrize("kernel", ["split", "resid", "gather"])
def test_forward_membership_varlen(kernel):
    """Packed sequences of several lengths (one empty, one of a single
    token): head h probes key h of every sequence longer than h."""
    lens = [0, 1, 37, 200, 129]
    k, pi, M, d = 10, 16, 6, 64
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H = int(cu[-1]), max(lens)
    for bidir in (False, True):
        q = torch.zeros((T, H, d), dtype=torch.bfloat16, device=DEV)
        q[..., 0] = 1
        kk = torch.zeros_like(q)
        vv = torch.zeros_like(q)
        for s, L in enumerate(lens):
            hh = torch.arange(L, device=DEV)
            kk[cu[s] + hh, hh, 0] = _scale_c(d)
            vv[cu[s] + hh, hh, :] = 1
        cu_t = torch.from_numpy(cu).to(DEV)
        shows = []
        for gval in (40.0, -40.0):
            g = torch.full((T, H), gval, dtype=torch.float32, device=DEV)
            try:
                with pa.forced_kernels(fwd=kernel):
                    out = pa.fwd(q, kk, vv, g, window_k=k, period_pi=pi, num_skips=M,
                                 bidirectional=bidir, cu_seqlens=cu_t)
            except pa.PiattnError as e:
                if e.code == 2:
                    pytest.skip("%s does not take this shape" % kernel)
                raise
            torch.cuda.synchronize()
            shows.append((out[..., 0].float() > 0.5).cpu().numpy())   # [T, H]
        for s, L in enumerate(lens):
            if L == 0:
                continue
            K = kind_matrix(L, k, pi, M, bidir, ())
            exp_local, exp_skip = expected_shows(K)
            for got, exp, tag in ((shows[0], exp_local, "local"), (shows[1], exp_skip, "skip")):
                sub = got[cu[s]:cu[s] + L, :L]               # [i, j0 = h]
                assert np.array_equal(sub, exp), (kernel, bidir, s, tag)


# ----------------------------------------------------------------- backward

def effective(K, gval):
    """[i, j] keys whose weight is nonzero under gate logit +inf / -inf."""
    local, skip = expected_shows(K)
    return local if gval > 0 else skip


def _bwd(path, q, kk, vv, g, out, dout, lse, k, pi, M, bidir, levels):
    try:
        with pa.forced_kernels(bwd=path):
            return pa.bwd(q, kk, vv, g, out, dout, window_k=k, period_pi=pi, num_skips=M,
                          bidirectional=bidir, lse=lse if path == "band" else None, levels=levels)
    except pa.PiattnError as e:
        if e.code == 2:
            pytest.skip("%s backward does not take this shape" % path)
        raise


def bwd_key_side(n, d, k, pi, M, bidir, levels, path, gval):
    """[i0, j] from dv and from dk: head h probes query row i0 = h."""
    H = n
    gen = torch.Generator(device=DEV).manual_seed(1234 + n + d)
    q, kk, vv = [(0.5 * torch.randn((1, H, n, d), generator=gen, device=DEV)).to(torch.bfloat16)
                 for _ in range(3)]
    g = torch.full((1, H, n), gval, dtype=torch.float32, device=DEV)
    lse = torch.empty_like(g)
    out = pa.fwd(q, kk, vv, g, window_k=k, period_pi=pi, num_skips=M, bidirectional=bidir,
                 levels=levels, lse=lse)
    dout = torch.zeros_like(q)
    hh = torch.arange(H, device=DEV)
    dout[0, hh, hh, :] = (0.5 + torch.rand((H, d), generator=gen, device=DEV)).to(torch.bfloat16)
    dq, dk, dv, dg = _bwd(path, q, kk, vv, g, out, dout, lse, k, pi, M, bidir, levels)
    torch.cuda.synchronize()
    for t in (dq, dk, dv, dg):
        assert torch.isfinite(t.float()).all()
    mem_v = (dv[0].float() != 0).any(dim=2).cpu().numpy()   # [i0 = h, j]
    mem_k = (dk[0].float() != 0).any(dim=2).cpu().numpy()
    return mem_v, mem_k


def bwd_query_side(n, d, k, pi, M, bidir, levels, path, gval):
    """[i, j0] from dq: head h probes key j0 = h."""
    H = n
    scale = 1.0 / np.sqrt(d)
    q = torch.zeros((1, H, n, d), dtype=torch.bfloat16, device=DEV)
    q[..., 0] = 1
    kk = torch.zeros_like(q)
    vv = torch.zeros_like(q)
    hh = torch.arange(H, device=DEV)
    kk[0, hh, hh, 0] = float(torch.tensor(1.0 / scale).to(torch.bfloat16))   # logit ~1
    vv[0, hh, hh, 0] = 1
    g = torch.full((1, H, n), gval, dtype=torch.float32, device=DEV)
    lse = torch.empty_like(g)
    out = pa.fwd(q, kk, vv, g, window_k=k, period_pi=pi, num_skips=M, bidirectional=bidir,
                 levels=levels, lse=lse)
    dout = torch.zeros_like(q)
    dout[..., 0] = 1
    dq, dk, dv, dg = _bwd(path, q, kk, vv, g, out, dout, lse, k, pi, M, bidir, levels)
    torch.cuda.synchronize()
    for t in (dq, dk, dv, dg):
        assert torch.isfinite(t.float()).all()
    return (dq[0, :, :, 0].float() != 0).cpu().numpy().T       # [i, j0]


BWD_CASES = [c for c in CASES if c[0] in ("causal", "k0", "pi_le_k", "no_skips", "long_band", "pi64",
                                          "short_n", "bidir", "bidir_pi_le_k", "d128", "d128_bidir",
                                          "schedule", "schedule_bidir")]


@pytest.mark.parametrize("path", ["band", "gather"])
@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_membership_bit_exact(case, path):
    name, n, d, k, pi, M, bidir, levels = case
    K = kind_matrix(n, k, pi, M, bidir, levels)
    for gval in (float("inf"), float("-inf")):
        E = effective(K, gval)                                 # [i, j]
        mem_v, mem_k = bwd_key_side(n, d, k, pi, M, bidir, levels, path, gval)
        single = E.sum(axis=1) == 1                            # P = 1: dS vanishes identically
        assert np.array_equal(mem_v, E), (name, path, gval, "dv", np.argwhere(mem_v != E)[:8])
        assert np.array_equal(mem_k[~single], E[~single]), (name, path, gval, "dk",
                                                             np.argwhere(mem_k[~single] != E[~single])[:8])
        # single-key rows: dS is zero only up to rounding (D and dP are summed in
        # different orders), so only keys outside the set are ruled out there
        assert not (mem_k[single] & ~E[single]).any(), (name, path, gval)
        mem_q = bwd_query_side(n, d, k, pi, M, bidir, levels, path, gval)
        assert np.array_equal(mem_q[~single], E[~single]), (name, path, gval, "dq",
                                                             np.argwhere(mem_q[~single] != E[~single])[:8])
        assert not (mem_q[single] & ~E[single]).any(), (name, path, gval)
