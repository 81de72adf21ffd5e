"""Pins for the CPU oracle: it is checked against facts that do not come from it.

* the sliding-window worked example printed on the ultralytics glossary page
  (58 vs 136 scored pairs, last-token reach 4 -> 7 -> 10 -> 13);
* closed-form pair counts (sums of min() terms worked out by hand);
* brute-force membership from index offsets (oracle/dense.py);
* library routines: torch scaled_dot_product_attention (fp64, CPU) for the
  dense-causal, dense-bidirectional, alpha -> 1 and alpha -> 0 special cases,
  and torch.logsumexp for the two-set mixture identity that the pages'
  "local sweep / periodic gather / fusion" decomposition implies;
* invariants (row 0, constant values, convex hull, varlen = separate runs,
  decode = last prefill row).

None of these needs a GPU.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _single(q, k, v, g, kw, pi, M, bidir, scale, want_lse=False):
    """Run the C oracle on one (sequence, head) given [n, d] arrays."""
    n, d = q.shape
    res = oracle.fwd(q[:, None, :], k[:, None, :], v[:, None, :], g[:, None],
                     np.array([0, n]), kw, pi, M, bidir, scale, want_lse=want_lse)
    if want_lse:
        return res[0], res[1]
    return res


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    o = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, is_causal=causal,
                                       scale=scale)
    return o[0, 0].numpy()


# ---------------------------------------------------------------- index sets

def test_swa_worked_example_counts_and_reach(oracle_lib):
    gold = json.load(open(os.path.join(GOLDEN, "swa_worked_example.json")))
    n, w = gold["seq_len"], gold["window"]
    idx, kind, cnt = oracle.neighbor_table(n, w - 1, 1, 0, False)
    assert int(cnt.sum()) == gold["scores_with_window"]
    _, _, cnt_full = oracle.neighbor_table(n, n - 1, 1, 0, False)
    assert int(cnt_full.sum()) == gold["scores_full_causal"]
    # neighbour matrix and its repeated boolean products
    mask = np.zeros((n, n), bool)
    for i in range(n):
        mask[i, idx[i, :cnt[i]]] = True
    reach = mask.copy()
    got = []
    for _layer in range(len(gold["last_token_reach_by_layer"])):
        got.append(int(reach[-1].sum()))
        reach = (mask.astype(np.int64) @ reach.astype(np.int64)) > 0
    assert got == gold["last_token_reach_by_layer"]


@pytest.mark.parametrize("bidir", [False, True])
def test_membership_matches_offset_masks(oracle_lib, bidir):
    """Exhaustive tiny sweep: oracle neighbour lists == offset-mask formulation."""
    for n in (1, 2, 5, 13, 24):
        for kw in range(0, n + 1):
            for pi in range(1, n + 2):
                for M in range(0, n // pi + 2):
                    local, skip = dense.masks(n, kw, pi, M, bidir)
                    idx, kind, cnt = oracle.neighbor_table(n, kw, pi, M, bidir)
                    for i in range(n):
                        ii = idx[i, :cnt[i]]
                        kk = kind[i, :cnt[i]]
                        assert np.all(np.diff(ii) > 0)
                        assert set(ii[kk == 1]) == set(np.nonzero(local[i])[0])
                        assert set(ii[kk == 2]) == set(np.nonzero(skip[i])[0])


def _counts(n, kw, pi, M, bidir):
    tot_l = tot_s = 0
    for i in range(n):
        _, kind = oracle.neighbors(n, kw, pi, M, bidir, i)
        tot_l += int((kind == 1).sum())
        tot_s += int((kind == 2).sum())
    return tot_l, tot_s


@pytest.mark.parametrize("n,kw,pi,M", [
    (256, 8, 16, 4),          # tiny fp32 workload
    (8192, 64, 128, 16),      # 8K prefill workload
    (1000, 3, 7, 9),
    (4096, 100, 101, 40),
])
def test_closed_form_causal_counts(oracle_lib, n, kw, pi, M):
    assert pi > kw and n >= M * pi and n > kw
    loc, sk = _counts(n, kw, pi, M, False)
    assert loc == n * (kw + 1) - kw * (kw + 1) // 2
    assert sk == pi * M * (M - 1) // 2 + M * (n - M * pi)


@pytest.mark.parametrize("n,kw,pi,M", [
    (4096, 32, 64, 32),       # shortest bidirectional varlen sequence
    (5000, 32, 64, 32),
    (777, 5, 9, 20),
])
def test_closed_form_bidir_counts(oracle_lib, n, kw, pi, M):
    assert pi > kw and n >= M * pi and n > 2 * kw
    loc, sk = _counts(n, kw, pi, M, True)
    assert loc == n * (2 * kw + 1) - kw * (kw + 1)
    assert sk == 2 * M * n - pi * M * (M + 1)


def test_long_prefill_counts_sampled(oracle_lib):
    """128K prefill: per-row counts equal min() closed forms on sampled rows."""
    n, kw, pi, M = 131072, 128, 256, 64
    rng = np.random.default_rng(5)
    rows = np.concatenate([np.arange(0, 600), rng.integers(0, n, 2000), np.arange(n - 50, n)])
    for i in rows:
        _, kind = oracle.neighbors(n, kw, pi, M, False, int(i))
        assert (kind == 1).sum() == min(i, kw) + 1
        assert (kind == 2).sum() == min(M, i // pi)


def test_decode_row_counts(oracle_lib):
    # decode workload: query at position 32767 of a 32768-token cache
    idx, kind = oracle.neighbors(32768, 256, 512, 63, False, 32767)
    assert (kind == 1).sum() == 257 and (kind == 2).sum() == 63
    assert idx[0] == 32767 - 63 * 512 and idx[-1] == 32767


# ------------------------------------------------------------------- values

@pytest.mark.parametrize("bidir", [False, True])
def test_dense_special_case_is_sdpa(oracle_lib, bidir):
    """k >= n-1 and M = 0: plain softmax attention (the gate is a constant shift)."""
    n, d = 37, 16
    q, k, v = (_rand((n, d), s) for s in (1, 2, 3))
    g = _rand(n, 4) * 3
    got = _single(q, k, v, g, n - 1, 5, 0, bidir, 1 / math.sqrt(d))
    ref = _sdpa(q, k, v, causal=not bidir)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_alpha_one_is_ring_local(oracle_lib):
    """g = +inf: skip weights vanish; result = SDPA with the causal window mask."""
    n, d, kw, pi, M = 64, 8, 3, 8, 5
    q, k, v = (_rand((n, d), s) for s in (11, 12, 13))
    pos = np.arange(n)
    off = pos[:, None] - pos[None, :]
    mask = (off >= 0) & (off < kw + 1)
    ref = _sdpa(q, k, v, mask=mask)
    got = _single(q, k, v, np.full(n, np.inf), kw, pi, M, False, 1 / math.sqrt(d))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    near = _single(q, k, v, np.full(n, 40.0), kw, pi, M, False, 1 / math.sqrt(d))
    np.testing.assert_allclose(near, ref, rtol=0, atol=1e-12)


def test_alpha_zero_is_skip_only(oracle_lib):
    """g = -inf: rows with skips attend over the skip set alone."""
    n, d, kw, pi, M = 64, 8, 3, 8, 5
    q, k, v = (_rand((n, d), s) for s in (21, 22, 23))
    local, skip = dense.masks(n, kw, pi, M, False)
    has = skip.any(1)
    mask = np.where(has[:, None], skip, local)
    ref = _sdpa(q, k, v, mask=mask)
    got = _single(q, k, v, np.full(n, -np.inf), kw, pi, M, False, 1 / math.sqrt(d))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("bidir", [False, True])
def test_mixture_identity(oracle_lib, bidir):
    """One softmax with a log-prior equals the alpha-weighted mix of the two
    per-set softmaxes, weighted by their normalisers:
        o = (a Z_L O_L + (1-a) Z_S O_S) / (a Z_L + (1-a) Z_S).
    O_L, O_S from torch SDPA; Z_L, Z_S from torch.logsumexp."""
    n, d, kw, pi, M = 70, 12, 4, 9, 6
    scale = 0.3
    q, k, v = (_rand((n, d), s) for s in (31, 32, 33))
    g = _rand(n, 34) * 2
    local, skip = dense.masks(n, kw, pi, M, bidir)
    has = skip.any(1)
    got, lse = _single(q, k, v, g, kw, pi, M, bidir, scale, want_lse=True)
    o_l = _sdpa(q, k, v, mask=local, scale=scale)
    skip_safe = np.where(has[:, None], skip, local)
    o_s = _sdpa(q, k, v, mask=skip_safe, scale=scale)
    s = torch.from_numpy(scale * (q @ k.T))
    lz_l = torch.logsumexp(s.masked_fill(~torch.from_numpy(local), -math.inf), 1).numpy()
    lz_s = torch.logsumexp(s.masked_fill(~torch.from_numpy(skip_safe), -math.inf), 1).numpy()
    a = 1 / (1 + np.exp(-g))
    wl = a * np.exp(lz_l)
    ws = (1 - a) * np.exp(lz_s)
    ref = np.where(has[:, None], (wl[:, None] * o_l + ws[:, None] * o_s) / (wl + ws)[:, None], o_l)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)
    ref_lse = np.where(has, np.log(wl + ws), lz_l)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-11)


@pytest.mark.parametrize("seed", range(6))
def test_c_oracle_matches_dense(oracle_lib, seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 60))
    d = int(rng.choice([4, 8, 16]))
    kw = int(rng.integers(0, 12))
    pi = int(rng.integers(1, 20))
    M = int(rng.integers(0, 8))
    bidir = bool(seed % 2)
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    g = rng.standard_normal(n) * 3
    got, lse = _single(q, k, v, g, kw, pi, M, bidir, 0.25, want_lse=True)
    ref, rlse = dense.attention(q, k, v, g, kw, pi, M, bidir, 0.25, want_lse=True)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-12)


def test_invariants(oracle_lib):
    n, d, kw, pi, M = 50, 8, 2, 7, 4
    q, k, v = (_rand((n, d), s) for s in (41, 42, 43))
    g = _rand(n, 44)
    got = _single(q, k, v, g, kw, pi, M, False, 0.5)
    np.testing.assert_array_equal(got[0], v[0])           # row 0 sees only itself
    const = np.tile(_rand(d, 45), (n, 1))
    np.testing.assert_allclose(_single(q, k, const, g, kw, pi, M, False, 0.5), const,
                               rtol=0, atol=1e-13)
    for i in range(n):                                      # convex hull of its keys
        ii, _ = oracle.neighbors(n, kw, pi, M, False, i)
        assert np.all(got[i] <= v[ii].max(0) + 1e-12)
        assert np.all(got[i] >= v[ii].min(0) - 1e-12)


def test_varlen_equals_separate(oracle_lib):
    lens = [5, 17, 1, 30]
    H, d, kw, pi, M = 3, 8, 3, 4, 3
    T = sum(lens)
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    g = rng.standard_normal((T, H))
    cu = np.concatenate([[0], np.cumsum(lens)])
    for bidir in (False, True):
        packed = oracle.fwd(q, k, v, g, cu, kw, pi, M, bidir, 0.4).reshape(T, H, d)
        for s in range(len(lens)):
            a, b = cu[s], cu[s + 1]
            alone = oracle.fwd(q[a:b], k[a:b], v[a:b], g[a:b], [0, b - a], kw, pi, M, bidir,
                               0.4).reshape(b - a, H, d)
            np.testing.assert_array_equal(packed[a:b], alone)


def test_decode_equals_last_prefill_row(oracle_lib):
    S, H, L, d, kw, pi, M = 3, 2, 90, 16, 6, 10, 7
    rng = np.random.default_rng(8)
    kc, vc = rng.standard_normal((S, H, L, d)), rng.standard_normal((S, H, L, d))
    lens = np.array([90, 41, 1], np.int32)
    g = rng.standard_normal((S, H))
    q = rng.standard_normal((S, H, d))
    out = oracle.decode(q, kc, vc, lens, g, kw, pi, M, 0.25)
    for s in range(S):
        n = int(lens[s])
        for h in range(H):
            qq = kc[s, h, :n].copy()
            qq[n - 1] = q[s, h]
            gg = np.zeros(n)
            gg[n - 1] = g[s, h]
            ref = _single(qq, kc[s, h, :n], vc[s, h, :n], gg, kw, pi, M, False, 0.25)
            np.testing.assert_array_equal(out[s, h], ref[n - 1])


def test_bf16_inputs_read_exactly(oracle_lib):
    n, H, d = 20, 2, 8
    t = torch.randn(n, H, d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    as64 = t.double().numpy()
    g = np.zeros((n, H))
    a = oracle.fwd(bits, bits, bits, g, [0, n], 2, 3, 2, False, 0.3)
    b = oracle.fwd(as64, as64, as64, g, [0, n], 2, 3, 2, False, 0.3)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- backward
# The backward oracle is pinned to central finite differences of the
# forward oracle (itself pinned above): for L = sum(dout * out), every
# element of q, k, v and g is moved by +-h and (L+ - L-) / 2h compared with
# the analytic gradient.  The truncation error is O(h^2 * third derivative)
# and the rounding error O(eps * |L| / h): with h = 1e-5 both stay below 1e-7.

def _fd_case(seed, lens, H, d, kw, pi, M, bidir, scale, gstd=1.5):
    T = sum(lens)
    q, k, v = (_rand((T, H, d), seed + i) for i in range(3))
    g = _rand((T, H), seed + 3, gstd)
    dout = _rand((T, H, d), seed + 4)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k, v, g, dout, cu


def _loss(q, k, v, g, dout, cu, kw, pi, M, bidir, scale):
    out = oracle.fwd(q, k, v, g, cu, kw, pi, M, bidir, scale)
    return float((out * dout.reshape(out.shape)).sum())


@pytest.mark.parametrize("bidir", [False, True])
@pytest.mark.parametrize("kw,pi,M", [(2, 3, 2), (0, 2, 3), (4, 3, 1), (3, 1, 2)])
def test_backward_matches_finite_differences(oracle_lib, bidir, kw, pi, M):
    lens = [9, 13]
    q, k, v, g, dout, cu = _fd_case(7 * kw + pi + 11 * M + int(bidir), lens, 2, 3, kw, pi, M, bidir, 0.7)
    args = (kw, pi, M, bidir, 0.7)
    dq, dk, dv, dg = oracle.bwd(q, k, v, g, dout, cu, *args)
    h = 1e-5
    worst = 0.0
    for name, x, gx in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("g", g, dg)):
        flat, gflat = x.reshape(-1), gx.reshape(-1)
        for e in range(flat.size):
            keep = flat[e]
            flat[e] = keep + h
            lp = _loss(q, k, v, g, dout, cu, *args)
            flat[e] = keep - h
            lm = _loss(q, k, v, g, dout, cu, *args)
            flat[e] = keep
            fd = (lp - lm) / (2 * h)
            worst = max(worst, abs(fd - gflat[e]))
            assert abs(fd - gflat[e]) <= 1e-6 * max(1.0, abs(fd)), (name, e, fd, gflat[e])
    assert worst <= 1e-6


def test_backward_gate_gradient_vanishes_without_skips(oracle_lib):
    # M = 0: no row has skip keys, so no prior and no dependence on g
    q, k, v, g, dout, cu = _fd_case(3, [12], 2, 4, 3, 4, 0, False, 0.5)
    dq, dk, dv, dg = oracle.bwd(q, k, v, g, dout, cu, 3, 4, 0, False, 0.5)
    assert not dg.any()
    assert np.abs(dq).max() > 0 and np.abs(dv).max() > 0


def test_backward_dv_columns_sum_to_dout(oracle_lib):
    # each row's softmax weights sum to 1, so summed over all keys dv equals
    # dout summed over all rows (per sequence and head)
    lens = [10, 7]
    q, k, v, g, dout, cu = _fd_case(5, lens, 3, 4, 2, 3, 2, True, 0.9)
    dq, dk, dv, dg = oracle.bwd(q, k, v, g, dout, cu, 2, 3, 2, True, 0.9)
    for s in range(len(lens)):
        sl = slice(cu[s], cu[s + 1])
        np.testing.assert_allclose(dv[sl].sum(axis=0), dout[sl].sum(axis=0), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- skip schedules
# A schedule is a list of levels (pi_r, M_r) whose skip sets are unioned (the
# hierarchical skip schedules the Dutch gist.science summary names as future
# work, section 5 "Betekenis en Conclusie").  Pins: the dense-mask oracle
# (an elementwise OR of per-level masks, written independently), closed-form
# pair counts from the set of distinct distances, and the fact that levels
# whose distances another level already has change nothing.

def _distances(kw, levels):
    return sorted({m * p for p, M in levels for m in range(1, M + 1) if m * p > kw})


@pytest.mark.parametrize("bidir", [False, True])
@pytest.mark.parametrize("n,kw,levels", [
    (200, 3, [(8, 2), (4, 3), (16, 2)]),
    (300, 5, [(16, 4), (32, 4), (64, 4)]),
    (150, 2, [(3, 9), (5, 6)]),
    (97, 20, [(8, 1), (7, 5), (50, 2)]),
])
def test_schedule_closed_form_counts(oracle_lib, n, kw, levels, bidir):
    (pi, M), extra = levels[0], levels[1:]
    idx, kind, cnt = oracle.neighbor_table(n, kw, pi, M, bidir, levels=extra)
    skips = int((kind == 2).sum())
    per_dir = sum(max(0, n - dd) for dd in _distances(kw, levels))
    assert skips == (2 if bidir else 1) * per_dir
    # every list is strictly ascending (no key twice)
    for r in range(n):
        row = idx[r, :cnt[r]]
        assert np.all(np.diff(row) > 0)


@pytest.mark.parametrize("seed", range(8))
def test_schedule_c_oracle_matches_dense(oracle_lib, seed):
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(1, 70))
    d = int(rng.choice([4, 8]))
    kw = int(rng.integers(0, 10))
    nlev = int(rng.integers(1, 4))
    levels = [(int(rng.integers(1, 14)), int(rng.integers(0, 7))) for _ in range(nlev)]
    bidir = bool(seed % 2)
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    g = rng.standard_normal(n) * 3
    (pi, M), extra = levels[0], levels[1:]
    out, lse = oracle.fwd(q[:, None], k[:, None], v[:, None], g[:, None], [0, n], kw, pi, M, bidir, 0.3,
                          want_lse=True, levels=extra)
    ref, rlse = dense.attention(q, k, v, g, kw, pi, M, bidir, 0.3, want_lse=True, levels=extra)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("bidir", [False, True])
def test_schedule_redundant_levels_change_nothing(oracle_lib, bidir):
    # (2 pi, M/2) and (pi, 1) add only distances (pi, M) already has
    n, d, kw, pi, M = 120, 8, 3, 5, 6
    q, k, v = (_rand((n, 2, d), s) for s in (61, 62, 63))
    g = _rand((n, 2), 64, 2.0)
    cu = [0, n]
    one = oracle.fwd(q, k, v, g, cu, kw, pi, M, bidir, 0.4)
    many = oracle.fwd(q, k, v, g, cu, kw, pi, M, bidir, 0.4, levels=[(2 * pi, M // 2), (pi, 1)])
    assert np.array_equal(one, many)
    dout = _rand((n, 2, d), 65)
    a = oracle.bwd(q, k, v, g, dout, cu, kw, pi, M, bidir, 0.4)
    b = oracle.bwd(q, k, v, g, dout, cu, kw, pi, M, bidir, 0.4, levels=[(2 * pi, M // 2)])
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


# ------------------------------------------------------ receptive field of layers
# The English gist.science summary (section 3 "Key Contributions", item
# "Theoretical Receptive Field Improvement") credits the periodic skips with a
# "binary lifting" growth of the receptive field over stacked layers.  The
# computable reading: key i - delta reaches query i through L layers of the
# pattern exactly when some path of at most L neighbour hops joins them (the
# repeated boolean products of the SWA worked example above; a token's own
# position is in its window, so shorter paths count too).  In a causal pattern
# every hop goes back by one of the pattern's offsets: 0..k in the window, or
# a skip distance.  For k < pi a skip hop replaces at least two window hops,
# so a shortest path covers q = delta // pi periods with skip hops and the
# rest r = delta % pi with ceil(r / k) window hops, and:
#   one period (pi, M):                  ceil(q / M) + ceil(r / k)
#   doubling schedule (pi 2^l, 1),
#   l = 0 .. R-1:                        q // 2^(R-1) + popcount(q % 2^(R-1)) + ceil(r / k)
# -- the second is the binary expansion of q: the layers needed grow with the
# logarithm of the distance, while a single period needs q / M of them.  Both
# are checked against breadth-first search over the oracle's neighbour lists.

def _min_layers(n, kw, pi, M, levels, i):
    idx, _, cnt = oracle.neighbor_table(n, kw, pi, M, False, q_begin=0, q_count=n, levels=levels)
    mask = np.zeros((n, n), bool)
    for r in range(n):
        mask[r, idx[r, :cnt[r]]] = True
    depth = np.full(n, -1)
    depth[i] = 0
    front = np.zeros(n, bool)
    front[i] = True
    layer = 0
    while front.any():
        layer += 1
        nxt = mask[front].any(axis=0) & (depth < 0)
        depth[nxt] = layer
        front = nxt
    return depth


def _ceil(a, b):
    return -(-a // b)


@pytest.mark.parametrize("n,kw,pi,M", [(700, 3, 8, 4), (500, 5, 16, 1), (400, 1, 4, 7), (300, 6, 7, 0)])
def test_receptive_field_single_period(oracle_lib, n, kw, pi, M):
    for i in (n - 1, n // 2 + 3):
        depth = _min_layers(n, kw, pi, M, None, i)
        for delta in range(0, i + 1):
            q, r = divmod(delta, pi)
            if M == 0:
                want = _ceil(delta, kw)
            else:
                want = _ceil(q, M) + _ceil(r, kw)
            assert depth[i - delta] == want, (i, delta)
        assert np.all(depth[i + 1:] == -1)                 # causal: nothing after i


@pytest.mark.parametrize("n,kw,pi,R", [(1200, 3, 8, 5), (900, 2, 5, 6), (640, 4, 9, 3)])
def test_receptive_field_doubling_schedule_is_binary_lifting(oracle_lib, n, kw, pi, R):
    levels = [(pi << l, 1) for l in range(1, R)]
    top = 1 << (R - 1)
    i = n - 1
    depth = _min_layers(n, kw, pi, 1, levels, i)
    for delta in range(0, i + 1):
        q, r = divmod(delta, pi)
        want = q // top + bin(q % top).count("1") + _ceil(r, kw)
        assert depth[i - delta] == want, delta
    # within R layers the periods alone reach back (2^R - 1) pi: every
    # multiple of pi up to there, each in popcount(q) <= R layers
    assert all(depth[i - m * pi] <= R for m in range(1, min(i // pi, (1 << R) - 1) + 1))


def test_schedule_decode_equals_last_prefill_row(oracle_lib):
    n, d, kw = 90, 8, 4
    levels = [(6, 3), (12, 3), (24, 3)]
    q, k, v = (_rand((n, 1, d), s) for s in (71, 72, 73))
    g = _rand((n, 1), 74)
    out = oracle.fwd(q, k, v, g, [0, n], kw, 6, 3, False, 0.5, levels=levels[1:])
    dec = oracle.decode(q[n - 1:n], k.transpose(1, 0, 2)[None], v.transpose(1, 0, 2)[None], [n],
                        g[n - 1:n], kw, 6, 3, 0.5, levels=levels[1:])
    np.testing.assert_allclose(dec[0], out[n - 1:n], rtol=0, atol=1e-13)


@pytest.mark.parametrize("bidir", [False, True])
def test_schedule_backward_matches_finite_differences(oracle_lib, bidir):
    lens = [11, 14]
    levels = [(2, 2), (3, 2), (6, 2)]
    q, k, v, g, dout, cu = _fd_case(91 + int(bidir), lens, 2, 3, 1, 2, 2, bidir, 0.6)

    def loss():
        out = oracle.fwd(q, k, v, g, cu, 1, 2, 2, bidir, 0.6, levels=levels[1:])
        return float((out * dout.reshape(out.shape)).sum())

    dq, dk, dv, dg = oracle.bwd(q, k, v, g, dout, cu, 1, 2, 2, bidir, 0.6, levels=levels[1:])
    h = 1e-5
    for name, x, gx in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("g", g, dg)):
        flat, gflat = x.reshape(-1), gx.reshape(-1)
        for e in range(flat.size):
            keep = flat[e]
            flat[e] = keep + h
            lp = loss()
            flat[e] = keep - h
            lm = loss()
            flat[e] = keep
            fd = (lp - lm) / (2 * h)
            assert abs(fd - gflat[e]) <= 1e-6 * max(1.0, abs(fd)), (name, e, fd, gflat[e])


# ---------------------------------------------------------------- gate and output projection
# oracle/proj.py writes the two maps as numpy products; the pins are
# brute-force loops over every index on tiny sizes, and special cases whose
# result is known without arithmetic (one-hot inputs pick a weight entry,
# identity weights return the concatenated heads).
from oracle import proj as oproj


def test_proj_matches_brute_force_loops():
    rng = np.random.default_rng(11)
    B, n, Dm, H, d, Dout = 2, 3, 5, 4, 2, 3
    x = rng.standard_normal((B, n, Dm))
    wg = rng.standard_normal((H, Dm))
    bg = rng.standard_normal(H)
    g = oproj.gate_logits(x, wg, bg)
    for b in range(B):
        for h in range(H):
            for i in range(n):
                acc = bg[h]
                for c in range(Dm):
                    acc += x[b, i, c] * wg[h, c]
                assert abs(g[b, h, i] - acc) <= 1e-12
    o = rng.standard_normal((B, H, n, d))
    wo = rng.standard_normal((Dout, H * d))
    bo = rng.standard_normal(Dout)
    y = oproj.out_proj(o, wo, bo)
    for b in range(B):
        for i in range(n):
            for r in range(Dout):
                acc = bo[r]
                for h in range(H):
                    for c in range(d):
                        acc += o[b, h, i, c] * wo[r, h * d + c]
                assert abs(y[b, i, r] - acc) <= 1e-12


def test_proj_special_cases():
    B, n, Dm, H, d = 1, 4, 6, 3, 2
    x = np.zeros((B, n, Dm))
    x[0, 2, 4] = 1.0                            # one-hot token 2, feature 4
    wg = np.arange(H * Dm, dtype=np.float64).reshape(H, Dm)
    g = oproj.gate_logits(x, wg)
    assert np.array_equal(g[0, :, 2], wg[:, 4]) and not g[0, :, [0, 1, 3]].any()
    o = np.arange(B * H * n * d, dtype=np.float64).reshape(B, H, n, d)
    y = oproj.out_proj(o, np.eye(H * d))
    for h in range(H):
        assert np.array_equal(y[0, :, h * d:(h + 1) * d], o[0, h])
    bits = np.array([[0x3f80, 0x4000]], np.uint16)   # bf16 1.0 and 2.0, read exactly
    assert np.array_equal(oproj.gate_logits(bits[None], np.array([[0x3f80, 0x3f80]], np.uint16)), [[[3.0]]])
