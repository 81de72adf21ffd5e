"""GPU tests of the rolling decode cache (position j in row j mod W,
W = max(k, M*pi) + 1): decode over a rolling cache must give bit for bit
what decode gives over a linear cache holding the same positions, and match
the fp64 oracle on the linear history; appends place each new row at
pos mod W."""
import numpy as np
import pytest
import torch

import sparse_long_context_piattn_amd as pa
from sparse_long_context_piattn_amd import workloads as wl

import oracle
from helpers import BF16_TOL, host_array, max_err, tol_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def ring_from_linear(cache, lens, W, fill=1e4):
    """Rolling cache [S, H, W, d] holding the last W positions of each
    sequence of a linear cache [S, H, L, d]; rows no position owns hold
    `fill` (large, so that reading one would show)."""
    S, H, L, d = cache.shape
    ring = torch.full((S, H, W, d), fill, dtype=cache.dtype, device=cache.device)
    for s, n in enumerate(lens):
        j = torch.arange(max(0, n - W), n, device=cache.device)
        ring[s, :, j % W] = cache[s, :, j]
    return ring


def oracle_decode(x, w):
    return oracle.decode(host_array(x["q"]), host_array(x["k_cache"]), host_array(x["v_cache"]),
                         x["lens"].cpu().numpy(), x["g"].cpu().double().numpy(), w.k, w.pi, w.M,
                         w.scale)


@pytest.mark.parametrize("dt,d,k,pi,M", [("bf16", 128, 20, 16, 5), ("bf16", 64, 40, 8, 3),
                                         ("f32", 32, 12, 16, 2), ("bf16", 128, 64, 32, 1)])
def test_rolling_decode_equals_linear(dt, d, k, pi, M):
    W = pa.rolling_slots(k, pi, M)
    assert W == max(k, M * pi if M >= k // pi + 1 else 0) + 1
    lens = [1, W // 2, W, W + 1, 3 * W + 7, 1000]
    w = wl.Workload("roll", "decode", dt, B=len(lens), H=3, n=max(lens), d=d, k=k, pi=pi, M=M, seed=41)
    x = wl.make_decode_inputs(w, device=DEV, lens=lens)
    kr = ring_from_linear(x["k_cache"], lens, W)
    vr = ring_from_linear(x["v_cache"], lens, W)
    ref = oracle_decode(x, w)
    for splits in (1, 0, 3):
        lin = pa.decode(x["q"], x["k_cache"], x["v_cache"], x["lens"], x["g"], window_k=k, period_pi=pi,
                        num_skips=M, num_splits=splits)
        rol = pa.decode(x["q"], kr, vr, x["lens"], x["g"], window_k=k, period_pi=pi, num_skips=M,
                        num_splits=splits, rolling=True)
        torch.cuda.synchronize()
        assert torch.equal(lin, rol), splits
        assert max_err(rol, ref, "decode rolling %s d=%d splits=%d" % (dt, d, splits)) <= tol_for(w)


def test_cache_append_places_rows_mod_W():
    S, H, d, k, pi, M = 4, 2, 64, 10, 8, 3
    W = pa.rolling_slots(k, pi, M)                        # max(10, 24) + 1 = 25
    assert W == 25
    T = 3 * W + 4
    gen = torch.Generator(device=DEV).manual_seed(5)
    ks = torch.randn((S, H, T, d), generator=gen, device=DEV).to(torch.bfloat16)
    vs = torch.randn((S, H, T, d), generator=gen, device=DEV).to(torch.bfloat16)
    kr = torch.zeros((S, H, W, d), dtype=torch.bfloat16, device=DEV)
    vr = torch.zeros_like(kr)
    offs = [0, 5, W - 1, -10 ** 6]                        # the last sequence never appends
    for t in range(T):
        pos = torch.tensor([t + o if o >= 0 else -1 for o in offs], dtype=torch.int32, device=DEV)
        pa.cache_append(ks[:, :, t].contiguous(), vs[:, :, t].contiguous(), kr, vr, pos)
    torch.cuda.synchronize()
    for s, o in enumerate(offs):
        if o < 0:
            assert not kr[s].any() and not vr[s].any()
            continue
        for t in range(T - W, T):                         # the last W appends own the rows
            assert torch.equal(kr[s, :, (t + o) % W], ks[s, :, t])
            assert torch.equal(vr[s, :, (t + o) % W], vs[s, :, t])


def test_append_then_decode_follows_a_growing_sequence():
    """Generate step by step: append the new token, then decode at it; each
    step equals decode over the linear cache of the same length."""
    S, H, d, k, pi, M = 2, 2, 128, 8, 16, 4
    W = pa.rolling_slots(k, pi, M)                        # 65
    T = 2 * W + 9
    w = wl.Workload("grow", "decode", "bf16", B=S, H=H, n=T, d=d, k=k, pi=pi, M=M, seed=43)
    x = wl.make_decode_inputs(w, device=DEV)
    kr = torch.zeros((S, H, W, d), dtype=torch.bfloat16, device=DEV)
    vr = torch.zeros_like(kr)
    for t in range(T):
        pos = torch.full((S,), t, dtype=torch.int32, device=DEV)
        pa.cache_append(x["k_cache"][:, :, t].contiguous(), x["v_cache"][:, :, t].contiguous(), kr, vr, pos)
        if t % 17 == 0 or t >= T - 3:
            lens = pos + 1
            rol = pa.decode(x["q"], kr, vr, lens, x["g"], window_k=k, period_pi=pi, num_skips=M, rolling=True)
            lin = pa.decode(x["q"], x["k_cache"], x["v_cache"], lens, x["g"], window_k=k, period_pi=pi,
                            num_skips=M)
            torch.cuda.synchronize()
            assert torch.equal(rol, lin), t


def test_rolling_decode_32k_pattern_sampled_sequences():
    """The decode_32k pattern (k=256, pi=512, M=63: W = 32257 rows) on a few
    sequences at the full cache length: rolling equals linear, and the oracle."""
    base = wl.WORKLOADS["decode_32k"]
    w = wl.Workload("dec32r", "decode", "bf16", B=4, H=8, n=base.n, d=base.d, k=base.k, pi=base.pi,
                    M=base.M, seed=44)
    W = pa.rolling_slots(w.k, w.pi, w.M)
    assert W == 63 * 512 + 1
    lens = [base.n, W, W + 1, 5000]
    x = wl.make_decode_inputs(w, device=DEV, lens=lens)
    kr = ring_from_linear(x["k_cache"], lens, W)
    vr = ring_from_linear(x["v_cache"], lens, W)
    lin = pa.decode(x["q"], x["k_cache"], x["v_cache"], x["lens"], x["g"], window_k=w.k, period_pi=w.pi,
                    num_skips=w.M)
    rol = pa.decode(x["q"], kr, vr, x["lens"], x["g"], window_k=w.k, period_pi=w.pi, num_skips=w.M,
                    rolling=True)
    torch.cuda.synchronize()
    assert torch.equal(lin, rol)
    sl = dict(q=x["q"][:, :2], k_cache=x["k_cache"][:, :2], v_cache=x["v_cache"][:, :2], lens=x["lens"],
              g=x["g"][:, :2])
    assert max_err(rol[:, :2], oracle_decode(sl, w), "decode rolling decode_32k pattern") <= BF16_TOL
    del x, kr, vr
    torch.cuda.empty_cache()
