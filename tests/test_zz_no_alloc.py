"""piattn_fwd_noalloc (the prefill for callers that cannot allocate) against
piattn_fwd with a caller workspace: the same kernels run on the same inputs,
so the outputs must be identical, on two calls in a row (the second smaller,
so it runs over what the first left in the library-held scratch array), and
a call whose workspace need exceeds the array is refused before launching."""
import pytest
import torch

import sparse_long_context_piattn_amd as pa
from sparse_long_context_piattn_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _both(w, x, **kw):
    args = dict(window_k=w.k, period_pi=w.pi, num_skips=w.M, bidirectional=w.bidir, levels=w.levels,
                cu_seqlens=x.get("cu_seqlens"), **kw)
    ref_lse = torch.empty_like(x["g"])
    ref = pa.fwd(x["q"], x["k"], x["v"], x["g"], lse=ref_lse, **args)
    out = torch.full_like(x["q"], float("nan"))
    lse = torch.full_like(x["g"], float("nan"))
    pa.fwd_noalloc(x["q"], x["k"], x["v"], x["g"], out=out, lse=lse, **args)
    torch.cuda.synchronize()
    return ref, ref_lse, out, lse


def test_noalloc_matches_workspace_entry_two_calls_second_smaller():
    big = wl.WORKLOADS["prefill_8k"]
    small = wl.Workload("small", "fwd", "bf16", B=2, H=3, n=3000, d=64, k=20, pi=64, M=10, seed=71)
    for w in (big, small):
        x = wl.make_fwd_inputs(w, device=DEV)
        ref, ref_lse, out, lse = _both(w, x)
        assert torch.equal(out, ref), w.name
        assert torch.equal(lse, ref_lse), w.name


def test_noalloc_varlen_bidirectional_and_d128():
    wv = wl.Workload("vl", "fwd", "bf16", H=4, d=64, k=12, pi=32, M=6, bidir=True, nseq=4,
                     len_lo=1, len_hi=2000, seed=72)
    x = wl.make_fwd_inputs(wv, device=DEV, lengths=[1500, 0, 37, 2000])
    ref, ref_lse, out, lse = _both(wv, x)
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
    w128 = wl.Workload("d128", "fwd", "bf16", B=1, H=2, n=5000, d=128, k=128, pi=256, M=12, seed=73)
    x = wl.make_fwd_inputs(w128, device=DEV)
    ref, ref_lse, out, lse = _both(w128, x)
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)


def test_noalloc_refuses_a_call_beyond_its_scratch():
    pat = pa.make_pattern(64, 128, 16)
    n = pa.binding.NOALLOC_SCRATCH_BYTES // (8 * 16) + 64        # one head more than fits, B = 1, H = 16
    assert pa.fwd_workspace_bytes(1, 1, 16, n, 64, pat) > pa.binding.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((1, 16, n, 64), dtype=torch.bfloat16, device=DEV)
    g = torch.zeros((1, 16, n), dtype=torch.float32, device=DEV)
    out = torch.full_like(q, 3.0)
    with pytest.raises(pa.PiattnError) as e:
        pa.fwd_noalloc(q, q, q, g, out=out, window_k=64, period_pi=128, num_skips=16)
    assert e.value.code == 3 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
