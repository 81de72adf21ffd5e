"""Seeded synthetic workloads (shapes and value distributions only).

This module generates inputs and holds the workload table; it contains none
of the attention arithmetic, so both the HIP path and the CPU oracle may be
fed from it.  Every tensor is drawn from a seeded ``torch.Generator``.

The five workloads are the shapes the pi-Attention write-ups motivate: a tiny
fp32 case, an 8K-token causal prefill, a 128K-token causal prefill, a 32K-cache
decode batch and a bidirectional variable-length encoder batch; a sixth is the
8K prefill under a hierarchical skip schedule.  The pages'
own evaluation data (WikiText-103, PG-19, LRA, MSCOCO, Flickr30K) is not used:
these synthetic tensors stand in for it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "fwd" or "decode"
    dtype: str           # "f32" or "bf16"
    H: int
    d: int
    k: int               # ring-local window half-width
    pi: int              # skip period
    M: int               # skips per direction
    bidir: bool = False
    B: int = 1           # dense fwd: batch; decode: number of sequences
    n: int = 0           # dense fwd: sequence length; decode: cache length
    nseq: int = 0        # varlen fwd: number of packed sequences (0 = dense)
    len_lo: int = 0
    len_hi: int = 0
    qkv_std: float = 1.0
    g_std: float = 1.0
    seed: int = 0
    levels: tuple = ()   # extra skip levels (pi_r, M_r) of a skip schedule
    extra: dict = field(default_factory=dict)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", "fwd", "f32", B=1, H=2, n=256, d=32, k=8, pi=16, M=4,
                          seed=1001),
    "prefill_8k": Workload("prefill_8k", "fwd", "bf16", B=4, H=16, n=8192, d=64, k=64, pi=128,
                           M=16, seed=1002),
    "prefill_128k": Workload("prefill_128k", "fwd", "bf16", B=1, H=32, n=131072, d=128, k=128,
                             pi=256, M=64, qkv_std=0.5, g_std=2.0, seed=1003),
    "decode_32k": Workload("decode_32k", "decode", "bf16", B=128, H=32, n=32768, d=128, k=256,
                           pi=512, M=63, seed=1004),
    "bidir_varlen": Workload("bidir_varlen", "fwd", "bf16", H=16, d=64, k=32, pi=64, M=32,
                             bidir=True, nseq=8, len_lo=4096, len_hi=32768, seed=1005),
    # prefill_8k with a hierarchical (doubling-period) skip schedule: the
    # skips of (128, 16), (256, 16) and (512, 16) unioned -- 32 distinct
    # distances, multiples 1..16, 18..32 step 2 and 36..64 step 4 of 128
    "prefill_8k_sched": Workload("prefill_8k_sched", "fwd", "bf16", B=4, H=16, n=8192, d=64, k=64,
                                 pi=128, M=16, levels=((256, 16), (512, 16)), seed=1006),
}


def varlen_lengths(w: Workload, seed: int | None = None) -> list[int]:
    """Sequence lengths drawn uniformly from the integers [len_lo, len_hi]."""
    gen = torch.Generator().manual_seed(w.seed if seed is None else seed)
    return torch.randint(w.len_lo, w.len_hi + 1, (w.nseq,), generator=gen).tolist()


def _randn(shape, std, dtype, device, gen):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def make_fwd_inputs(w: Workload, device="cpu", seed: int | None = None, lengths=None,
                    layout: str = "bhnd"):
    """Inputs for a prefill call.

    Dense workloads: q, k, v [B, H, n, d] (layout "bhnd") or [B, n, H, d]
    ("bnhd"); g [B, H, n] fp32.  Varlen workloads: q, k, v packed [T, H, d],
    g [T, H] fp32 and cu_seqlens int32 [nseq + 1].
    """
    seed = w.seed if seed is None else seed
    gen = torch.Generator(device=device).manual_seed(seed)
    dt = w.torch_dtype
    if w.nseq:
        lens = list(lengths) if lengths is not None else varlen_lengths(w, seed)
        T = int(sum(lens))
        cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
        shape = (T, w.H, w.d)
        q = _randn(shape, w.qkv_std, dt, device, gen)
        k = _randn(shape, w.qkv_std, dt, device, gen)
        v = _randn(shape, w.qkv_std, dt, device, gen)
        g = _randn((T, w.H), w.g_std, torch.float32, device, gen)
        return dict(q=q, k=k, v=v, g=g, cu_seqlens=cu.to(device), lengths=lens)
    shape = (w.B, w.H, w.n, w.d) if layout == "bhnd" else (w.B, w.n, w.H, w.d)
    q = _randn(shape, w.qkv_std, dt, device, gen)
    k = _randn(shape, w.qkv_std, dt, device, gen)
    v = _randn(shape, w.qkv_std, dt, device, gen)
    g = _randn((w.B, w.H, w.n), w.g_std, torch.float32, device, gen)
    return dict(q=q, k=k, v=v, g=g)


def make_decode_inputs(w: Workload, device="cpu", seed: int | None = None, lens=None,
                       chunk_seqs: int = 8):
    """Inputs for a decode call: q [S, H, d], caches [S, H, L, d], lens int32 [S],
    g [S, H] fp32.  Caches are generated a few sequences at a time so that the
    fp32 staging stays small."""
    seed = w.seed if seed is None else seed
    gen = torch.Generator(device=device).manual_seed(seed)
    dt = w.torch_dtype
    S, H, L, d = w.B, w.H, w.n, w.d
    q = _randn((S, H, d), w.qkv_std, dt, device, gen)
    kc = torch.empty((S, H, L, d), dtype=dt, device=device)
    vc = torch.empty((S, H, L, d), dtype=dt, device=device)
    for s0 in range(0, S, chunk_seqs):
        s1 = min(S, s0 + chunk_seqs)
        kc[s0:s1] = _randn((s1 - s0, H, L, d), w.qkv_std, dt, device, gen)
        vc[s0:s1] = _randn((s1 - s0, H, L, d), w.qkv_std, dt, device, gen)
    g = _randn((S, H), w.g_std, torch.float32, device, gen)
    if lens is None:
        lens = torch.full((S,), L, dtype=torch.int32)
    lens = torch.as_tensor(lens, dtype=torch.int32).to(device)
    return dict(q=q, k_cache=kc, v_cache=vc, lens=lens, g=g)


def bf16_bits(t: torch.Tensor):
    """Raw bf16 bit patterns as a numpy uint16 array (for exact host reads)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
