"""GPU parity of the gate logits and the output projection (piattn_gate_logits,
piattn_out_proj) against the fp64 oracle in oracle/proj.py.

Tolerance, elementwise, from the arithmetic: the products of bf16 (or fp32)
inputs are summed in fp32, so |err| <= c_acc * sum_k |a_k b_k| with
c_acc = 2e-5 (a few ulps of fp32 times the sum's condition, generous for
K up to 4096); a bf16 output adds its round-to-nearest-even error,
2^-9 |ref|, taken as 4e-3 |ref|.
"""
import numpy as np
import pytest
import torch

import sparse_long_context_piattn_amd as pa

from helpers import host_array, max_err
from oracle import proj as oproj

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _rand(shape, seed, dtype, std=1.0):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=gen, device=DEV) * std).to(dtype)


def _check(got, ref, absref, bf16_out, tag):
    got = got.detach().float().cpu().double().numpy()
    tol = 2e-5 * absref + 1e-6 + (4e-3 * np.abs(ref) if bf16_out else 0.0)
    err = np.abs(got - ref)
    max_err(torch.from_numpy(got), ref, tag)
    assert np.all(err <= tol), (tag, float(err.max()), float((err / tol).max()))


GATE = [
    # name, dtype, B, n, Dm, H, bias
    ("bf16_1024x16", torch.bfloat16, 2, 300, 1024, 16, True),
    ("bf16_ragged_h20", torch.bfloat16, 1, 77, 96, 20, False),
    ("bf16_4096x32", torch.bfloat16, 1, 130, 4096, 32, True),
    ("bf16_h1", torch.bfloat16, 3, 5, 64, 1, True),
    ("f32_256x8", torch.float32, 2, 50, 256, 8, True),
    ("f32_odd", torch.float32, 1, 33, 37, 5, False),
]


@pytest.mark.parametrize("case", GATE, ids=[c[0] for c in GATE])
def test_gate_logits_match_oracle(case):
    name, dt, B, n, Dm, H, with_bias = case
    x = _rand((B, n, Dm), 1, dt)
    w = _rand((H, Dm), 2, dt, Dm ** -0.5)
    bias = _rand((H,), 3, torch.float32) if with_bias else None
    print("gate %s" % name, flush=True)
    g = pa.gate_logits(x, w, bias)
    torch.cuda.synchronize()
    ref = oproj.gate_logits(host_array(x), host_array(w), None if bias is None else bias.cpu().numpy())
    absref = oproj.gate_logits(np.abs(oproj._f64(host_array(x))), np.abs(oproj._f64(host_array(w))))
    _check(g, ref, absref, False, "gate " + name)


@pytest.mark.parametrize("T,Dm,H", [(40_000, 96, 20), (70_001, 128, 16), (66_000, 160, 32)])
def test_gate_logits_long_inputs(T, Dm, H):
    """Token counts that make the kernel take two (T >= 32768) or four
    (T >= 65536) blocks of 16 tokens per wave, with one and two head blocks
    and a ragged tail."""
    x = _rand((1, T, Dm), 20, torch.bfloat16)
    w = _rand((H, Dm), 21, torch.bfloat16, Dm ** -0.5)
    bias = _rand((H,), 22, torch.float32)
    print("gate long T=%d Dm=%d H=%d" % (T, Dm, H), flush=True)
    g = pa.gate_logits(x, w, bias)
    torch.cuda.synchronize()
    ref = oproj.gate_logits(host_array(x), host_array(w), bias.cpu().numpy())
    absref = oproj.gate_logits(np.abs(oproj._f64(host_array(x))), np.abs(oproj._f64(host_array(w))))
    _check(g, ref, absref, False, "gate long %d" % T)


def test_gate_logits_packed_and_strided():
    """Packed [T, Dm] input gives [T, H] logits (the varlen gate layout); a
    strided x view ([B, n, Dm] out of a wider buffer) and a preallocated
    strided output are honoured."""
    x = _rand((500, 128), 4, torch.bfloat16)
    w = _rand((16, 128), 5, torch.bfloat16, 0.1)
    g = pa.gate_logits(x, w)
    wide = _rand((2, 60, 256), 6, torch.bfloat16)
    xv = wide[:, :, 64:192]
    out = torch.zeros((2, 16, 60 * 2), device=DEV)[:, :, ::2]
    pa.gate_logits(xv, w, out=out)
    torch.cuda.synchronize()
    ref = oproj.gate_logits(host_array(x)[None], host_array(w))[0].T
    absref = oproj.gate_logits(np.abs(oproj._f64(host_array(x)))[None], np.abs(oproj._f64(host_array(w))))[0].T
    _check(g, ref, absref, False, "gate packed")
    ref2 = oproj.gate_logits(host_array(xv.contiguous()), host_array(w))
    absref2 = oproj.gate_logits(np.abs(oproj._f64(host_array(xv.contiguous()))), np.abs(oproj._f64(host_array(w))))
    _check(out, ref2, absref2, False, "gate strided")


PROJ = [
    # name, dtype, B, H, n, d, Dout, bias
    ("bf16_h16_d64", torch.bfloat16, 2, 16, 300, 64, 1024, True),
    ("bf16_ragged", torch.bfloat16, 1, 3, 77, 32, 200, False),
    ("bf16_h32_d128", torch.bfloat16, 1, 32, 130, 128, 4096, True),
    ("bf16_plain_d8", torch.bfloat16, 2, 2, 40, 8, 24, True),
    ("f32_h4_d32", torch.float32, 2, 4, 50, 32, 96, True),
]


@pytest.mark.parametrize("case", PROJ, ids=[c[0] for c in PROJ])
def test_out_proj_matches_oracle(case):
    name, dt, B, H, n, d, Dout, with_bias = case
    # o as the attention would leave it in a token-major buffer: [B, n, H, d]
    # storage viewed as [B, H, n, d]
    o = _rand((B, n, H, d), 7, dt).permute(0, 2, 1, 3)
    w = _rand((Dout, H * d), 8, dt, (H * d) ** -0.5)
    bias = _rand((Dout,), 9, torch.float32) if with_bias else None
    print("out_proj %s" % name, flush=True)
    y = pa.out_proj(o, w, bias)
    torch.cuda.synchronize()
    oh = host_array(o.contiguous())
    ref = oproj.out_proj(oh, host_array(w), None if bias is None else bias.cpu().numpy())
    absref = oproj.out_proj(np.abs(oproj._f64(oh)), np.abs(oproj._f64(host_array(w))))
    _check(y, ref, absref, dt == torch.bfloat16, "out_proj " + name)


def test_out_proj_320_row_tiles():
    """At least 2048 tiles of 320 rows (here 129 x 16): the dispatch takes the
    80-row waves; a ragged last row tile, checked on sampled rows (the first
    two tiles, the last 700 rows, 2000 more at random)."""
    B, H, n, d, Dout = 1, 2, 40_960 + 77, 32, 4096
    o = _rand((B, n, H, d), 30, torch.bfloat16).permute(0, 2, 1, 3)
    w = _rand((Dout, H * d), 31, torch.bfloat16, (H * d) ** -0.5)
    bias = _rand((Dout,), 32, torch.float32)
    print("out_proj 320-row tiles", flush=True)
    y = pa.out_proj(o, w, bias)
    torch.cuda.synchronize()
    rng = np.random.default_rng(33)
    rows = np.unique(np.concatenate([np.arange(640), np.arange(n - 700, n), rng.integers(0, n, 2000)]))
    oh = host_array(o.contiguous())[:, :, rows, :]
    ref = oproj.out_proj(oh, host_array(w), bias.cpu().numpy())
    absref = oproj.out_proj(np.abs(oproj._f64(oh)), np.abs(oproj._f64(host_array(w))))
    got = y[:, torch.from_numpy(rows).to(DEV), :]
    _check(got, ref, absref, True, "out_proj 320-row tiles")


def test_out_proj_packed_and_padded_weights():
    """Packed [T, H, d] attention output (varlen) gives [T, Dout]; a weight
    matrix with a row stride above H*d is read through ldw."""
    T, H, d, Dout = 333, 4, 64, 160
    o = _rand((T, H, d), 10, torch.bfloat16)
    wbig = _rand((Dout, H * d + 64), 11, torch.bfloat16, 0.06)
    w = wbig[:, :H * d]
    y = pa.out_proj(o, w)
    torch.cuda.synchronize()
    oh = host_array(o.permute(1, 0, 2).contiguous())[None]
    ref = oproj.out_proj(oh, host_array(w.contiguous()))[0]
    absref = oproj.out_proj(np.abs(oproj._f64(oh)), np.abs(oproj._f64(host_array(w.contiguous()))))[0]
    _check(y, ref, absref, True, "out_proj packed")


def test_layer_chain_runs_on_the_prefill_shape():
    """gate -> attention -> output projection at the prefill_8k shape (B4 H16
    n8192 d64, Dm = H d = 1024): the chain runs without copies between the
    stages and the projection of one sequence matches the oracle applied to
    the GPU attention output of that sequence."""
    B, H, n, d = 4, 16, 8192, 64
    Dm = H * d
    x = _rand((B, n, Dm), 12, torch.bfloat16)
    q, k, v = (_rand((B, H, n, d), 13 + i, torch.bfloat16) for i in range(3))
    wg = _rand((H, Dm), 16, torch.bfloat16, Dm ** -0.5)
    wo = _rand((Dm, Dm), 17, torch.bfloat16, Dm ** -0.5)
    g = pa.gate_logits(x, wg)
    o = pa.fwd(q, k, v, g, window_k=64, period_pi=128, num_skips=16)
    y = pa.out_proj(o, wo)
    torch.cuda.synchronize()
    assert g.shape == (B, H, n) and y.shape == (B, n, Dm)
    b = 3
    ob = host_array(o[b:b + 1].contiguous())
    ref = oproj.out_proj(ob, host_array(wo))
    absref = oproj.out_proj(np.abs(oproj._f64(ob)), np.abs(oproj._f64(host_array(wo))))
    _check(y[b:b + 1], ref, absref, True, "layer out_proj")
