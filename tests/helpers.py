"""Test-side glue: run the oracle on the same seeded inputs the GPU sees.

Layout conversion only (torch views to the oracle's packed [T, H, d] arrays);
no attention arithmetic lives here.
"""
import json
import os

import numpy as np
import torch

import oracle
from sparse_long_context_piattn_amd import workloads as wl

BF16_TOL = 2e-2
F32_TOL = 1e-5
# Row log-normaliser.  On every path it is log(sum exp(logit)) computed in
# fp32 from exact inputs (bf16 values are exact in fp32): scores accumulated
# in fp32 (MFMA or VALU) over d <= 128 exact products, the exponentials
# summed in fp32 before any bf16 rounding of the weights, one log.  For the
# magnitudes of these workloads that stays well under 1e-5 in natural-log
# units, the same bound on both dtypes.
LSE_TOL_BF16 = 1e-5
LSE_TOL_F32 = 1e-5


def host_array(t: torch.Tensor):
    """Exact host copy: float32 stays float32, bf16 becomes its raw bits."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def packed(t: torch.Tensor):
    """[B, H, n, d] -> [B*n, H, d] host array (exact)."""
    B, H, n, d = t.shape
    return host_array(t.permute(0, 2, 1, 3).reshape(B * n, H, d))


def oracle_dense_fwd(x, w, rows=None, want_lse=False, bidir=None):
    """Oracle on dense [B, H, n, d] inputs; returns [B, H, n, d] (rows=None) or
    [len(rows), d] for flat row ids (b*n + i)*H + h."""
    q, k, v, g = x["q"], x["k"], x["v"], x["g"]
    B, H, n, d = q.shape
    gg = g.detach().cpu().permute(0, 2, 1).reshape(B * n, H).double().numpy()
    res = oracle.fwd(packed(q), packed(k), packed(v), gg, np.arange(B + 1) * n, w.k, w.pi, w.M,
                     w.bidir if bidir is None else bidir, w.scale, rows=rows,
                     want_lse=want_lse, levels=w.levels)
    if rows is not None:
        return res
    if want_lse:
        out, lse = res
        return (out.reshape(B, n, H, d).transpose(0, 2, 1, 3),
                lse.reshape(B, n, H).transpose(0, 2, 1))
    return res.reshape(B, n, H, d).transpose(0, 2, 1, 3)


def oracle_varlen_fwd(x, w, rows=None, want_lse=False):
    q, k, v, g, cu = x["q"], x["k"], x["v"], x["g"], x["cu_seqlens"]
    return oracle.fwd(host_array(q), host_array(k), host_array(v),
                      g.detach().cpu().double().numpy(), cu.cpu().numpy().astype(np.int64),
                      w.k, w.pi, w.M, w.bidir, w.scale, rows=rows, want_lse=want_lse)


def max_err(got: torch.Tensor, ref, tag: str | None = None) -> float:
    g = got.detach().float().cpu().double().numpy()
    err = float(np.abs(g - np.asarray(ref)).max()) if g.size else 0.0
    log_path = os.environ.get("PIATTN_ERRLOG")
    if log_path and tag:
        with open(log_path, "a") as f:
            f.write(json.dumps({"case": tag, "max_abs_err": err}) + "\n")
    return err


def lse_tol_for(w) -> float:
    return LSE_TOL_F32 if w.dtype == "f32" else LSE_TOL_BF16


def tol_for(w) -> float:
    return F32_TOL if w.dtype == "f32" else BF16_TOL
