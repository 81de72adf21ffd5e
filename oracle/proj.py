"""fp64 oracle of the linear maps around pi-Attention (test infrastructure
only; shares no code with the HIP library).

The pages give the gate as a learnable shallow MLP of the input (gist.science
"pi-Attention: Periodic Sparse Transformers ...", section 2 "Methodology",
item "Dynamic Adaptive Fusion") and end with a fusion-and-projection stage
(section 2 "Execution & Scheduling").  The plainest form is taken, and
computed here straight from its definition with numpy fp64 products:

  gate logits   g[b, h, i] = sum_c x[b, i, c] w[h, c] + bias[h]
  output proj.  y[b, i, r] = sum_{h, c} o[b, h, i, c] w[r, h d + c] + bias[r]

Inputs may be float64/float32 arrays or bf16 raw bits (uint16), read exactly.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def gate_logits(x, w, bias=None):
    """x [B, n, Dm], w [H, Dm], bias [H] -> g [B, H, n] fp64."""
    x, w = _f64(x), _f64(w)
    g = np.matmul(x, w.T)                       # [B, n, H]
    if bias is not None:
        g = g + _f64(bias)
    return np.ascontiguousarray(g.transpose(0, 2, 1))


def out_proj(o, w, bias=None):
    """o [B, H, n, d], w [Dout, H*d], bias [Dout] -> y [B, n, Dout] fp64."""
    o, w = _f64(o), _f64(w)
    B, H, n, d = o.shape
    cat = o.transpose(0, 2, 1, 3).reshape(B, n, H * d)   # heads concatenated per token
    y = np.matmul(cat, w.T)
    if bias is not None:
        y = y + _f64(bias)
    return y
