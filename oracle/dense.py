"""Dense-mask formulation of pi-Attention for tiny n (test infrastructure only).

This is the second, independent oracle: instead of enumerating neighbours it
writes the whole [n, n] boolean masks from index offsets and evaluates
softmax(scale * Q K^T + P) V with a prior matrix P that is log(alpha) on the
local mask, log(1 - alpha) on the skip mask and -inf elsewhere, all in numpy
fp64.  Method: gist.science "pi-Attention: Periodic Sparse Transformers for
Efficient Long-Context Modeling", section 2 "Methodology".

The boolean-mask construction follows the sliding-window glossary page
(ultralytics.com "Sliding Window Attention", section "Wie das Fenster mit der
Tiefe wächst"): an offset matrix pos[:, None] - pos[None, :] and comparisons on
it.  With no skips and a causal window of w = k + 1 keys it is exactly that
page's mask.
"""
from __future__ import annotations

import numpy as np


def masks(n: int, k: int, pi: int, M: int, bidir: bool, levels=None):
    """(local, skip) boolean [n, n] masks; row = query i, column = key j.
    levels: extra (pi_r, M_r) levels of a skip schedule; the skip mask is the
    elementwise OR of each level's mask."""
    pos = np.arange(n)
    off = pos[:, None] - pos[None, :]          # i - j
    if bidir:
        local = np.abs(off) <= k
        cand = off != 0
    else:
        local = (off >= 0) & (off <= k)
        cand = off > 0
    dist = np.abs(off)
    skip = np.zeros((n, n), bool)
    for p_r, m_r in [(pi, M)] + list(levels or ()):
        skip |= cand & (dist % p_r == 0) & (dist <= m_r * p_r) & ~local
    return local, skip


def attention(q, k, v, g, kw: int, pi: int, M: int, bidir: bool, scale: float,
              want_lse: bool = False, levels=None):
    """One (sequence, head): q, k, v [n, d] float64, g [n] gate logits."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    n = q.shape[0]
    local, skip = masks(n, kw, pi, M, bidir, levels)
    with np.errstate(divide="ignore"):
        alpha = 1.0 / (1.0 + np.exp(-g))
        log_a = np.log(alpha)
        log_1ma = np.log1p(-alpha)
    # stable forms for the tails (|g| large makes alpha round to 0 or 1)
    big = g > 30
    log_1ma = np.where(big, -g - np.log1p(np.exp(-np.abs(g))), log_1ma)
    small = g < -30
    log_a = np.where(small, g - np.log1p(np.exp(-np.abs(g))), log_a)
    has_skip = skip.any(axis=1)
    prior = np.full((n, n), -np.inf)
    prior = np.where(local, np.where(has_skip, log_a, 0.0)[:, None], prior)
    prior = np.where(skip, log_1ma[:, None], prior)
    logits = scale * (q @ k.T) + prior
    mx = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - mx)
    z = w.sum(axis=1, keepdims=True)
    out = (w @ v) / z
    if want_lse:
        return out, (mx + np.log(z))[:, 0]
    return out
