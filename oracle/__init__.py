"""fp64 CPU oracle for pi-Attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
in ``sparse_long_context_piattn_amd``; neither imports the other.

Two independent formulations live here:

* ``piattn_oracle.c`` (loaded through ctypes): neighbour sets built by
  membership tests, one fp64 softmax per row, OpenMP over rows.  Fast enough
  for every workload when only sampled rows are requested.
* ``dense.py``: the whole [n, n] boolean masks and prior matrix, numpy fp64,
  for tiny n.

Method: pi-Attention, gist.science "pi-Attention: Periodic Sparse
Transformers for Efficient Long-Context Modeling", section 2 "Methodology"
(ring-local window, pi-skip attention, dynamic adaptive fusion as a
log-prior inside one softmax).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "piattn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_piattn.so")
# A prebuilt copy of the same source to load instead (the sanitizer tests
# build one with AddressSanitizer and UBSan and point this at it).
_LIB_OVERRIDE = os.environ.get("PIATTN_ORACLE_LIB")
_lib = None

OR_F64, OR_F32, OR_BF16 = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP).  Returns the .so path."""
    if _LIB_OVERRIDE:
        return _LIB_OVERRIDE
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
             "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_OVERRIDE or _LIB)
        i32, i64, dbl, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.oracle_neighbors.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp]
        lib.oracle_neighbors.restype = i32
        lib.oracle_fwd.argtypes = [i32, vp, i32, i32, vp, vp, vp, i32, vp, i32, i32, i32,
                                   i32, dbl, i64, vp, vp, vp, i32]
        lib.oracle_fwd.restype = None
        lib.oracle_decode.argtypes = [i32, i32, i32, vp, vp, vp, i32, vp, vp, vp, i32, i32,
                                      i32, dbl, vp, vp, i32]
        lib.oracle_decode.restype = None
        lib.oracle_neighbor_table.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp]
        lib.oracle_neighbor_table.restype = i32
        lib.oracle_bwd.argtypes = [i32, vp, i32, i32, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32,
                                   i32, dbl, vp, vp, vp, vp]
        lib.oracle_bwd.restype = None
        lib.oracle_neighbors_levels.argtypes = [i32, i32, i32, vp, vp, i32, i32, vp, vp]
        lib.oracle_neighbors_levels.restype = i32
        lib.oracle_neighbor_table_levels.argtypes = [i32, i32, i32, vp, vp, i32, i32, i32, i32, vp, vp,
                                                     vp]
        lib.oracle_neighbor_table_levels.restype = i32
        lib.oracle_fwd_levels.argtypes = [i32, vp, i32, i32, vp, vp, vp, i32, vp, i32, i32, vp, vp,
                                          i32, dbl, i64, vp, vp, vp, i32]
        lib.oracle_fwd_levels.restype = None
        lib.oracle_decode_levels.argtypes = [i32, i32, i32, vp, vp, vp, i32, vp, vp, vp, i32, i32, vp,
                                             vp, dbl, vp, vp, i32]
        lib.oracle_decode_levels.restype = None
        lib.oracle_bwd_levels.argtypes = [i32, vp, i32, i32, vp, vp, vp, i32, vp, vp, i32, i32, i32,
                                          vp, vp, i32, dbl, vp, vp, vp, vp]
        lib.oracle_bwd_levels.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = i32
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_input(x):
    """Accept float64/float32 arrays, or bf16 given as raw uint16 bits."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float64:
        return x, OR_F64
    if x.dtype == np.float32:
        return x, OR_F32
    if x.dtype == np.uint16:
        return x, OR_BF16
    raise TypeError("oracle inputs must be float64, float32 or uint16 (bf16 bits), got %s" % x.dtype)


def _levels(pi: int, M: int, levels):
    """Level arrays (periods, counts): the base level (pi, M), then the extra
    levels of a skip schedule, each an (pi_r, M_r) pair."""
    lv = [(int(pi), int(M))] + [(int(a), int(b)) for a, b in (levels or ())]
    lpi = np.array([a for a, _ in lv], np.int32)
    lM = np.array([b for _, b in lv], np.int32)
    return len(lv), lpi, lM


def neighbors(n: int, k: int, pi: int, M: int, bidir: bool, i: int, levels=None):
    """Ascending neighbour keys of query i and their kinds (1 local, 2 skip).
    levels: extra (pi_r, M_r) levels of a skip schedule (union of skip sets)."""
    nlev, lpi, lM = _levels(pi, M, levels)
    cap = 2 * k + 1 + 2 * int(lM.sum())
    idx = np.zeros(max(cap, 1), np.int32)
    kind = np.zeros(max(cap, 1), np.int8)
    c = _load().oracle_neighbors_levels(n, k, nlev, _ptr(lpi), _ptr(lM), int(bool(bidir)), i,
                                        _ptr(idx), _ptr(kind))
    return idx[:c].copy(), kind[:c].copy()


def neighbor_table(n: int, k: int, pi: int, M: int, bidir: bool, q_begin: int = 0,
                   q_count: int | None = None, cap: int | None = None, levels=None):
    """[q_count, cap] int32 keys (-1 padded), int8 kinds (0 padded), int32 counts."""
    nlev, lpi, lM = _levels(pi, M, levels)
    if q_count is None:
        q_count = n - q_begin
    if cap is None:
        msum = int(lM.sum())
        cap = (2 * k + 1 + 2 * msum) if bidir else (k + 1 + msum)
    idx = np.empty((q_count, cap), np.int32)
    kind = np.empty((q_count, cap), np.int8)
    cnt = np.empty(q_count, np.int32)
    rc = _load().oracle_neighbor_table_levels(n, k, nlev, _ptr(lpi), _ptr(lM), int(bool(bidir)),
                                              q_begin, q_count, cap, _ptr(idx), _ptr(kind),
                                              _ptr(cnt))
    if rc != 0:
        raise ValueError("a neighbour list does not fit in cap=%d" % cap)
    return idx, kind, cnt


def fwd(q, k, v, g, cu_seqlens, kw: int, pi: int, M: int, bidir: bool, scale: float,
        rows=None, nthreads: int = 0, want_lse: bool = False, levels=None):
    """Prefill over a packed batch.

    q, k, v: [T, H, d] (float64 / float32 / bf16-bits uint16); g: [T, H] gate
    logits; cu_seqlens: [nseq + 1] token offsets.  rows: optional flat row ids
    (token * H + head).  Returns out [rows, d] fp64 (and lse [rows]).
    """
    q, dt = _as_input(q)
    k, dtk = _as_input(k)
    v, dtv = _as_input(v)
    assert dt == dtk == dtv and q.shape == k.shape == v.shape and q.ndim == 3
    T, H, d = q.shape
    g = np.ascontiguousarray(g, dtype=np.float64).reshape(T, H)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    assert cu[0] == 0 and cu[-1] == T
    if rows is None:
        nrows, rows_arr, rp = T * H, None, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, rp = rows_arr.size, _ptr(rows_arr)
    out = np.zeros((nrows, d), np.float64)
    lse = np.zeros(nrows, np.float64)
    nlev, lpi, lM = _levels(pi, M, levels)
    _load().oracle_fwd_levels(len(cu) - 1, _ptr(cu), H, d, _ptr(q), _ptr(k), _ptr(v), dt, _ptr(g),
                              kw, nlev, _ptr(lpi), _ptr(lM), int(bool(bidir)), float(scale), nrows,
                              rp, _ptr(out), _ptr(lse), int(nthreads))
    return (out, lse) if want_lse else out


def decode(q, k_cache, v_cache, lens, g, kw: int, pi: int, M: int, scale: float,
           nthreads: int = 0, want_lse: bool = False, levels=None):
    """One query per (sequence, head) at position lens[s]-1.

    q: [S, H, d]; k_cache, v_cache: [S, H, L, d]; lens: [S]; g: [S, H].
    """
    q, dt = _as_input(q)
    kc, dtk = _as_input(k_cache)
    vc, dtv = _as_input(v_cache)
    assert dt == dtk == dtv and kc.shape == vc.shape and kc.ndim == 4
    S, H, L, d = kc.shape
    assert q.shape == (S, H, d)
    cs = np.array([H * L * d, L * d, d], np.int64)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    assert lens.shape == (S,) and lens.min() >= 1 and lens.max() <= L
    g = np.ascontiguousarray(g, dtype=np.float64).reshape(S, H)
    out = np.zeros((S, H, d), np.float64)
    lse = np.zeros((S, H), np.float64)
    nlev, lpi, lM = _levels(pi, M, levels)
    _load().oracle_decode_levels(S, H, d, _ptr(q), _ptr(kc), _ptr(vc), dt, _ptr(cs), _ptr(lens),
                                 _ptr(g), kw, nlev, _ptr(lpi), _ptr(lM), float(scale), _ptr(out),
                                 _ptr(lse), int(nthreads))
    return (out, lse) if want_lse else out


def bwd(q, k, v, g, dout, cu_seqlens, kw: int, pi: int, M: int, bidir: bool, scale: float,
        levels=None):
    """Gradients of sum(dout * out) for the prefill over a packed batch.

    q, k, v, dout: [T, H, d] (float64 / float32 / bf16-bits uint16); g: [T, H];
    cu_seqlens: [nseq + 1].  Returns dq, dk, dv [T, H, d] and dg [T, H], fp64.
    """
    q, dt = _as_input(q)
    k, dtk = _as_input(k)
    v, dtv = _as_input(v)
    dout, dtd = _as_input(dout)
    assert dt == dtk == dtv and q.shape == k.shape == v.shape == dout.shape and q.ndim == 3
    T, H, d = q.shape
    g = np.ascontiguousarray(g, dtype=np.float64).reshape(T, H)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    assert cu[0] == 0 and cu[-1] == T
    dq = np.zeros((T, H, d), np.float64)
    dk = np.zeros((T, H, d), np.float64)
    dv = np.zeros((T, H, d), np.float64)
    dg = np.zeros((T, H), np.float64)
    nlev, lpi, lM = _levels(pi, M, levels)
    _load().oracle_bwd_levels(len(cu) - 1, _ptr(cu), H, d, _ptr(q), _ptr(k), _ptr(v), dt, _ptr(g),
                              _ptr(dout), dtd, kw, nlev, _ptr(lpi), _ptr(lM), int(bool(bidir)),
                              float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg))
    return dq, dk, dv, dg
