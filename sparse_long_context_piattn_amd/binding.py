"""Thin ctypes binding over libpiattn (include/piattn.h).

Argument marshalling only: shapes and dtypes are checked, strides and data
pointers are read from torch tensors, and the call is enqueued on torch's
current HIP stream.  Every step of the computation runs in the HIP kernels of
libpiattn.so; if that library is missing the calls raise -- there is no
fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpiattn.so")

PIATTN_F32, PIATTN_BF16 = 0, 1
STATUS = {0: "PIATTN_OK", 1: "PIATTN_EINVAL", 2: "PIATTN_EUNSUPPORTED", 3: "PIATTN_EWORKSPACE",
          4: "PIATTN_EHIP"}

EXPORTS = ["piattn_fwd", "piattn_fwd_workspace_bytes", "piattn_bwd", "piattn_bwd_workspace_bytes",
           "piattn_gate_logits", "piattn_out_proj",
           "piattn_decode", "piattn_decode_workspace_bytes",
           "piattn_decode_auto_splits", "piattn_rolling_slots", "piattn_cache_append",
           "piattn_decode_rolling", "piattn_neighbors", "piattn_neighbors_cap",
           "piattn_last_error", "piattn_version", "piattn_debug_force_kernels", "piattn_fwd_noalloc"]

NOALLOC_SCRATCH_BYTES = 64 << 20     # PIATTN_NOALLOC_SCRATCH_BYTES


class PiattnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s: %s" % (STATUS.get(code, str(code)), msg))
        self.code = code


MAX_LEVELS = 7


class Pattern(ctypes.Structure):
    """piattn_pattern: window half-width k, period pi, skips M, direction,
    scale, and the extra levels (pi_r, M_r) of a skip schedule."""
    _fields_ = [("window_k", ctypes.c_int32), ("period_pi", ctypes.c_int32),
                ("num_skips_M", ctypes.c_int32), ("bidirectional", ctypes.c_int32),
                ("scale", ctypes.c_float), ("num_levels", ctypes.c_int32),
                ("level_pi", ctypes.c_int32 * MAX_LEVELS), ("level_M", ctypes.c_int32 * MAX_LEVELS)]


Strides = ctypes.c_int64 * 15
Strides4 = ctypes.c_int64 * 12
_lib = None


def lib():
    """Load libpiattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libpiattn.so is not built; run "
                               "`python -m sparse_long_context_piattn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        pat = ctypes.POINTER(Pattern)
        L.piattn_fwd.argtypes = [ctypes.c_int, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                 ctypes.POINTER(Strides), vp, pat, vp, sz, vp]
        L.piattn_fwd.restype = ctypes.c_int
        L.piattn_fwd_noalloc.argtypes = [ctypes.c_int, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                         ctypes.POINTER(Strides), vp, pat, vp]
        L.piattn_fwd_noalloc.restype = ctypes.c_int
        L.piattn_fwd_workspace_bytes.argtypes = [ctypes.c_int, i32, i32, i32, i32, pat]
        L.piattn_fwd_workspace_bytes.restype = sz
        L.piattn_bwd.argtypes = [ctypes.c_int, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                 ctypes.POINTER(Strides), vp, pat, vp, sz, vp]
        L.piattn_bwd.restype = ctypes.c_int
        L.piattn_bwd_workspace_bytes.argtypes = [i32, i32, i32]
        L.piattn_bwd_workspace_bytes.restype = sz
        L.piattn_decode.argtypes = [ctypes.c_int, i32, i32, i32, vp, vp, vp, vp, i32, vp, vp,
                                    ctypes.POINTER(Strides), pat, i32, vp, sz, vp]
        L.piattn_decode.restype = ctypes.c_int
        L.piattn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, pat]
        L.piattn_decode_workspace_bytes.restype = sz
        L.piattn_decode_auto_splits.argtypes = [i32, i32, i32, pat]
        L.piattn_decode_auto_splits.restype = i32
        L.piattn_decode_rolling.argtypes = L.piattn_decode.argtypes
        L.piattn_decode_rolling.restype = ctypes.c_int
        L.piattn_rolling_slots.argtypes = [pat]
        L.piattn_rolling_slots.restype = i32
        L.piattn_cache_append.argtypes = [ctypes.c_int, i32, i32, i32, vp, vp, vp, vp, vp, i32,
                                          ctypes.POINTER(Strides4), vp]
        L.piattn_cache_append.restype = ctypes.c_int
        L.piattn_neighbors.argtypes = [i32, pat, i32, i32, i32, vp, vp, vp, vp]
        L.piattn_neighbors.restype = ctypes.c_int
        L.piattn_gate_logits.argtypes = [ctypes.c_int, i32, i32, i32, i32, vp, ctypes.POINTER(ctypes.c_int64 * 2),
                                         vp, vp, vp, ctypes.POINTER(ctypes.c_int64 * 3), vp]
        L.piattn_gate_logits.restype = ctypes.c_int
        L.piattn_out_proj.argtypes = [ctypes.c_int, i32, i32, i32, i32, vp, ctypes.POINTER(ctypes.c_int64 * 3), i32,
                                      vp, ctypes.c_int64, vp, vp, ctypes.POINTER(ctypes.c_int64 * 2), vp]
        L.piattn_out_proj.restype = ctypes.c_int
        L.piattn_neighbors_cap.argtypes = [pat]
        L.piattn_neighbors_cap.restype = i32
        L.piattn_last_error.argtypes = []
        L.piattn_last_error.restype = ctypes.c_char_p
        L.piattn_version.argtypes = []
        L.piattn_version.restype = ctypes.c_char_p
        L.piattn_debug_force_kernels.argtypes = [i32, i32]
        L.piattn_debug_force_kernels.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise PiattnError(rc, lib().piattn_last_error().decode())


def make_pattern(k: int, pi: int, M: int, bidir: bool = False, scale: float = 0.0, levels=()) -> Pattern:
    """levels: extra (pi_r, M_r) skip levels; the skip set is the union over
    (pi, M) and these (a skip schedule)."""
    levels = [(int(a), int(b)) for a, b in (levels or ())]
    if len(levels) > MAX_LEVELS:
        raise ValueError("at most %d extra levels" % MAX_LEVELS)
    p = Pattern(int(k), int(pi), int(M), int(bool(bidir)), float(scale), len(levels))
    for r, (a, b) in enumerate(levels):
        p.level_pi[r] = a
        p.level_M[r] = b
    return p


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PIATTN_F32
    if t.dtype == torch.bfloat16:
        return PIATTN_BF16
    raise TypeError("q/k/v must be float32 or bfloat16, got %s" % t.dtype)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _prefill_geometry(q, k, v, g, out, cu_seqlens, max_seqlen):
    """(B, H, n, d, strides, cu pointer) of a prefill call, or None when the
    varlen batch is empty.  Dense: q, k, v, out [B, H, n, d], g [B, H, n];
    varlen: [T, H, d] and g [T, H] with cu_seqlens int32 [B + 1]."""
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError("dense mode expects q [B, H, n, d]")
        B, H, n, d = q.shape
        if k.shape != q.shape or v.shape != q.shape or out.shape != q.shape:
            raise ValueError("q, k, v, out shapes differ")
        if tuple(g.shape) != (B, H, n):
            raise ValueError("g must be [B, H, n]")
        st4 = [tuple(t.stride()[:3]) for t in (q, k, v, out)]
        gst = tuple(g.stride())
        cu_ptr = None
    else:
        if q.dim() != 3:
            raise ValueError("varlen mode expects q [T, H, d]")
        T, H, d = q.shape
        if k.shape != q.shape or v.shape != q.shape or out.shape != q.shape:
            raise ValueError("q, k, v, out shapes differ")
        if tuple(g.shape) != (T, H):
            raise ValueError("g must be [T, H]")
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor")
        B = cu_seqlens.numel() - 1
        if max_seqlen is None:
            cu_h = cu_seqlens.cpu()
            max_seqlen = int((cu_h[1:] - cu_h[:-1]).max()) if B > 0 else 0
        n = int(max_seqlen)
        if n == 0:
            return None
        st4 = [(0, t.stride(1), t.stride(0)) for t in (q, k, v, out)]
        gst = (0, g.stride(1), g.stride(0))
        cu_ptr = _ptr(cu_seqlens)
    for t in (q, k, v, out):
        if t.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous")
    return B, H, n, d, Strides(*[x for s in st4 for x in s], *gst), cu_ptr


def fwd_workspace_bytes(dtype_code: int, B: int, H: int, n: int, d: int, pattern: Pattern) -> int:
    return int(lib().piattn_fwd_workspace_bytes(dtype_code, B, H, n, d, ctypes.byref(pattern)))


def fwd(q, k, v, g, *, window_k: int, period_pi: int, num_skips: int, bidirectional=False,
        scale: float = 0.0, cu_seqlens=None, max_seqlen: int | None = None, out=None,
        lse=None, workspace=None, levels=()):
    """pi-Attention prefill.

    Dense: q, k, v [B, H, n, d] (any strides, last dim contiguous), g [B, H, n].
    Varlen: q, k, v [T, H, d], g [T, H], cu_seqlens int32 [B + 1] on the GPU.
    Returns out (same shape and dtype as q); lse, if given, is written with
    the natural-log normaliser of each row (shape of g, fp32).  workspace, if
    given, is a uint8 device tensor of at least fwd_workspace_bytes(...)
    bytes; otherwise one is taken from torch's allocator on the current
    stream for the call.
    """
    code = _dtype_code(q)
    _need_cuda(q, k, v, g, out, lse, cu_seqlens)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    if g.dtype != torch.float32:
        raise TypeError("gate logits must be float32")
    if out is None:
        out = torch.empty_like(q)
    if q.numel() == 0 or (cu_seqlens is not None and cu_seqlens.numel() <= 1):
        return out  # nothing to attend
    geo = _prefill_geometry(q, k, v, g, out, cu_seqlens, max_seqlen)
    if geo is None:
        return out
    B, H, n, d, strides, cu_ptr = geo
    if lse is not None and (lse.shape != g.shape or lse.stride() != g.stride()):
        raise ValueError("lse must have g's shape and strides")
    pat = make_pattern(window_k, period_pi, num_skips, bidirectional, scale, levels)
    need = fwd_workspace_bytes(code, B, H, n, d, pat)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _need_cuda(workspace)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().piattn_fwd(code, B, H, n, d, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out),
                          _ptr(lse), ctypes.byref(strides), cu_ptr, ctypes.byref(pat),
                          _ptr(workspace), wbytes, ctypes.c_void_p(_stream(q.device)))
    _check(rc)
    return out


def fwd_noalloc(q, k, v, g, *, out, window_k: int, period_pi: int, num_skips: int, bidirectional=False,
                scale: float = 0.0, cu_seqlens=None, max_seqlen: int | None = None, lse=None, levels=()):
    """fwd through piattn_fwd_noalloc: the library-held scratch array stands in
    for the workspace, so the C call allocates nothing; the caller passes
    out (and lse, if wanted).  Arguments as for fwd."""
    code = _dtype_code(q)
    _need_cuda(q, k, v, g, out, lse, cu_seqlens)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    if g.dtype != torch.float32:
        raise TypeError("gate logits must be float32")
    if q.numel() == 0 or (cu_seqlens is not None and cu_seqlens.numel() <= 1):
        return out
    geo = _prefill_geometry(q, k, v, g, out, cu_seqlens, max_seqlen)
    if geo is None:
        return out
    B, H, n, d, strides, cu_ptr = geo
    if lse is not None and (lse.shape != g.shape or lse.stride() != g.stride()):
        raise ValueError("lse must have g's shape and strides")
    pat = make_pattern(window_k, period_pi, num_skips, bidirectional, scale, levels)
    rc = lib().piattn_fwd_noalloc(code, B, H, n, d, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out), _ptr(lse),
                                  ctypes.byref(strides), cu_ptr, ctypes.byref(pat),
                                  ctypes.c_void_p(_stream(q.device)))
    _check(rc)
    return out


def bwd(q, k, v, g, out, dout, *, window_k: int, period_pi: int, num_skips: int, bidirectional=False,
        scale: float = 0.0, cu_seqlens=None, max_seqlen: int | None = None, lse=None, workspace=None,
        levels=()):
    """Backward of fwd: the gradients (dq, dk, dv, dg) of a loss whose gradient
    with respect to fwd's output `out` is `dout`.  dq, dk, dv have the shapes
    and strides of q, k, v (allocated like them); dg is fp32 like g.  dout
    must have out's strides.  lse: the log-sum-exp fwd wrote (fp32, g's shape
    and strides), or None; bf16 with d 64 / 128 runs on the MFMA kernels when
    it is given, everything else on the gather kernels (which recompute it)."""
    code = _dtype_code(q)
    _need_cuda(q, k, v, g, out, dout, cu_seqlens, workspace, lse)
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != g.shape or lse.stride() != g.stride()):
        raise ValueError("lse must be float32 with g's shape and strides")
    for t in (k, v, out, dout):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, out, dout must share a dtype")
    if g.dtype != torch.float32:
        raise TypeError("gate logits must be float32")
    if dout.shape != out.shape or dout.stride() != out.stride():
        raise ValueError("dout must have out's shape and strides")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty_like(g)
    if q.numel() == 0:
        return dq, dk, dv, dg
    if not (dq.stride() == q.stride() and dk.stride() == k.stride() and dv.stride() == v.stride()
            and dg.stride() == g.stride()):
        raise ValueError("q, k, v and g must be dense (gradients take their strides)")
    geo = _prefill_geometry(q, k, v, g, out, cu_seqlens, max_seqlen)
    if geo is None:
        return dq, dk, dv, dg
    B, H, n, d, strides, cu_ptr = geo
    pat = make_pattern(window_k, period_pi, num_skips, bidirectional, scale, levels)
    need = int(lib().piattn_bwd_workspace_bytes(B, H, n))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    rc = lib().piattn_bwd(code, B, H, n, d, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out), _ptr(lse), _ptr(dout),
                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), ctypes.byref(strides), cu_ptr,
                          ctypes.byref(pat), _ptr(workspace), wbytes, ctypes.c_void_p(_stream(q.device)))
    _check(rc)
    return dq, dk, dv, dg


def gate_logits(x, w, bias=None, *, out=None):
    """Gate logits g = x w^T + bias of a linear gate per head.

    x [B, n, Dm] (last dim contiguous) or packed [T, Dm]; w [H, Dm]
    contiguous; bias [H] fp32 or None.  Returns g fp32 [B, H, n] (packed:
    [T, H]), the prefill's gate layout, or writes into out of that shape."""
    code = _dtype_code(x)
    _need_cuda(x, w, bias, out)
    if w.dtype != x.dtype or w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous [H, Dm] tensor of x's dtype")
    if bias is not None and (bias.dtype != torch.float32 or bias.shape != (w.shape[0],)):
        raise ValueError("bias must be float32 [H]")
    packed_in = x.dim() == 2
    x3 = x.unsqueeze(0) if packed_in else x
    if x3.dim() != 3 or x3.stride(-1) != 1:
        raise ValueError("x must be [B, n, Dm] or [T, Dm] with a contiguous last dim")
    B, n, Dm = x3.shape
    H = w.shape[0]
    if w.shape[1] != Dm:
        raise ValueError("w is [H, %d], x has Dm=%d" % (w.shape[1], Dm))
    if out is None:
        out = torch.empty((n, H) if packed_in else (B, H, n), dtype=torch.float32, device=x.device)
    gs = (0, out.stride(1), out.stride(0)) if packed_in else tuple(out.stride())
    xs = (ctypes.c_int64 * 2)(x3.stride(0), x3.stride(1))
    gst = (ctypes.c_int64 * 3)(*gs)
    rc = lib().piattn_gate_logits(code, B, n, Dm, H, _ptr(x3), ctypes.byref(xs), _ptr(w), _ptr(bias), _ptr(out),
                                  ctypes.byref(gst), ctypes.c_void_p(_stream(x.device)))
    _check(rc)
    return out


def out_proj(o, w, bias=None, *, out=None):
    """Output projection y = concat_h(o) w^T + bias, read from the attention's
    output layout.  o [B, H, n, d] (any strides, last dim contiguous) or
    packed [T, H, d]; w [Dout, H*d] (last dim contiguous); bias [Dout] fp32
    or None.  Returns y [B, n, Dout] (packed: [T, Dout]) of o's dtype."""
    code = _dtype_code(o)
    _need_cuda(o, w, bias, out)
    if w.dtype != o.dtype or w.dim() != 2 or w.stride(-1) != 1:
        raise ValueError("w must be a [Dout, H*d] tensor of o's dtype with a contiguous last dim")
    packed_in = o.dim() == 3
    if packed_in:
        T, H, d = o.shape
        B, n = 1, T
        ost = (0, o.stride(1), o.stride(0))
    else:
        B, H, n, d = o.shape
        ost = tuple(o.stride()[:3])
    if o.stride(-1) != 1:
        raise ValueError("the head dimension of o must be contiguous")
    Dout = w.shape[0]
    if w.shape[1] != H * d:
        raise ValueError("w is [Dout, %d], o has H*d=%d" % (w.shape[1], H * d))
    if bias is not None and (bias.dtype != torch.float32 or bias.shape != (Dout,)):
        raise ValueError("bias must be float32 [Dout]")
    if out is None:
        out = torch.empty((n, Dout) if packed_in else (B, n, Dout), dtype=o.dtype, device=o.device)
    if out.stride(-1) != 1:
        raise ValueError("out must have a contiguous last dim")
    ys = (0, out.stride(0)) if packed_in else (out.stride(0), out.stride(1))
    os_ = (ctypes.c_int64 * 3)(*ost)
    yst = (ctypes.c_int64 * 2)(*ys)
    rc = lib().piattn_out_proj(code, B, H, n, d, _ptr(o), ctypes.byref(os_), Dout, _ptr(w), w.stride(0),
                               _ptr(bias), _ptr(out), ctypes.byref(yst), ctypes.c_void_p(_stream(o.device)))
    _check(rc)
    return out


def decode_workspace_bytes(S, H, d, num_splits, pattern: Pattern) -> int:
    return int(lib().piattn_decode_workspace_bytes(S, H, d, num_splits, ctypes.byref(pattern)))


def rolling_slots(window_k: int, period_pi: int, num_skips: int, levels=()) -> int:
    """Rows of a rolling decode cache for this pattern: max(k, longest skip) + 1."""
    pat = make_pattern(window_k, period_pi, num_skips, levels=levels)
    return int(lib().piattn_rolling_slots(ctypes.byref(pat)))


def cache_append(k_new, v_new, k_cache, v_cache, positions):
    """Write k_new, v_new [S, H, d] to row positions[s] mod W of the rolling
    caches [S, H, W, d] (positions: int32 [S] on the GPU; negative = skip)."""
    code = _dtype_code(k_new)
    _need_cuda(k_new, v_new, k_cache, v_cache, positions)
    if k_new.dim() != 3 or v_new.shape != k_new.shape or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expect k_new, v_new [S, H, d] and caches [S, H, W, d]")
    S, H, d = k_new.shape
    if tuple(k_cache.shape[:2]) != (S, H) or k_cache.shape[3] != d:
        raise ValueError("cache shape does not match the new rows")
    if positions.dtype != torch.int32 or tuple(positions.shape) != (S,):
        raise ValueError("positions must be int32 [S]")
    for t in (k_new, v_new, k_cache, v_cache):
        if t.dtype != k_new.dtype or t.stride(-1) != 1:
            raise ValueError("same dtype and a contiguous head dimension expected")
    st = [(k_new.stride(0), k_new.stride(1), 0), (v_new.stride(0), v_new.stride(1), 0),
          tuple(k_cache.stride()[:3]), tuple(v_cache.stride()[:3])]
    strides = Strides4(*[x for s in st for x in s])
    rc = lib().piattn_cache_append(code, S, H, d, _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(positions), k_cache.shape[2], ctypes.byref(strides),
                                   ctypes.c_void_p(_stream(k_new.device)))
    _check(rc)


def decode(q, k_cache, v_cache, cache_lens, g, *, window_k: int, period_pi: int,
           num_skips: int, scale: float = 0.0, num_splits: int = 0, workspace=None, out=None,
           rolling: bool = False, levels=()):
    """pi-Attention decode: q [S, H, d], caches [S, H, L, d] (strided, last dim
    contiguous), cache_lens int32 [S] (query position len-1), g [S, H].
    rolling: the caches are rolling caches of L rows (position j in row j mod L).
    workspace: optional uint8 GPU tensor; allocated here when needed and absent."""
    code = _dtype_code(q)
    _need_cuda(q, k_cache, v_cache, cache_lens, g, out, workspace)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expect q [S, H, d] and caches [S, H, L, d]")
    S, H, d = q.shape
    if tuple(k_cache.shape[:2]) != (S, H) or k_cache.shape[3] != d:
        raise ValueError("cache shape does not match q")
    if cache_lens.dtype != torch.int32 or tuple(cache_lens.shape) != (S,):
        raise ValueError("cache_lens must be int32 [S]")
    if g.dtype != torch.float32 or tuple(g.shape) != (S, H):
        raise ValueError("g must be float32 [S, H]")
    if out is None:
        out = torch.empty_like(q)
    pat = make_pattern(window_k, period_pi, num_skips, False, scale, levels)
    need = decode_workspace_bytes(S, H, d, num_splits, pat)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    for t in (q, k_cache, v_cache, out):
        if t.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous")
    st = [(q.stride(0), q.stride(1), 0), tuple(k_cache.stride()[:3]),
          tuple(v_cache.stride()[:3]), (out.stride(0), out.stride(1), 0),
          (g.stride(0), g.stride(1), 0)]
    strides = Strides(*[x for s in st for x in s])
    fn = lib().piattn_decode_rolling if rolling else lib().piattn_decode
    rc = fn(code, S, H, d, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_lens), k_cache.shape[2],
            _ptr(g), _ptr(out), ctypes.byref(strides), ctypes.byref(pat), int(num_splits),
            _ptr(workspace), wbytes, ctypes.c_void_p(_stream(q.device)))
    _check(rc)
    return out


def neighbors_cap(window_k, period_pi, num_skips, bidirectional=False, levels=()) -> int:
    pat = make_pattern(window_k, period_pi, num_skips, bidirectional, levels=levels)
    return int(lib().piattn_neighbors_cap(ctypes.byref(pat)))


def neighbors(n: int, *, window_k: int, period_pi: int, num_skips: int, bidirectional=False,
              q_begin: int = 0, q_count: int | None = None, cap: int | None = None,
              device="cuda", levels=()):
    """Debug dump: (idx int32 [q_count, cap], kind int8, count int32) on the GPU."""
    pat = make_pattern(window_k, period_pi, num_skips, bidirectional, levels=levels)
    if q_count is None:
        q_count = n - q_begin
    if cap is None:
        cap = min(int(lib().piattn_neighbors_cap(ctypes.byref(pat))), n)
    idx = torch.empty((q_count, cap), dtype=torch.int32, device=device)
    kind = torch.empty((q_count, cap), dtype=torch.int8, device=device)
    count = torch.empty(q_count, dtype=torch.int32, device=device)
    rc = lib().piattn_neighbors(n, ctypes.byref(pat), q_begin, q_count, cap, _ptr(idx),
                                _ptr(kind), _ptr(count), ctypes.c_void_p(_stream(idx.device)))
    _check(rc)
    return idx, kind, count


FWD_KERNELS = {"auto": 0, "split": 1, "resid": 2, "gather": 3, "f32mfma": 4}
BWD_KERNELS = {"auto": 0, "band": 1, "gather": 2}


@contextlib.contextmanager
def forced_kernels(fwd: str = "auto", bwd: str = "auto"):
    """Testing and measurement: run fwd / bwd calls inside the block on the
    named kernels (piattn_debug_force_kernels; process-wide).  A forced
    kernel that cannot take a call makes it raise PiattnError
    (PIATTN_EUNSUPPORTED).  The automatic choice is restored on exit."""
    _check(lib().piattn_debug_force_kernels(FWD_KERNELS[fwd], BWD_KERNELS[bwd]))
    try:
        yield
    finally:
        _check(lib().piattn_debug_force_kernels(0, 0))


def version() -> str:
    return lib().piattn_version().decode()


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
