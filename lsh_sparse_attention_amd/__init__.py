"""Shared-QK LSH attention (Reformer) on MI355X: thin Python binding of liblsh.

Every call below marshals torch device tensors into the C ABI of
include/lsh.h and enqueues the library's HIP kernels on the current torch
stream.  No step of the computation runs in Python or torch; torch provides
device memory and streams only.  If liblsh.so is missing, the calls raise.

Pipeline (per (batch, head, round)): ``lsh_hash`` -> ``lsh_sort`` ->
``lsh_attn_fwd`` -> ``lsh_combine``; backward: ``lsh_attn_bwd``, or
``lsh_attn_bwd_saved`` on the workspace the forward filled, or
``lsh_attn_bwd_rehash``, which recomputes the hashing and sorting (nothing kept
from the forward but its output and lse).
"""
from __future__ import annotations

import ctypes
import math

import torch

from ._lib import (FF, LSH_BF16, LSH_F32, LSH_FLAG_DUP_BY_BUCKET, LSH_FLAG_NO_BUCKET_MASK, LSH_WS_BWD, LSH_WS_FWD,
                   LSH_WS_REHASH, LSH_WS_SORT, LSH_WS_TRAIN, LshError, Problem, check, lib)

__all__ = ["Problem", "LshError", "problem", "workspace_bytes", "lsh_hash", "lsh_sort", "lsh_sort_noalloc",
           "lsh_attn_fwd",
           "lsh_combine", "lsh_attn_bwd", "lsh_attn_bwd_saved", "lsh_attn_bwd_rehash", "LshAttention", "FF",
           "ff_problem", "ff_workspace_bytes", "lsh_ff_fwd", "lsh_ff_bwd"]

_DTYPES = {torch.float32: LSH_F32, torch.bfloat16: LSH_BF16}


def problem(batch, heads, seq_len, head_dim, n_hashes, n_buckets, chunk_len, scale=None,
            dtype=torch.bfloat16, causal=True, bucket_mask=True, dup_by_bucket=False) -> Problem:
    """lsh_problem_t; ``bucket_mask=False`` sets LSH_FLAG_NO_BUCKET_MASK, ``dup_by_bucket=True``
    LSH_FLAG_DUP_BY_BUCKET."""
    if isinstance(dtype, str):
        dtype = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype}")
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return Problem(batch, heads, seq_len, head_dim, n_hashes, n_buckets, chunk_len, int(bool(causal)),
                   float(scale), _DTYPES[dtype],
                   (0 if bucket_mask else LSH_FLAG_NO_BUCKET_MASK) | (LSH_FLAG_DUP_BY_BUCKET if dup_by_bucket else 0))


def torch_dtype(prob: Problem):
    return torch.bfloat16 if prob.dtype == LSH_BF16 else torch.float32


def _ptr(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _numel_check(t, n, name):
    if t.numel() < n:
        raise ValueError(f"{name} has {t.numel()} elements, needs {n}")


def workspace_bytes(prob: Problem, kind: int) -> int:
    return int(lib().lsh_workspace_bytes(ctypes.byref(prob), kind))


def _ws(ws, prob, kind):
    need = workspace_bytes(prob, kind)
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace has {ws.numel() * ws.element_size()} bytes, needs {need}")
    return _ptr(ws, "workspace"), ctypes.c_size_t(ws.numel() * ws.element_size())


def _tok(prob):
    return prob.batch * prob.heads * prob.seq_len


def lsh_hash(prob, q, rot, buckets, stream=None):
    dt = torch_dtype(prob)
    _numel_check(q, _tok(prob) * prob.head_dim, "q")
    _numel_check(rot, prob.n_hashes * prob.head_dim * (prob.n_buckets // 2), "rot")
    _numel_check(buckets, _tok(prob) * prob.n_hashes, "buckets")
    check("lsh_hash", lib().lsh_hash(ctypes.byref(prob), _ptr(q, "q", dt), _ptr(rot, "rot", dt),
                                     _ptr(buckets, "buckets", torch.int32), _stream(stream)))


def lsh_sort(prob, buckets, perm, inv, win_lo, ws, stream=None):
    n = _tok(prob) * prob.n_hashes
    for t, nm in ((buckets, "buckets"), (perm, "perm"), (inv, "inv"), (win_lo, "win_lo")):
        _numel_check(t, n, nm)
    wp, wn = _ws(ws, prob, LSH_WS_SORT)
    check("lsh_sort", lib().lsh_sort(ctypes.byref(prob), _ptr(buckets, "buckets", torch.int32),
                                     _ptr(perm, "perm", torch.int32), _ptr(inv, "inv", torch.int32),
                                     _ptr(win_lo, "win_lo", torch.int32), wp, wn, _stream(stream)))


def lsh_sort_noalloc(prob, buckets, perm, inv, win_lo, stream=None):
    """lsh_sort with the library's static scratch instead of a workspace (allocates nothing)."""
    n = _tok(prob) * prob.n_hashes
    for t, nm in ((buckets, "buckets"), (perm, "perm"), (inv, "inv"), (win_lo, "win_lo")):
        _numel_check(t, n, nm)
    check("lsh_sort_noalloc", lib().lsh_sort_noalloc(
        ctypes.byref(prob), _ptr(buckets, "buckets", torch.int32), _ptr(perm, "perm", torch.int32),
        _ptr(inv, "inv", torch.int32), _ptr(win_lo, "win_lo", torch.int32), _stream(stream)))


def lsh_attn_fwd(prob, q, v, perm, inv, win_lo, o_rounds, lse_rounds, ws, stream=None):
    dt = torch_dtype(prob)
    n, nd = _tok(prob), _tok(prob) * prob.head_dim
    _numel_check(q, nd, "q")
    _numel_check(v, nd, "v")
    _numel_check(o_rounds, nd * prob.n_hashes, "o_rounds")
    _numel_check(lse_rounds, n * prob.n_hashes, "lse_rounds")
    for t, nm in ((perm, "perm"), (inv, "inv"), (win_lo, "win_lo")):
        _numel_check(t, n * prob.n_hashes, nm)
    wp, wn = _ws(ws, prob, LSH_WS_FWD)
    check("lsh_attn_fwd", lib().lsh_attn_fwd(
        ctypes.byref(prob), _ptr(q, "q", dt), _ptr(v, "v", dt), _ptr(perm, "perm", torch.int32),
        _ptr(inv, "inv", torch.int32), _ptr(win_lo, "win_lo", torch.int32), _ptr(o_rounds, "o_rounds", dt),
        _ptr(lse_rounds, "lse_rounds", torch.float32), wp, wn, _stream(stream)))


def lsh_combine(prob, q, v, o_rounds, lse_rounds, out, lse, stream=None):
    dt = torch_dtype(prob)
    n, nd = _tok(prob), _tok(prob) * prob.head_dim
    for t, nm, k in ((q, "q", nd), (v, "v", nd), (o_rounds, "o_rounds", nd * prob.n_hashes),
                     (lse_rounds, "lse_rounds", n * prob.n_hashes), (out, "out", nd), (lse, "lse", n)):
        _numel_check(t, k, nm)
    check("lsh_combine", lib().lsh_combine(
        ctypes.byref(prob), _ptr(q, "q", dt), _ptr(v, "v", dt), _ptr(o_rounds, "o_rounds", dt),
        _ptr(lse_rounds, "lse_rounds", torch.float32), _ptr(out, "out", dt), _ptr(lse, "lse", torch.float32),
        _stream(stream)))


def lsh_attn_bwd(prob, q, v, out, dout, lse, perm, inv, win_lo, dq, dv, ws, stream=None):
    dt = torch_dtype(prob)
    n, nd = _tok(prob), _tok(prob) * prob.head_dim
    for t, nm, k in ((q, "q", nd), (v, "v", nd), (out, "out", nd), (dout, "dout", nd), (lse, "lse", n),
                     (perm, "perm", n * prob.n_hashes), (inv, "inv", n * prob.n_hashes),
                     (win_lo, "win_lo", n * prob.n_hashes), (dq, "dq", nd), (dv, "dv", nd)):
        _numel_check(t, k, nm)
    wp, wn = _ws(ws, prob, LSH_WS_BWD)
    check("lsh_attn_bwd", lib().lsh_attn_bwd(
        ctypes.byref(prob), _ptr(q, "q", dt), _ptr(v, "v", dt), _ptr(out, "out", dt), _ptr(dout, "dout", dt),
        _ptr(lse, "lse", torch.float32), _ptr(perm, "perm", torch.int32), _ptr(inv, "inv", torch.int32),
        _ptr(win_lo, "win_lo", torch.int32), _ptr(dq, "dq", dt), _ptr(dv, "dv", dt), wp, wn, _stream(stream)))


def lsh_attn_bwd_saved(prob, q, v, out, dout, lse, dq, dv, ws, stream=None):
    """lsh_attn_bwd on the records that lsh_attn_fwd left in ``ws`` (an LSH_WS_TRAIN workspace)."""
    dt = torch_dtype(prob)
    n, nd = _tok(prob), _tok(prob) * prob.head_dim
    for t, nm, k in ((q, "q", nd), (v, "v", nd), (out, "out", nd), (dout, "dout", nd), (lse, "lse", n),
                     (dq, "dq", nd), (dv, "dv", nd)):
        _numel_check(t, k, nm)
    wp, wn = _ws(ws, prob, LSH_WS_TRAIN)
    check("lsh_attn_bwd_saved", lib().lsh_attn_bwd_saved(
        ctypes.byref(prob), _ptr(q, "q", dt), _ptr(v, "v", dt), _ptr(out, "out", dt), _ptr(dout, "dout", dt),
        _ptr(lse, "lse", torch.float32), _ptr(dq, "dq", dt), _ptr(dv, "dv", dt), wp, wn, _stream(stream)))


def lsh_attn_bwd_rehash(prob, q, v, rot, out, dout, lse, dq, dv, ws, stream=None):
    """lsh_attn_bwd with buckets, sorted order and windows recomputed from q and rot (an LSH_WS_REHASH workspace)."""
    dt = torch_dtype(prob)
    n, nd = _tok(prob), _tok(prob) * prob.head_dim
    for t, nm, k in ((q, "q", nd), (v, "v", nd), (rot, "rot", prob.n_hashes * prob.head_dim * (prob.n_buckets // 2)),
                     (out, "out", nd), (dout, "dout", nd), (lse, "lse", n), (dq, "dq", nd), (dv, "dv", nd)):
        _numel_check(t, k, nm)
    wp, wn = _ws(ws, prob, LSH_WS_REHASH)
    check("lsh_attn_bwd_rehash", lib().lsh_attn_bwd_rehash(
        ctypes.byref(prob), _ptr(q, "q", dt), _ptr(v, "v", dt), _ptr(rot, "rot", dt), _ptr(out, "out", dt),
        _ptr(dout, "dout", dt), _ptr(lse, "lse", torch.float32), _ptr(dq, "dq", dt), _ptr(dv, "dv", dt), wp, wn,
        _stream(stream)))


class LshAttention:
    """Device buffers for one problem shape and the five calls in order.

    ``forward(q, v, rot)`` runs hash, sort, per-round attention and combine;
    ``backward(q, v, dout)`` runs the backward of the last forward (same q
    and v), on the records the forward left in the shared workspace.  Buffers
    are allocated once, here; the calls themselves allocate nothing.
    """

    def __init__(self, prob: Problem, device="cuda", backward=True):
        self.prob = prob
        B, H, L, d, nh = prob.batch, prob.heads, prob.seq_len, prob.head_dim, prob.n_hashes
        dt = torch_dtype(prob)
        kw = dict(device=device)
        self.buckets = torch.empty((B, H, nh, L), dtype=torch.int32, **kw)
        self.perm = torch.empty_like(self.buckets)
        self.inv = torch.empty_like(self.buckets)
        self.win_lo = torch.empty_like(self.buckets)
        self.o_rounds = torch.empty((B, H, nh, L, d), dtype=dt, **kw)
        self.lse_rounds = torch.empty((B, H, nh, L), dtype=torch.float32, **kw)
        self.out = torch.empty((B, H, L, d), dtype=dt, **kw)
        self.lse = torch.empty((B, H, L), dtype=torch.float32, **kw)
        self.ws_sort = torch.empty(max(1, workspace_bytes(prob, LSH_WS_SORT)), dtype=torch.uint8, **kw)
        # with a backward, one workspace serves both (the backward reads the forward's records)
        kind = LSH_WS_TRAIN if backward else LSH_WS_FWD
        self.ws_fwd = torch.empty(max(1, workspace_bytes(prob, kind)), dtype=torch.uint8, **kw)
        if backward:
            self.dq = torch.empty((B, H, L, d), dtype=dt, **kw)
            self.dv = torch.empty((B, H, L, d), dtype=dt, **kw)

    def forward(self, q, v, rot, stream=None):
        p = self.prob
        lsh_hash(p, q, rot, self.buckets, stream)
        lsh_sort(p, self.buckets, self.perm, self.inv, self.win_lo, self.ws_sort, stream)
        lsh_attn_fwd(p, q, v, self.perm, self.inv, self.win_lo, self.o_rounds, self.lse_rounds, self.ws_fwd, stream)
        lsh_combine(p, q, v, self.o_rounds, self.lse_rounds, self.out, self.lse, stream)
        return self.out, self.lse

    def backward(self, q, v, dout, stream=None):
        p = self.prob
        lsh_attn_bwd_saved(p, q, v, self.out, dout, self.lse, self.dq, self.dv, self.ws_fwd, stream)
        return self.dq, self.dv


# ----------------------------------------------------------------------------- chunked feed-forward

def ff_problem(rows, d_model, d_ff, chunks=1) -> FF:
    """lsh_ff_t for bf16 activations."""
    return FF(rows, d_model, d_ff, chunks, LSH_BF16)


def ff_workspace_bytes(ff: FF, backward: bool) -> int:
    return lib().lsh_ff_workspace_bytes(ctypes.byref(ff), 1 if backward else 0)


def _ff_ws(ws, ff, backward):
    need = ff_workspace_bytes(ff, backward)
    if ws is None:
        ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")
    return ws, need


def lsh_ff_fwd(ff, x, w1, b1, w2, b2, y, ws=None, stream=None):
    """y = relu(x w1 + b1) w2 + b2 in ff.chunks chunks of rows (lsh_ff_fwd)."""
    ws, need = _ff_ws(ws, ff, False)
    bf, f32 = torch.bfloat16, torch.float32
    check("lsh_ff_fwd", lib().lsh_ff_fwd(ctypes.byref(ff), _ptr(x, "x", bf), _ptr(w1, "w1", bf), _ptr(b1, "b1", f32),
                                         _ptr(w2, "w2", bf), _ptr(b2, "b2", f32), _ptr(y, "y", bf),
                                         _ptr(ws, "ws"), ctypes.c_size_t(ws.numel()), _stream(stream)))
    return y


def lsh_ff_bwd(ff, x, w1, b1, w2, dy, dx, dw1, db1, dw2, db2, ws=None, stream=None):
    """Gradients of sum(y * dy) (lsh_ff_bwd); the hidden activations are recomputed per chunk."""
    ws, need = _ff_ws(ws, ff, True)
    bf, f32 = torch.bfloat16, torch.float32
    check("lsh_ff_bwd", lib().lsh_ff_bwd(ctypes.byref(ff), _ptr(x, "x", bf), _ptr(w1, "w1", bf), _ptr(b1, "b1", f32),
                                         _ptr(w2, "w2", bf), _ptr(dy, "dy", bf), _ptr(dx, "dx", bf),
                                         _ptr(dw1, "dw1", f32), _ptr(db1, "db1", f32), _ptr(dw2, "dw2", f32),
                                         _ptr(db2, "db2", f32), _ptr(ws, "ws"), ctypes.c_size_t(ws.numel()),
                                         _stream(stream)))
    return dx, dw1, db1, dw2, db2
