"""ctypes wrapper of the fp64 CPU oracle (``lsh_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg.  The GPU library never imports it.

Arrays are per (batch, head) slice: q, v, dout [L, d] fp64, rot [nh, d, nb/2]
fp64; integer outputs are int32 [nh, L].  ``causal`` selects the causal sets
(the default) or the non-causal ones (no "not after the query" condition);
``bucket_mask`` False drops the same-bucket condition (chunks alone restrict);
``dup_by_bucket`` True counts duplicates over bucket co-membership in every
round instead of over the attended sets.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsh_oracle.c")
_LIB = os.path.join(_HERE, "liblsh_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, IEEE arithmetic)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        _lib = ctypes.CDLL(_LIB)
        _lib.lsh_oracle_threads.restype = ctypes.c_int
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def threads() -> int:
    return lib().lsh_oracle_threads()


def hash_(q, rot, n_buckets):
    q, rot = _f64(q), _f64(rot)
    L, d = q.shape
    nh = rot.shape[0]
    bk = np.empty((nh, L), np.int32)
    rc = lib().lsh_oracle_hash(ctypes.c_int(L), ctypes.c_int(d), ctypes.c_int(nh),
                               ctypes.c_int(n_buckets), _p(q), _p(rot), _p(bk))
    if rc:
        raise ValueError("oracle hash: invalid arguments")
    return bk


def sort(buckets, chunk_len):
    bk = _i32(buckets)
    nh, L = bk.shape
    perm = np.empty_like(bk)
    inv = np.empty_like(bk)
    win_lo = np.empty_like(bk)
    rc = lib().lsh_oracle_sort(ctypes.c_int(L), ctypes.c_int(nh), ctypes.c_int(chunk_len), _p(bk),
                               _p(perm), _p(inv), _p(win_lo))
    if rc:
        raise ValueError("oracle sort: invalid arguments")
    return perm, inv, win_lo


def union_mask(buckets, perm, inv, chunk_len, causal=True, bucket_mask=True):
    bk, perm, inv = _i32(buckets), _i32(perm), _i32(inv)
    nh, L = bk.shape
    mask = np.empty((L, L), np.uint8)
    rc = lib().lsh_oracle_union_mask(ctypes.c_int(L), ctypes.c_int(nh), ctypes.c_int(chunk_len),
                                     ctypes.c_int(int(bool(causal))), ctypes.c_int(int(bool(bucket_mask))),
                                     _p(bk), _p(perm), _p(inv), _p(mask))
    if rc:
        raise ValueError("oracle union_mask: invalid arguments")
    return mask.astype(bool)


def forward(q, v, buckets, perm, inv, chunk_len, scale, causal=True, bucket_mask=True, dup_by_bucket=False):
    q, v = _f64(q), _f64(v)
    bk, perm, inv = _i32(buckets), _i32(perm), _i32(inv)
    L, d = q.shape
    nh = bk.shape[0]
    out = np.empty((L, d), np.float64)
    lse = np.empty(L, np.float64)
    rc = lib().lsh_oracle_forward(ctypes.c_int(L), ctypes.c_int(d), ctypes.c_int(nh),
                                  ctypes.c_int(chunk_len), ctypes.c_int(int(bool(causal))),
                                  ctypes.c_int(int(bool(bucket_mask))), ctypes.c_int(int(bool(dup_by_bucket))),
                                  ctypes.c_double(scale), _p(q), _p(v),
                                  _p(bk), _p(perm), _p(inv), _p(out), _p(lse))
    if rc:
        raise ValueError("oracle forward: invalid arguments")
    return out, lse


def backward(q, v, dout, buckets, perm, inv, out, lse, chunk_len, scale, causal=True, bucket_mask=True,
             dup_by_bucket=False):
    q, v, dout, out, lse = _f64(q), _f64(v), _f64(dout), _f64(out), _f64(lse)
    bk, perm, inv = _i32(buckets), _i32(perm), _i32(inv)
    L, d = q.shape
    nh = bk.shape[0]
    dq = np.empty((L, d), np.float64)
    dv = np.empty((L, d), np.float64)
    rc = lib().lsh_oracle_backward(ctypes.c_int(L), ctypes.c_int(d), ctypes.c_int(nh),
                                   ctypes.c_int(chunk_len), ctypes.c_int(int(bool(causal))),
                                   ctypes.c_int(int(bool(bucket_mask))), ctypes.c_int(int(bool(dup_by_bucket))),
                                   ctypes.c_double(scale), _p(q), _p(v),
                                   _p(dout), _p(bk), _p(perm), _p(inv), _p(out), _p(lse), _p(dq),
                                   _p(dv))
    if rc:
        raise ValueError("oracle backward: invalid arguments")
    return dq, dv


def head(q, v, rot, n_buckets, chunk_len, scale, dout=None, causal=True, bucket_mask=True, dup_by_bucket=False):
    """Hash, sort, forward and (with ``dout``) backward of one slice."""
    q, v, rot = _f64(q), _f64(v), _f64(rot)
    L, d = q.shape
    nh = rot.shape[0]
    res = {k: np.empty((nh, L), np.int32) for k in ("buckets", "perm", "inv", "win_lo")}
    res["out"] = np.empty((L, d), np.float64)
    res["lse"] = np.empty(L, np.float64)
    if dout is not None:
        dout = _f64(dout)
        res["dq"] = np.empty((L, d), np.float64)
        res["dv"] = np.empty((L, d), np.float64)
    rc = lib().lsh_oracle_head(
        ctypes.c_int(L), ctypes.c_int(d), ctypes.c_int(nh), ctypes.c_int(n_buckets),
        ctypes.c_int(chunk_len), ctypes.c_int(int(bool(causal))), ctypes.c_int(int(bool(bucket_mask))),
        ctypes.c_int(int(bool(dup_by_bucket))), ctypes.c_double(scale), _p(q), _p(v),
        _p(rot), _p(dout),
        _p(res["buckets"]), _p(res["perm"]), _p(res["inv"]), _p(res["win_lo"]), _p(res["out"]),
        _p(res["lse"]), _p(res.get("dq")), _p(res.get("dv")))
    if rc:
        raise ValueError("oracle head: invalid arguments")
    return res


def run_inputs(inputs, slices=None, backward=None):
    """Run the oracle on (b, h) slices of an ``inputs.generate`` result.

    Returns {(b, h): head-result}.  ``slices`` defaults to all of them.
    """
    from lsh_sparse_attention_amd.inputs import to_f64
    cfg = inputs["cfg"]
    if backward is None:
        backward = "dout" in inputs
    if slices is None:
        slices = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    rot = to_f64(inputs["rot"], cfg.dtype)
    res = {}
    for (b, h) in slices:
        q = to_f64(inputs["q"][b, h], cfg.dtype)
        v = to_f64(inputs["v"][b, h], cfg.dtype)
        do = to_f64(inputs["dout"][b, h], cfg.dtype) if backward else None
        res[(b, h)] = head(q, v, rot, cfg.n_buckets, cfg.chunk_len, cfg.scale, do, causal=cfg.causal,
                           bucket_mask=cfg.bucket_mask, dup_by_bucket=cfg.dup_by_bucket)
    return res
