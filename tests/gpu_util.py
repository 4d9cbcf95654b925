"""Helpers of the GPU parity tests: run the library through its C ABI on
seeded inputs, run the oracle on the same inputs, compare."""
import os
import sys

import numpy as np
import torch

import lsh_sparse_attention_amd as lsh
from lsh_sparse_attention_amd import inputs as gen
from oracle import oracle as ora

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def to_f64(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def run_gpu(x, backward=True, rounds=False):
    cfg = x["cfg"]
    prob = lsh.problem(cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.n_hashes, cfg.n_buckets,
                       cfg.chunk_len, cfg.scale, cfg.dtype, causal=cfg.causal, bucket_mask=cfg.bucket_mask,
                       dup_by_bucket=cfg.dup_by_bucket)
    q = to_device(x["q"], cfg.dtype)
    v = to_device(x["v"], cfg.dtype)
    rot = to_device(x["rot"], cfg.dtype)
    mod = lsh.LshAttention(prob, backward=backward)
    mod.forward(q, v, rot)
    res = {}
    if backward:
        do = to_device(x["dout"], cfg.dtype)
        mod.backward(q, v, do)
    torch.cuda.synchronize()
    for k in ("buckets", "perm", "inv", "win_lo"):
        res[k] = getattr(mod, k).cpu().numpy()
    res["out"] = to_f64(mod.out)
    res["lse"] = mod.lse.cpu().numpy().astype(np.float64)
    if rounds:
        res["o_rounds"] = to_f64(mod.o_rounds)
        res["lse_rounds"] = mod.lse_rounds.cpu().numpy().astype(np.float64)
    if backward:
        res["dq"] = to_f64(mod.dq)
        res["dv"] = to_f64(mod.dv)
    del mod
    return res


def assert_close(name, got, want, tol):
    err = np.abs(got - want)
    bad = err > tol + tol * np.abs(want)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} outside atol=rtol={tol}; max abs err "
                             f"{err.max():.3e}; first at {idx.tolist()}: got {got[tuple(idx[0])]} "
                             f"want {want[tuple(idx[0])]}")


def check_sort_properties(res, cfg):
    """Any-size properties of lsh_sort's output, for every (b, h, round)."""
    B, H, nh, L = res["buckets"].shape
    m = cfg.chunk_len
    bk = res["buckets"].reshape(-1, L)
    perm = res["perm"].reshape(-1, L)
    inv = res["inv"].reshape(-1, L)
    wl = res["win_lo"].reshape(-1, L)
    assert bk.min() >= 0 and bk.max() < cfg.n_buckets
    ar = np.arange(L)
    for s in range(bk.shape[0]):
        p = perm[s]
        assert np.array_equal(np.sort(p), ar), "perm is not a permutation"
        assert np.array_equal(inv[s][p], ar), "inv is not perm^-1"
        sb = bk[s][p]
        assert np.all(np.diff(sb) >= 0), "not sorted by bucket"
        assert np.all(np.diff(p)[np.diff(sb) == 0] > 0), "not stable"
        first = np.searchsorted(sb, sb, side="left")       # first sorted index of each sorted row's bucket
        start_of_pos = np.empty(L, np.int64)
        start_of_pos[p] = first
        want = np.maximum(start_of_pos, (inv[s] // m - 1) * m)
        assert np.array_equal(wl[s], want), "win_lo"


def compare_slices(x, res, slices, backward=True, check_rounds=True):
    """Bit-exact hash/sort and toleranced outputs against the oracle for (b, h) slices."""
    cfg = x["cfg"]
    tol = TOL[cfg.dtype]
    ores = ora.run_inputs(x, slices=slices, backward=backward)
    for (b, h), o in ores.items():
        tag = f"{cfg.name}[b={b},h={h}]"
        for k in ("buckets", "perm", "inv", "win_lo"):
            got = res[k][b, h]
            if not np.array_equal(got, o[k]):
                n = int((got != o[k]).sum())
                raise AssertionError(f"{tag} {k}: {n} mismatches")
        assert_close(tag + " out", res["out"][b, h], o["out"], tol)
        assert_close(tag + " lse", res["lse"][b, h], o["lse"], tol)
        if backward:
            assert_close(tag + " dq", res["dq"][b, h], o["dq"], tol)
            assert_close(tag + " dv", res["dv"][b, h], o["dv"], tol)
    return ores


BACKWARD_ENTRIES = ("saved", "standalone", "rehash")


def run_gpu_backward_entries(x):
    """The forward, then the gradient from each of the three backward entry points:
    lsh_attn_bwd_saved (on the forward's workspace, as LshAttention runs it), lsh_attn_bwd (records
    derived again from perm, inv, win_lo) and lsh_attn_bwd_rehash (buckets, order and windows
    recomputed from q and the rotations).  Returns the forward's results and, per entry point,
    dq and dv as fp64 arrays and their raw bits."""
    from lsh_sparse_attention_amd import _lib
    cfg = x["cfg"]
    prob = lsh.problem(cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.n_hashes, cfg.n_buckets,
                       cfg.chunk_len, cfg.scale, cfg.dtype, causal=cfg.causal, bucket_mask=cfg.bucket_mask,
                       dup_by_bucket=cfg.dup_by_bucket)
    q, v = to_device(x["q"], cfg.dtype), to_device(x["v"], cfg.dtype)
    rot, do = to_device(x["rot"], cfg.dtype), to_device(x["dout"], cfg.dtype)
    mod = lsh.LshAttention(prob)
    mod.forward(q, v, rot)
    grads = {"saved": tuple(t.clone() for t in mod.backward(q, v, do))}
    ws = torch.empty(max(1, lsh.workspace_bytes(prob, _lib.LSH_WS_BWD)), dtype=torch.uint8, device="cuda")
    dq, dv = torch.empty_like(q), torch.empty_like(v)
    lsh.lsh_attn_bwd(prob, q, v, mod.out, do, mod.lse, mod.perm, mod.inv, mod.win_lo, dq, dv, ws)
    grads["standalone"] = (dq, dv)
    del ws
    wr = torch.empty(max(1, lsh.workspace_bytes(prob, _lib.LSH_WS_REHASH)), dtype=torch.uint8, device="cuda")
    dq2, dv2 = torch.empty_like(q), torch.empty_like(v)
    lsh.lsh_attn_bwd_rehash(prob, q, v, rot, mod.out, do, mod.lse, dq2, dv2, wr)
    grads["rehash"] = (dq2, dv2)
    torch.cuda.synchronize()
    del wr
    res = {k: getattr(mod, k).cpu().numpy() for k in ("buckets", "perm", "inv", "win_lo")}
    res["out"] = to_f64(mod.out)
    res["lse"] = mod.lse.cpu().numpy().astype(np.float64)
    bits = (lambda t: t.view(torch.int16)) if cfg.dtype == "bf16" else (lambda t: t.view(torch.int32))
    for name, (a, b) in grads.items():
        res["dq_" + name], res["dv_" + name] = to_f64(a), to_f64(b)
        res["bits_" + name] = (bits(a).cpu().numpy(), bits(b).cpu().numpy())
    del mod
    return res


def compare_backward_entries(x, res, slices):
    """Each backward entry point's dq and dv against the oracle's on (b, h) slices (elementwise,
    to the problem's tolerance), the forward's hash, sort and outputs likewise, and the three entry
    points against one another bit for bit (the same kernels on the same records)."""
    cfg = x["cfg"]
    tol = TOL[cfg.dtype]
    ores = ora.run_inputs(x, slices=slices, backward=True)
    for (b, h), o in ores.items():
        tag = f"{cfg.name}[b={b},h={h}]"
        for k in ("buckets", "perm", "inv", "win_lo"):
            if not np.array_equal(res[k][b, h], o[k]):
                raise AssertionError(f"{tag} {k}: {int((res[k][b, h] != o[k]).sum())} mismatches")
        assert_close(tag + " out", res["out"][b, h], o["out"], tol)
        for name in BACKWARD_ENTRIES:
            assert_close(f"{tag} dq ({name})", res["dq_" + name][b, h], o["dq"], tol)
            assert_close(f"{tag} dv ({name})", res["dv_" + name][b, h], o["dv"], tol)
    for name in BACKWARD_ENTRIES[1:]:
        for i, what in enumerate(("dq", "dv")):
            assert np.array_equal(res["bits_" + name][i], res["bits_saved"][i]), f"{what} of {name} differs from saved"
    return ores


def compare_hash_sort_all_slices(x, res):
    """Buckets, perm, inv and win_lo of every (b, h) slice against the oracle's hash and sort, bit for bit."""
    cfg = x["cfg"]
    rot = gen.to_f64(x["rot"], cfg.dtype)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            bk = ora.hash_(gen.to_f64(x["q"][b, h], cfg.dtype), rot, cfg.n_buckets)
            if not np.array_equal(res["buckets"][b, h], bk):
                raise AssertionError(f"{cfg.name}[b={b},h={h}] buckets: {int((res['buckets'][b, h] != bk).sum())} "
                                     "mismatches")
            perm, inv, wl = ora.sort(bk, cfg.chunk_len)
            for k, want in (("perm", perm), ("inv", inv), ("win_lo", wl)):
                if not np.array_equal(res[k][b, h], want):
                    raise AssertionError(f"{cfg.name}[b={b},h={h}] {k}: {int((res[k][b, h] != want).sum())} "
                                         "mismatches")
