"""Dense NumPy brute force used to pin the oracle on tiny problems.

Independent of the oracle: it evaluates the attended-set predicate for every
(query, key) pair from a sort computed with ``numpy.lexsort``, then runs dense
masked softmax attention in fp64.  Definitions follow "Reformer: The Efficient
Transformer" §2 (hash h(x) = argmax([xR; -xR]), sort by bucket, causal mask,
self only when nothing else) and App. A (union of round sets, each key once).
"""
import numpy as np


def buckets(q, rot):
    """[nh, L] int32: argmax of [qR_r; -qR_r] (first index on ties)."""
    out = []
    for r in range(rot.shape[0]):
        y = q @ rot[r]
        out.append(np.argmax(np.concatenate([y, -y], axis=1), axis=1))
    return np.asarray(out, dtype=np.int32)


def sort(bk):
    """perm (sorted -> position) and inv (position -> sorted) per round."""
    nh, L = bk.shape
    pos = np.arange(L)
    perm = np.stack([np.lexsort((pos, bk[r])) for r in range(nh)]).astype(np.int32)
    inv = np.empty_like(perm)
    for r in range(nh):
        inv[r, perm[r]] = pos
    return perm, inv


def round_masks(bk, m, causal=True, bucket_mask=True):
    """[nh, L, L] bool: j in A_i^r (self included).  Without ``causal`` the
    condition j <= i is dropped (same bucket, own chunk or the one before);
    without ``bucket_mask`` the same-bucket condition is dropped."""
    nh, L = bk.shape
    _, inv = sort(bk)
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    out = []
    for r in range(nh):
        c = inv[r] // m
        same = (bk[r][:, None] == bk[r][None, :]) if bucket_mask else np.ones((L, L), dtype=bool)
        dc = c[:, None] - c[None, :]
        order = (j <= i) if causal else np.ones((L, L), dtype=bool)
        out.append(same & order & ((dc == 0) | (dc == 1)))
    return np.asarray(out)


def union_mask(bk, m, causal=True, bucket_mask=True):
    return round_masks(bk, m, causal, bucket_mask).any(axis=0)


def dup_weights(bk, m, causal=True):
    """[L, L] k_ij / N_ij: rounds whose set holds j over rounds in which j
    shares i's bucket (the duplicate count over bucket co-membership)."""
    k = round_masks(bk, m, causal).sum(axis=0)
    n = sum((bk[r][:, None] == bk[r][None, :]).astype(np.int64) for r in range(bk.shape[0]))
    return np.divide(k, n, out=np.zeros(k.shape), where=n > 0)


def attention(q, v, mask, scale, weights=None):
    """Dense masked softmax over the union without self; a row with nothing
    else attends to itself.  ``weights`` multiply the members' exponentials.
    Returns (out, lse)."""
    L = q.shape[0]
    k = q / np.linalg.norm(q, axis=1, keepdims=True)
    logits = scale * (q @ k.T)
    if weights is not None:
        logits = logits + np.log(np.where(mask & (weights > 0), weights, 1.0))
    allowed = mask & ~np.eye(L, dtype=bool)
    empty = ~allowed.any(axis=1)
    allowed[empty, empty.nonzero()[0]] = True
    lg = np.where(allowed, logits, -np.inf)
    mx = lg.max(axis=1, keepdims=True)
    e = np.exp(lg - mx)
    den = e.sum(axis=1, keepdims=True)
    out = (e / den) @ v
    lse = (mx + np.log(den))[:, 0]
    return out, lse
