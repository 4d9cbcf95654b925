"""Seeded synthetic inputs for shared-QK LSH attention.

This module only draws numbers.  It is shared by the tests, the benchmark and
the smoke check, and it holds none of the attention arithmetic: no hashing,
sorting, masking or softmax happens here.  The one place it looks at the
rotation is the argmax-margin rule, which conditions the draw so that the
bucket of every (row, round) is decided by a gap far larger than any fp32
rounding error; it computes the gap between the two largest entries of
[xR; -xR], never which entry wins.

Workload shapes stand in for the two workloads the Reformer paper trains on
(12K-token image generation and 64K-token text; "Reformer: The Efficient
Transformer", §1 Introduction and §5 Experiments).  The datasets themselves are
not used: Q, V and the upstream gradient are Gaussian (or a Gaussian mixture
for the skewed-occupancy stress case).

Recipe, for every configuration:
  * ``numpy.random.default_rng(seed)`` (PCG64); draws are fp64;
  * draw order: rotation R, [mixture centres and assignments], Q, margin
    redraws of failing Q rows (in row order), [V assignments], V, dO;
  * values are rounded fp64 -> fp32 (round-to-nearest-even) and, for bf16
    problems, fp32 -> bf16 (round-to-nearest-even); R is rounded the same way;
  * margin rule: for every row q and round r, with y = qR_r and z = [y; -y],
    (top1(z) - top2(z)) / ||q|| >= 1e-4, and the gap is at least twice the
    fp32 rounding bound of y, (d+2) 2^-24 ||q|| max_j ||R_:j||.  Failing rows
    are redrawn until all pass.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
import math

import numpy as np

MARGIN = 1e-4


@dataclass(frozen=True)
class Config:
    """One problem shape.  ``dtype`` is 'f32' or 'bf16'."""
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    n_buckets: int
    n_hashes: int
    chunk_len: int
    dtype: str
    clustered: bool
    backward: bool
    seed: int
    n_clusters: int = 256
    cluster_sigma: float = 0.1
    causal: bool = True
    bucket_mask: bool = True
    dup_by_bucket: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


# The five workload shapes: a tiny fp32 forward case, a mid-size case, the
# 12K-token image-shaped case, the 64K-token text-shaped case and a 64K stress
# case whose inputs are a 256-component Gaussian mixture (heavily skewed
# bucket occupancy, so buckets overflow the two-chunk window).
CONFIGS = {
    "tiny": Config("tiny", 1, 1, 1024, 64, 32, 1, 64, "f32", False, False, 1),
    "mid": Config("mid", 8, 8, 4096, 64, 64, 2, 128, "bf16", False, True, 2),
    "image": Config("image", 1, 8, 12288, 64, 192, 8, 128, "bf16", False, True, 3),
    "text": Config("text", 1, 8, 65536, 128, 1024, 4, 128, "bf16", False, True, 4),
    "stress": Config("stress", 4, 8, 65536, 64, 1024, 8, 128, "bf16", True, True, 5),
}


# ----------------------------------------------------------------------------
# rounding helpers (storage form: float32 arrays for f32, uint16 bits for bf16)

def f64_to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even; returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = f64_to_f32(x64)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of a stored array."""
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(stored).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# margin rule

def margin_ok(q64: np.ndarray, rot64: np.ndarray, block_elems: int = 1 << 25) -> np.ndarray:
    """Boolean per row of ``q64`` [N, d]: does the row meet the argmax margin in
    every round of ``rot64`` [nh, d, nb/2]?

    The projections are computed in fp32 (torch CPU).  Each computed entry of
    y = qR is within e = (d+2) 2^-24 |q| max_j |R_j| of the exact value
    (recursive-summation bound with Cauchy-Schwarz), so the computed top-2 gap
    is within 2e of the exact one; the rule asks the computed gap for both
    thresholds plus that 2e.
    """
    import torch
    nh, d, half = rot64.shape
    rcat = torch.from_numpy(np.ascontiguousarray(rot64.transpose(1, 0, 2).reshape(d, nh * half))).float()
    col_norm = float(torch.linalg.vector_norm(rcat.double(), dim=0).max())
    gamma = (d + 2) * 2.0 ** -24
    n = q64.shape[0]
    ok = np.empty(n, dtype=bool)
    rows = max(1, block_elems // max(1, nh * half))
    for a in range(0, n, rows):
        qb64 = np.ascontiguousarray(q64[a:a + rows])
        qb = torch.from_numpy(qb64).float()
        y = (qb @ rcat).view(-1, nh, half)
        if half >= 2:
            top = y.abs().topk(2, dim=-1).values
            gap = (top[..., 0] - top[..., 1]).double()
        else:
            gap = 2.0 * y[..., 0].abs().double()
        norm = torch.from_numpy(np.sqrt(np.einsum("ij,ij->i", qb64, qb64)))[:, None]
        err = 2.0 * gamma * norm * col_norm            # bound on |computed gap - exact gap|
        good = (gap >= MARGIN * norm + err) & (gap >= 2.0 * err) & (norm > 0)
        ok[a:a + rows] = good.all(dim=-1).numpy()
    return ok


def generate_tied_rotation(seed: int, rows: int, d: int, n_buckets: int, n_hashes: int, n_base: int = 6,
                           dtype: str = "bf16") -> dict:
    """Inputs with exact ties in [qR ; -qR], for the hash's first-index rule.

    Each round's rotation is built from ``n_base`` random base columns: column j
    is base column c_j times a sign s_j (both drawn), so the entries of
    [qR ; -qR] take only the values +-(q . B_c) and every value occurs several
    times, in one 32-column tile and across tiles.  Half of the base columns
    keep one sign over all their copies, so their largest entries lie in the
    -y half for half of the rows; the others occur with both signs.  A negated
    copy of a column gives the exactly negated products and sums, so these
    ties are exact in any precision.  Rows are drawn, and redrawn in order,
    until in every round the largest |q . B_c| beats the second largest base
    column by the margin rule's gap (computed as in ``margin_ok``, over the
    base columns): the winning value is then decided far from any rounding,
    and which of its equal copies wins only by the tie rule.
    Returns q [rows, d] and rot [nh, d, nb/2] in storage form, the rotation's
    and the base columns' fp64 values, and each column's base index and sign.
    """
    import torch
    rng = np.random.default_rng(seed)
    half = n_buckets // 2
    base = to_storage(rng.standard_normal((n_hashes, d, n_base)), dtype)
    base64 = to_f64(base, dtype)
    cls = rng.integers(0, n_base, size=(n_hashes, half))
    # the first half of the base columns keep one sign over all their copies (so
    # their largest entries can lie in the -y half only), the others mix signs
    fixed = rng.choice(np.array([-1.0, 1.0]), size=(n_hashes, n_base))
    mixed = rng.choice(np.array([-1.0, 1.0]), size=(n_hashes, half))
    sign = np.where(cls < n_base // 2, np.take_along_axis(fixed, cls, axis=1), mixed)
    rot64 = np.stack([base64[r][:, cls[r]] * sign[r] for r in range(n_hashes)])
    rot = to_storage(rot64, dtype)
    assert np.array_equal(to_f64(rot, dtype), rot64)
    q = to_storage(rng.standard_normal((rows, d)), dtype)
    bt = torch.from_numpy(np.ascontiguousarray(base64.transpose(1, 0, 2).reshape(d, -1))).float()
    col_norm = float(np.sqrt((base64 ** 2).sum(axis=1)).max())
    gamma = (d + 2) * 2.0 ** -24

    def ok(qs):
        q64 = to_f64(qs, dtype)
        v = (torch.from_numpy(q64).float() @ bt).view(-1, n_hashes, n_base).abs()
        top = v.topk(2, dim=-1).values
        gap = (top[..., 0] - top[..., 1]).double()
        norm = torch.from_numpy(np.sqrt(np.einsum("ij,ij->i", q64, q64)))[:, None]
        err = 2.0 * gamma * norm * col_norm
        return ((gap >= MARGIN * norm + err) & (gap >= 2.0 * err) & (norm > 0)).all(dim=-1).numpy()

    bad = np.nonzero(~ok(q))[0]
    while bad.size:
        q[bad] = to_storage(rng.standard_normal((bad.size, d)), dtype)
        bad = bad[~ok(q[bad])]
    return {"q": q, "rot": rot, "rot64": rot64, "base64": base64, "classes": cls, "signs": sign}


# ----------------------------------------------------------------------------
# generation

def generate(cfg: Config, with_grad: bool | None = None) -> dict:
    """Draw the inputs of ``cfg``.

    Returns a dict with storage-form arrays ``q`` and ``v`` [B,H,L,d], ``rot``
    [nh,d,nb/2], ``dout`` [B,H,L,d] (when a gradient is wanted), the config,
    and the number of margin redraws.
    """
    if with_grad is None:
        with_grad = cfg.backward
    B, H, L, d = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim
    nh, nb = cfg.n_hashes, cfg.n_buckets
    if nb % 2:
        raise ValueError("n_buckets must be even")
    rng = np.random.default_rng(cfg.seed)
    rot = to_storage(rng.standard_normal((nh, d, nb // 2)), cfg.dtype)
    rot64 = to_f64(rot, cfg.dtype)

    n = B * H * L
    if cfg.clustered:
        k = cfg.n_clusters
        centres = rng.standard_normal((B * H, k, d))
        assign = rng.integers(0, k, size=(B * H, L))
        head_of_row = np.repeat(np.arange(B * H), L)
        q64 = centres[head_of_row, assign.reshape(-1)] + cfg.cluster_sigma * rng.standard_normal((n, d))
    else:
        q64 = rng.standard_normal((n, d))
    q = to_storage(q64, cfg.dtype)
    del q64
    redraws = 0
    bad = np.nonzero(~margin_ok(to_f64(q, cfg.dtype), rot64))[0]
    while bad.size:
        redraws += int(bad.size)
        if cfg.clustered:
            fresh = centres[bad // L, assign.reshape(-1)[bad]] + cfg.cluster_sigma * rng.standard_normal((bad.size, d))
        else:
            fresh = rng.standard_normal((bad.size, d))
        q[bad] = to_storage(fresh, cfg.dtype)
        still = ~margin_ok(to_f64(q[bad], cfg.dtype), rot64)
        bad = bad[still]

    if cfg.clustered:
        assign_v = rng.integers(0, cfg.n_clusters, size=(B * H, L))
        v64 = centres[head_of_row, assign_v.reshape(-1)] + cfg.cluster_sigma * rng.standard_normal((n, d))
    else:
        v64 = rng.standard_normal((n, d))
    v = to_storage(v64, cfg.dtype)
    del v64
    out = {
        "cfg": cfg,
        "q": q.reshape(B, H, L, d),
        "v": v.reshape(B, H, L, d),
        "rot": rot,
        "redraws": redraws,
    }
    if with_grad:
        out["dout"] = to_storage(rng.standard_normal((n, d)), cfg.dtype).reshape(B, H, L, d)
    return out


def small_config(name="small", batch=1, heads=1, seq_len=256, head_dim=64, n_buckets=8,
                 n_hashes=2, chunk_len=32, dtype="f32", clustered=False, seed=11, **kw) -> Config:
    """A parity-test shape; any field can be overridden."""
    return Config(name, batch, heads, seq_len, head_dim, n_buckets, n_hashes, chunk_len, dtype,
                  clustered, True, seed, **kw)


# ----------------------------------------------------------------------------- feed-forward layer
# The ablation shape of the Reformer paper (§5 Experiments): d_model = 1024,
# d_ff = 4096; rows are the B * L positions of a batch.
FF_SHAPE = {"d_model": 1024, "d_ff": 4096}


def generate_ff(n: int, d_model: int, d_ff: int, seed: int, grid: bool = True) -> dict:
    """Seeded inputs of the feed-forward layer: x, w1, w2, dy as bf16 bit
    patterns (uint16), b1, b2 as float32.

    With ``grid`` every value lies on a coarse power-of-two grid (x, dy in
    multiples of 1/4 up to 1, weights in multiples of 1/64 up to 1/8, biases
    in multiples of 1/256), so every pre-activation x W1 + b1 and every
    dy W2^T is a sum of exactly representable terms whose partial sums stay
    exact in fp32 (at most 2^15 distinct steps): the ReLU decisions of an fp32
    kernel and of an fp64 oracle then agree exactly (the role the argmax
    margin rule plays for the hash).  Without ``grid`` (timing only) the
    values are Gaussian, scaled as for a trained layer.
    Draw order: x, w1, b1, w2, b2, dy.
    """
    rng = np.random.default_rng(seed)
    if grid:
        def g(shape, num, den):
            return rng.integers(-num, num + 1, size=shape).astype(np.float64) / den
        x, w1, b1 = g((n, d_model), 4, 4), g((d_model, d_ff), 8, 64), g(d_ff, 64, 256)
        w2, b2, dy = g((d_ff, d_model), 8, 64), g(d_model, 64, 256), g((n, d_model), 4, 4)
    else:
        x = rng.standard_normal((n, d_model))
        w1 = rng.standard_normal((d_model, d_ff)) / np.sqrt(d_model)
        b1 = rng.standard_normal(d_ff) * 0.1
        w2 = rng.standard_normal((d_ff, d_model)) / np.sqrt(d_ff)
        b2 = rng.standard_normal(d_model) * 0.1
        dy = rng.standard_normal((n, d_model))
    bits = lambda a: f32_to_bf16_bits(f64_to_f32(a))
    return {"x": bits(x), "w1": bits(w1), "b1": f64_to_f32(b1), "w2": bits(w2), "b2": f64_to_f32(b2),
            "dy": bits(dy), "n": n, "d_model": d_model, "d_ff": d_ff, "grid": grid}
