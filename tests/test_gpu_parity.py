"""GPU parity: the library (called through its C ABI) against the fp64 oracle.

Hash buckets, permutations, inverse permutations and window bounds must match
bit for bit; outputs, lse and gradients within atol = rtol = 1e-4 (fp32
problems) or 2e-2 (bf16 problems), elementwise, against the fp64 oracle.
Small shapes are compared whole; the five workload shapes at full size have
the hash and sort of every (batch, head) slice compared with the oracle's bit
for bit, and outputs and gradients compared on sampled slices.  Each of the
three backward entry points is compared with the oracle on its own.
"""
import numpy as np
import pytest
import torch

from lsh_sparse_attention_amd import inputs as gen
import gpu_util as gu
from oracle import oracle as ora

pytestmark = pytest.mark.gpu

# name, B, H, L, d, nb, nh, m, dtype, clustered
SMALL = [
    ("f32-base", 1, 2, 1024, 64, 16, 3, 32, "f32", False),
    ("bf16-base", 2, 2, 1024, 64, 16, 3, 32, "bf16", False),
    ("bf16-d128", 1, 2, 2048, 128, 32, 2, 64, "bf16", False),
    ("f32-d128", 1, 1, 1024, 128, 64, 2, 64, "f32", False),
    ("f32-d32", 1, 1, 512, 32, 8, 2, 16, "f32", False),
    ("bf16-d32", 1, 2, 512, 32, 8, 2, 16, "bf16", False),
    ("ragged-sort-tile", 1, 2, 2016, 64, 64, 2, 32, "bf16", False),
    ("multi-tile", 1, 1, 5120, 64, 128, 2, 64, "bf16", False),
    ("two-buckets", 1, 2, 512, 64, 2, 2, 32, "f32", False),
    ("one-chunk", 1, 1, 256, 64, 8, 2, 256, "f32", False),
    ("chunk-1", 1, 1, 128, 32, 4, 2, 1, "f32", False),
    ("one-round", 1, 2, 1024, 64, 32, 1, 64, "bf16", False),
    ("eight-rounds", 1, 1, 1024, 64, 16, 8, 32, "bf16", False),
    ("clustered", 1, 2, 2048, 64, 64, 4, 64, "bf16", True),
    ("many-buckets", 1, 1, 4096, 64, 4096, 2, 128, "bf16", False),
    ("tiny-L", 1, 1, 8, 32, 4, 2, 2, "f32", False),
    ("single-token", 1, 1, 1, 32, 2, 1, 1, "f32", False),
    ("bf16-m96", 1, 2, 1536, 64, 32, 3, 96, "bf16", False),
    ("bf16-m256", 1, 1, 2048, 128, 16, 2, 256, "bf16", False),
    ("bf16-runs", 1, 4, 8192, 64, 128, 2, 128, "bf16", False),
    ("bf16-m1", 1, 2, 512, 64, 8, 2, 1, "bf16", False),
    ("bf16-nh16", 1, 1, 512, 64, 16, 16, 32, "bf16", False),
    ("bf16-hash-d128", 1, 2, 1024, 128, 256, 3, 64, "bf16", False),
    ("bf16-hash-d32", 1, 1, 1024, 32, 128, 2, 32, "bf16", False),
    ("bf16-hash-ragged", 1, 1, 1000, 64, 128, 2, 8, "bf16", False),
    ("bf16-nh12-d128", 1, 1, 1024, 128, 32, 12, 64, "bf16", False),
    ("bf16-nh10-d64", 1, 2, 512, 64, 16, 10, 32, "bf16", False),
    ("bf16-nh6", 1, 1, 1024, 128, 64, 6, 128, "bf16", False),
    # persistent runs whose last one is short (40 tiles per segment in runs of 3; 50 in runs of 4;
    # 50 in runs of 13, two runs per CU, eight rounds); with m = 32 and ~20 rows per bucket, some
    # key tiles are reached by no query block past their own four
    ("bf16-ragged-runs", 1, 8, 5120, 64, 64, 2, 128, "bf16", False),
    ("bf16-ragged-runs-d128", 1, 4, 6400, 128, 64, 4, 128, "bf16", False),
    ("bf16-split-runs-nh8", 2, 8, 6400, 64, 64, 8, 128, "bf16", False),
    ("bf16-ragged-runs-m32", 1, 8, 5120, 64, 256, 2, 32, "bf16", False),
]


def _small_cfg(case):
    name, B, H, L, d, nb, nh, m, dt, cl = case
    return gen.Config(name, B, H, L, d, nb, nh, m, dt, cl, True, 100 + SMALL.index(case), n_clusters=16)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes_match_oracle(case):
    cfg = _small_cfg(case)
    gu.say(f"[gpu] small case {cfg}")
    x = gen.generate(cfg)
    res = gu.run_gpu(x)
    gu.check_sort_properties(res, cfg)
    gu.compare_slices(x, res, [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)])


# head dim, buckets: nb/2 a multiple of 64 runs the pipelined hash kernel (slot search deferred to
# the end of each round), the others the per-tile search
TIES = [(128, 1024), (64, 1024), (32, 128), (64, 192), (128, 96), (64, 4096)]


@pytest.mark.parametrize("d,nb", TIES, ids=[f"d{d}-nb{nb}" for d, nb in TIES])
def test_hash_first_index_on_exact_ties(d, nb):
    # rotations made of a few base columns repeated with signs: many entries of
    # [qR ; -qR] are exactly equal, inside a 32-column tile, across tiles and
    # in both halves; the first index must win, as in the oracle
    import lsh_sparse_attention_amd as lsh
    L, nh = 1000, 3
    x = gen.generate_tied_rotation(21 + d + nb, L, d, nb, nh)
    gu.say(f"[gpu] hash on exact ties d={d} nb={nb} L={L} nh={nh}")
    prob = lsh.problem(1, 1, L, d, nh, nb, 8, dtype="bf16")
    q = gu.to_device(x["q"], "bf16").view(1, 1, L, d)
    rot = gu.to_device(x["rot"], "bf16")
    bk = torch.full((1, 1, nh, L), -1, dtype=torch.int32, device="cuda")
    lsh.lsh_hash(prob, q, rot, bk)
    torch.cuda.synchronize()
    want = ora.hash_(gen.to_f64(x["q"], "bf16"), x["rot64"], nb)
    got = bk.cpu().numpy()[0, 0]
    assert np.array_equal(got, want), f"{int((got != want).sum())} of {got.size} buckets differ"


_CACHE = {}


def _full(name):
    if name not in _CACHE:
        _CACHE.clear()
        cfg = gen.CONFIGS[name]
        gu.say(f"[gpu] generating {name}: {cfg}")
        _CACHE[name] = gen.generate(cfg, with_grad=True)
    return _CACHE[name]


SAMPLES = {
    "tiny": [(0, 0)],
    "mid": [(0, 0), (7, 5)],
    "image": [(0, 3)],
    "text": [(0, 6)],
    "stress": [(3, 1)],
}


@pytest.mark.parametrize("name", list(SAMPLES))
def test_workload_shapes_match_oracle(name):
    x = _full(name)
    cfg = x["cfg"]
    gu.say(f"[gpu] full-size {name}: running the library")
    res = gu.run_gpu(x)
    gu.check_sort_properties(res, cfg)
    gu.say(f"[gpu] full-size {name}: oracle on slices {SAMPLES[name]}")
    gu.compare_slices(x, res, SAMPLES[name])
    # the first token of every slice attends only to itself
    assert np.array_equal(res["out"][:, :, 0], gen.to_f64(x["v"][:, :, 0], cfg.dtype))
    # buckets, perm, inv and win_lo of every (b, h) slice against the oracle's hash and sort
    gu.say(f"[gpu] full-size {name}: oracle hash and sort on all {cfg.batch * cfg.heads} slices")
    gu.compare_hash_sort_all_slices(x, res)


def test_maximum_segment_count():
    """B*H*n_hashes = 65528 (segments are capped at 65535): the grids that index segments or heads
    run at their largest; every segment's sort is checked and three heads against the oracle."""
    cfg = gen.Config("max-segments", 1, 8191, 128, 64, 8, 8, 32, "bf16", False, True, 901, n_clusters=16)
    gu.say(f"[gpu] maximum segment count: {cfg}")
    x = gen.generate(cfg, with_grad=True)
    res = gu.run_gpu(x)
    gu.check_sort_properties(res, cfg)
    gu.compare_slices(x, res, [(0, 0), (0, 4095), (0, 8190)])


def test_rounds_combine_to_output():
    cfg = _small_cfg(SMALL[1])
    gu.say(f"[gpu] combine identity {cfg}")
    x = gen.generate(cfg)
    res = gu.run_gpu(x, backward=False, rounds=True)
    lr = res["lse_rounds"]                       # [B,H,nh,L]
    mx = lr.max(axis=2, keepdims=True)
    alone = ~np.isfinite(mx[:, :, 0])
    mx = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(lr - mx)
    den = np.where(alone, 1.0, w.sum(axis=2))
    lse = mx[:, :, 0] + np.log(den)
    out = (w[..., None] * res["o_rounds"]).sum(axis=2) / den[..., None]
    v = gen.to_f64(x["v"], cfg.dtype)
    out = np.where(alone[..., None], v, out)
    gu.assert_close("combine", res["out"], out, 2e-2)
    gu.assert_close("lse", res["lse"][~alone], lse[~alone], 1e-5)


def test_deterministic():
    cfg = _small_cfg(SMALL[13])
    gu.say(f"[gpu] determinism {cfg}")
    x = gen.generate(cfg)
    a = gu.run_gpu(x)
    b = gu.run_gpu(x)
    for k in ("buckets", "perm", "inv", "win_lo", "out", "lse", "dq", "dv"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("idx", [1, 0, 2, 17, 19, 13, 21])
def test_backward_entry_points_match_oracle(idx):
    # lsh_attn_bwd_saved, lsh_attn_bwd (records derived again from perm, inv,
    # win_lo) and lsh_attn_bwd_rehash (buckets, order and windows recomputed
    # from q and rot): each one's dq and dv against the oracle, and the three
    # bit for bit against one another
    cfg = _small_cfg(SMALL[idx])
    gu.say(f"[gpu] backward entry points {cfg}")
    x = gen.generate(cfg)
    res = gu.run_gpu_backward_entries(x)
    gu.compare_backward_entries(x, res, [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)])


BWD_FULL = {"text": [(0, 5)], "stress": [(2, 6)]}


@pytest.mark.parametrize("name", list(BWD_FULL))
def test_backward_entry_points_at_workload_size(name):
    # the standalone and rehash backwards at full size (the rehash path hashes
    # and sorts every (b, h, round) segment inside the call), against the oracle
    x = _full(name)
    gu.say(f"[gpu] backward entry points, full-size {name}: running the library")
    res = gu.run_gpu_backward_entries(x)
    gu.say(f"[gpu] backward entry points, full-size {name}: oracle on slices {BWD_FULL[name]}")
    gu.compare_backward_entries(x, res, BWD_FULL[name])


# ----------------------------------------------------------------------------- non-causal
# Encoder (non-causal) sets: same bucket, own chunk or the one before, no
# "not after the query" condition.  bf16 problems whose chunk length divides
# 128 run on the matrix-core stream kernels; the others (fp32, other chunk
# lengths, lengths not a multiple of 128) on the per-query kernels.

# name, B, H, L, d, nb, nh, m, dtype, clustered
NC_SMALL = [
    ("nc-f32-base", 1, 2, 1024, 64, 16, 3, 32, "f32", False),
    ("nc-f32-d32", 1, 1, 512, 32, 8, 2, 16, "f32", False),
    ("nc-f32-d128", 1, 1, 1024, 128, 64, 2, 64, "f32", False),
    ("nc-f32-one-chunk", 1, 1, 256, 64, 8, 2, 256, "f32", False),
    ("nc-f32-chunk-1", 1, 1, 128, 32, 4, 2, 1, "f32", False),
    ("nc-f32-two-buckets", 1, 2, 512, 64, 2, 2, 32, "f32", False),
    ("nc-tiny-L", 1, 1, 8, 32, 4, 2, 2, "f32", False),
    ("nc-single-token", 1, 1, 1, 32, 2, 1, 1, "f32", False),
    ("nc-bf16-base", 2, 2, 1024, 64, 16, 3, 32, "bf16", False),
    ("nc-bf16-d128", 1, 2, 2048, 128, 32, 2, 64, "bf16", False),
    ("nc-bf16-one-round", 1, 2, 1024, 64, 32, 1, 64, "bf16", False),
    ("nc-bf16-m128", 1, 4, 4096, 64, 64, 2, 128, "bf16", False),
    ("nc-bf16-m8", 1, 1, 1024, 64, 128, 2, 8, "bf16", False),
    ("nc-bf16-m1", 1, 2, 512, 64, 8, 2, 1, "bf16", False),
    ("nc-bf16-nh6", 1, 1, 1024, 128, 64, 6, 128, "bf16", False),
    ("nc-bf16-nh12-d128", 1, 1, 1024, 128, 32, 12, 64, "bf16", False),
    ("nc-bf16-nh16", 1, 1, 512, 64, 16, 16, 32, "bf16", False),
    ("nc-bf16-clustered", 1, 2, 2048, 64, 64, 4, 64, "bf16", True),
    ("nc-bf16-clustered-d128", 1, 1, 2048, 128, 64, 8, 128, "bf16", True),
    ("nc-bf16-m96", 1, 2, 1536, 64, 32, 3, 96, "bf16", False),
    ("nc-bf16-m256", 1, 1, 2048, 128, 16, 2, 256, "bf16", False),
    ("nc-bf16-ragged", 1, 2, 2016, 64, 64, 2, 32, "bf16", False),
    ("nc-bf16-d32", 1, 2, 512, 32, 8, 2, 16, "bf16", False),
]


def _nc_cfg(case):
    name, B, H, L, d, nb, nh, m, dt, cl = case
    return gen.Config(name, B, H, L, d, nb, nh, m, dt, cl, True, 300 + NC_SMALL.index(case), n_clusters=16,
                      causal=False)


@pytest.mark.parametrize("case", NC_SMALL, ids=[c[0] for c in NC_SMALL])
def test_noncausal_small_shapes_match_oracle(case):
    cfg = _nc_cfg(case)
    gu.say(f"[gpu] non-causal small case {cfg}")
    x = gen.generate(cfg)
    res = gu.run_gpu(x)
    gu.check_sort_properties(res, cfg)
    gu.compare_slices(x, res, [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)])


NC_SAMPLES = {"image": [(0, 5)], "text": [(0, 2)]}


@pytest.mark.parametrize("name", list(NC_SAMPLES))
def test_noncausal_workload_shapes_match_oracle(name):
    # the same inputs as the causal full-size case, non-causal sets
    x = dict(_full(name))
    x["cfg"] = x["cfg"].with_(causal=False)
    gu.say(f"[gpu] non-causal full-size {name}: running the library")
    res = gu.run_gpu(x)
    gu.check_sort_properties(res, x["cfg"])
    gu.say(f"[gpu] non-causal full-size {name}: oracle on slices {NC_SAMPLES[name]}")
    gu.compare_slices(x, res, NC_SAMPLES[name])


@pytest.mark.parametrize("idx", [0, 8, 9, 15, 19])
def test_noncausal_backward_entry_points_match_oracle(idx):
    cfg = _nc_cfg(NC_SMALL[idx])
    gu.say(f"[gpu] non-causal backward entry points {cfg}")
    x = gen.generate(cfg)
    res = gu.run_gpu_backward_entries(x)
    gu.compare_backward_entries(x, res, [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)])


# ----------------------------------------------------------------------------- no bucket mask
# LSH_FLAG_NO_BUCKET_MASK: the chunks of the sorted order alone restrict
# attention (causal: positions not after the query; non-causal: all).

# name, B, H, L, d, nb, nh, m, dtype, clustered, causal
NB_SMALL = [
    ("nb-f32-causal", 1, 2, 1024, 64, 16, 3, 32, "f32", False, True),
    ("nb-f32-noncausal", 1, 1, 512, 32, 8, 2, 16, "f32", False, False),
    ("nb-f32-d128-m1", 1, 1, 256, 128, 8, 2, 1, "f32", False, True),
    ("nb-f32-one-chunk", 1, 1, 256, 64, 8, 2, 256, "f32", False, True),
    ("nb-tiny-L", 1, 1, 8, 32, 4, 2, 2, "f32", False, True),
    ("nb-single-token", 1, 1, 1, 32, 2, 1, 1, "f32", False, True),
    ("nb-bf16-causal", 2, 2, 1024, 64, 16, 3, 32, "bf16", False, True),
    ("nb-bf16-causal-d128", 1, 2, 2048, 128, 32, 2, 64, "bf16", False, True),
    ("nb-bf16-causal-m128", 1, 2, 4096, 64, 64, 1, 128, "bf16", False, True),
    ("nb-bf16-causal-m8", 1, 1, 1024, 64, 128, 2, 8, "bf16", False, True),
    ("nb-bf16-causal-nh8", 1, 1, 1024, 128, 64, 8, 128, "bf16", False, True),
    ("nb-bf16-causal-nh14", 1, 1, 512, 64, 16, 14, 32, "bf16", False, True),
    ("nb-bf16-noncausal", 1, 2, 2048, 64, 32, 3, 64, "bf16", False, False),
    ("nb-bf16-noncausal-d128-nh12", 1, 1, 1024, 128, 32, 12, 64, "bf16", False, False),
    ("nb-bf16-clustered", 1, 2, 2048, 64, 64, 4, 64, "bf16", True, True),
    ("nb-bf16-m96", 1, 2, 1536, 64, 32, 3, 96, "bf16", False, True),
    ("nb-bf16-ragged-noncausal", 1, 1, 2016, 64, 64, 2, 32, "bf16", False, False),
]


def _nb_cfg(case):
    name, B, H, L, d, nb, nh, m, dt, cl, causal = case
    return gen.Config(name, B, H, L, d, nb, nh, m, dt, cl, True, 500 + NB_SMALL.index(case), n_clusters=16,
                      causal=causal, bucket_mask=False)


@pytest.mark.parametrize("case", NB_SMALL, ids=[c[0] for c in NB_SMALL])
def test_no_bucket_mask_small_shapes_match_oracle(case):
    cfg = _nb_cfg(case)
    gu.say(f"[gpu] no-bucket-mask small case {cfg}")
    x = gen.generate(cfg)
    res = gu.run_gpu(x)
    gu.check_sort_properties(res, cfg)
    gu.compare_slices(x, res, [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)])


@pytest.mark.parametrize("name,causal,sl", [("text", True, (0, 4)), ("image", False, (0, 1))])
def test_no_bucket_mask_workload_shapes_match_oracle(name, causal, sl):
    x = dict(_full(name))
    x["cfg"] = x["cfg"].with_(causal=causal, bucket_mask=False)
    gu.say(f"[gpu] no-bucket-mask full-size {name} causal={causal}: running the library")
    res = gu.run_gpu(x)
    gu.say(f"[gpu] no-bucket-mask full-size {name}: oracle on slice {sl}")
    gu.compare_slices(x, res, [sl])


@pytest.mark.parametrize("idx", [0, 5, 7, 11, 14])
def test_no_bucket_mask_backward_entry_points_match_oracle(idx):
    cfg = _nb_cfg(NB_SMALL[idx])
    gu.say(f"[gpu] no-bucket-mask backward entry points {cfg}")
    x = gen.generate(cfg)
    res = gu.run_gpu_backward_entries(x)
    gu.compare_backward_entries(x, res, [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)])


# ----------------------------------------------------------------------------- duplicates by bucket
# LSH_FLAG_DUP_BY_BUCKET: a member attended in k rounds weighs k / N, N =
# rounds sharing the query's bucket.  Few buckets and short chunks (and the
# clustered inputs) cut buckets by the window, where this differs from the
# default count.

# name, B, H, L, d, nb, nh, m, dtype, clustered, causal
DB_SMALL = [
    ("db-f32", 1, 2, 1024, 64, 8, 3, 16, "f32", False, True),
    ("db-f32-noncausal", 1, 1, 512, 32, 4, 2, 8, "f32", False, False),
    ("db-tiny-L", 1, 1, 8, 32, 4, 2, 2, "f32", False, True),
    ("db-single-token", 1, 1, 1, 32, 2, 2, 1, "f32", False, True),
    ("db-bf16", 2, 2, 1024, 64, 8, 3, 16, "bf16", False, True),
    ("db-bf16-d128", 1, 2, 2048, 128, 16, 2, 32, "bf16", False, True),
    ("db-bf16-d128-nh4", 1, 1, 2048, 128, 16, 4, 32, "bf16", False, True),
    ("db-bf16-nh8", 1, 1, 1024, 64, 16, 8, 32, "bf16", False, True),
    ("db-bf16-nh14-d128", 1, 1, 1024, 128, 16, 14, 64, "bf16", False, True),
    ("db-bf16-noncausal", 1, 2, 2048, 64, 16, 3, 32, "bf16", False, False),
    ("db-bf16-noncausal-d128-nh12", 1, 1, 1024, 128, 16, 12, 64, "bf16", False, False),
    ("db-bf16-clustered", 1, 2, 2048, 64, 64, 4, 64, "bf16", True, True),
    ("db-bf16-m96", 1, 2, 1536, 64, 8, 3, 96, "bf16", False, True),
    ("db-bf16-one-round", 1, 2, 1024, 64, 8, 1, 32, "bf16", False, True),
]


def _db_cfg(case):
    name, B, H, L, d, nb, nh, m, dt, cl, causal = case
    return gen.Config(name, B, H, L, d, nb, nh, m, dt, cl, True, 700 + DB_SMALL.index(case), n_clusters=16,
                      causal=causal, dup_by_bucket=True)


@pytest.mark.parametrize("case", DB_SMALL, ids=[c[0] for c in DB_SMALL])
def test_dup_by_bucket_small_shapes_match_oracle(case):
    cfg = _db_cfg(case)
    gu.say(f"[gpu] dup-by-bucket small case {cfg}")
    x = gen.generate(cfg)
    res = gu.run_gpu(x)
    gu.compare_slices(x, res, [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)])


def test_dup_by_bucket_stress_workload_matches_oracle():
    # the clustered 64K workload: buckets of ~256 rows overflow the window
    x = dict(_full("stress"))
    x["cfg"] = x["cfg"].with_(dup_by_bucket=True)
    gu.say("[gpu] dup-by-bucket full-size stress: running the library")
    res = gu.run_gpu(x)
    gu.say("[gpu] dup-by-bucket full-size stress: oracle on slice (1, 2)")
    gu.compare_slices(x, res, [(1, 2)])


@pytest.mark.parametrize("idx", [0, 3, 5, 9, 10])
def test_dup_by_bucket_backward_entry_points_match_oracle(idx):
    cfg = _db_cfg(DB_SMALL[idx])
    gu.say(f"[gpu] dup-by-bucket backward entry points {cfg}")
    x = gen.generate(cfg)
    res = gu.run_gpu_backward_entries(x)
    gu.compare_backward_entries(x, res, [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)])


def test_empty_problem_is_a_no_op():
    import lsh_sparse_attention_amd as lsh
    gu.say("[gpu] empty problem L=0")
    p = lsh.problem(1, 2, 0, 64, 2, 16, 32, dtype="bf16")
    att = lsh.LshAttention(p)
    q = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    rot = torch.randn((2, 64, 8), device="cuda").to(torch.bfloat16)
    out, lse = att.forward(q, q, rot)
    dq, dv = att.backward(q, q, q)
    torch.cuda.synchronize()
    assert out.shape == (1, 2, 0, 64) and lse.shape == (1, 2, 0) and dq.numel() == 0 and dv.numel() == 0
