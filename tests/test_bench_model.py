"""The bench's algorithmic work model, checked against brute-force counts on small problems.

The roofline figures divide these counts by measured kernel times, so a wrong count would
misstate every fraction of peak.  Reformer §2 (chunked attention over the sorted order): each
chunk of m sorted rows attends to itself and to the chunk before it; the first chunk has no
predecessor.  §2 (random projections): one rotation of nb/2 columns per round.
"""
import os
import sys
from types import SimpleNamespace

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def cfg(**kw):
    base = dict(batch=2, heads=3, seq_len=512, head_dim=64, n_hashes=2, n_buckets=16, chunk_len=64, dtype="bf16")
    base.update(kw)
    return SimpleNamespace(**base)


def brute_pairs(L, m):
    """(query, key) pairs of the dense chunk tiles, enumerated chunk by chunk."""
    n = 0
    for c in range(L // m):
        keys = m * (2 if c > 0 else 1)
        for _ in range(m):
            n += keys
    return n


def test_chunk_tile_flops_match_enumeration():
    for L, m in ((512, 64), (1024, 128), (256, 256), (96, 32)):
        c = cfg(seq_len=L, chunk_len=m)
        rows = c.batch * c.heads * c.n_hashes
        pairs = brute_pairs(L, m) * rows
        flops, _ = bench.algorithmic_work("attn_fwd", c)
        # two products of d multiply-adds per pair (scores and the weighted sum of values)
        assert flops == 2 * 2 * c.head_dim * pairs
        flops_dq, _ = bench.algorithmic_work("bwd_dq", c)
        flops_dkv, _ = bench.algorithmic_work("bwd_dkv", c)
        assert flops_dq == 3 * 2 * c.head_dim * pairs
        assert flops_dkv == 4 * 2 * c.head_dim * pairs


def test_hash_flops_match_enumeration():
    c = cfg()
    n = 0
    for _ in range(c.batch * c.heads * c.seq_len):      # every token ...
        for _ in range(c.n_hashes):                     # ... in every round ...
            n += (c.n_buckets // 2) * c.head_dim        # ... projected on nb/2 rotation columns
    flops, nbytes = bench.algorithmic_work("hash", c)
    assert flops == 2 * n
    # q read once, the rotation read once, one int32 bucket per token and round written
    T = c.batch * c.heads * c.seq_len
    assert nbytes == T * c.head_dim * 2 + c.n_hashes * c.head_dim * (c.n_buckets // 2) * 2 + T * c.n_hashes * 4


def test_byte_counts_scale_with_element_size():
    b16 = bench.algorithmic_work("combine", cfg(dtype="bf16"))[1]
    f32 = bench.algorithmic_work("combine", cfg(dtype="f32"))[1]
    c = cfg()
    T = c.batch * c.heads * c.seq_len
    # every row's d elements, rounds in and one out, grow by 2 bytes each from bf16 to fp32
    assert f32 - b16 == (T * c.n_hashes + T) * c.head_dim * 2


def test_kernel_table_skips_kernels_that_did_not_run():
    c = cfg()
    table = bench.kernel_rooflines({"hash": 10.0, "combine": 5.0}, c, None)
    assert set(table) == {"hash", "combine"}
    assert "tflops" in table["hash"] and "frac_of_gemm" not in table["hash"]
    assert "tflops" not in table["combine"]
    t2 = bench.kernel_rooflines({"hash": 10.0}, c, 1000.0)
    assert t2["hash"]["frac_of_gemm"] == round(t2["hash"]["tflops"] / 1000.0, 3)
    flops, nbytes = bench.algorithmic_work("hash", c)
    assert abs(t2["hash"]["gbs"] - round(nbytes / 10e-6 / 1e9, 1)) < 1e-9


def test_every_library_kernel_has_a_model():
    from lsh_sparse_attention_amd import _lib
    for k in _lib.KERNELS:
        flops, nbytes = bench.algorithmic_work(k, cfg())
        assert nbytes > 0 and flops >= 0


def test_sort_bytes_match_definition():
    # the sort reads every bucket id once per launch and writes perm, inv and win_lo once (12 bytes
    # per token-round, the scope table's unit), plus one 16-bit count per (segment, 4096-position
    # tile, bucket), written by the first launch and read by the second
    c = cfg(seq_len=10000)
    S = c.batch * c.heads * c.n_hashes
    Tr = S * c.seq_len
    tiles = -(-c.seq_len // 4096)
    cnt = S * tiles * c.n_buckets * 2
    assert bench.algorithmic_work("sort_count", c) == (0.0, Tr * 4 + cnt)
    assert bench.algorithmic_work("sort_scatter", c) == (0.0, Tr * 4 + cnt + Tr * 12)
