"""lsh_sort_noalloc (count matrix in the library's static scratch, no
workspace, nothing allocated) against lsh_sort (the caller's workspace), bit
for bit, on two calls in a row, the second on a smaller problem than the
first, so the second reads the scratch after the first has filled it."""
import numpy as np
import pytest
import torch

import lsh_sparse_attention_amd as lsh
from lsh_sparse_attention_amd import _lib
from oracle import oracle as ora
import gpu_util as gu

pytestmark = pytest.mark.gpu

# name, B, H, L, nb, nh, m, clustered bucket ids
CALLS = [("text-sized", 1, 8, 65536, 1024, 4, 128, False),
         ("smaller", 2, 3, 5000, 64, 2, 40, True)]


def _buckets(B, H, L, nb, nh, clustered, seed):
    rng = np.random.default_rng(seed)
    if clustered:   # a few heavy buckets, many empty ones
        hot = rng.integers(0, nb, size=8)
        ids = hot[rng.integers(0, 8, size=(B, H, nh, L))]
    else:
        ids = rng.integers(0, nb, size=(B, H, nh, L))
    return ids.astype(np.int32)


def test_sort_noalloc_matches_sort_twice():
    for i, (name, B, H, L, nb, nh, m, cl) in enumerate(CALLS):
        gu.say(f"[gpu] lsh_sort_noalloc vs lsh_sort, call {i + 1}: {name} B={B} H={H} L={L} nb={nb} nh={nh} m={m}")
        prob = lsh.problem(B, H, L, 64, nh, nb, m, dtype="bf16")
        assert lsh.workspace_bytes(prob, _lib.LSH_WS_SORT) <= _lib.LSH_SORT_NOALLOC_MAX_BYTES
        ids = _buckets(B, H, L, nb, nh, cl, 40 + i)
        bk = torch.from_numpy(ids).cuda()
        ws = torch.empty(lsh.workspace_bytes(prob, _lib.LSH_WS_SORT), dtype=torch.uint8, device="cuda")
        ref = [torch.full_like(bk, -7) for _ in range(3)]
        lsh.lsh_sort(prob, bk, *ref, ws)
        got = [torch.full_like(bk, -9) for _ in range(3)]
        lsh.lsh_sort_noalloc(prob, bk, *got)
        torch.cuda.synchronize()
        for what, a, b in zip(("perm", "inv", "win_lo"), got, ref):
            assert torch.equal(a, b), f"{name}: {what} differs from lsh_sort's"
        # and both against the oracle's sort on two segments
        perm = got[0].cpu().numpy()
        for (b, h) in ((0, 0), (B - 1, H - 1)):
            p, _, _ = ora.sort(ids[b, h], m)
            assert np.array_equal(perm[b, h], p), f"{name}: perm of ({b}, {h}) differs from the oracle's"
