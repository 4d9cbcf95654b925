"""Host-side checks of the C ABI: the library loads without a GPU, exports
every symbol that include/lsh.h declares, and validates arguments before
launching anything (all calls here return before touching a device)."""
import ctypes
import os
import re

import pytest

from lsh_sparse_attention_amd import _lib
import lsh_sparse_attention_amd as lsh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "lsh.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(lsh_[a-z_]+)\s*\(", src))


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    declared = _declared()
    assert declared == set(_lib.SYMBOLS)
    for name in declared:
        assert hasattr(L, name)


def test_status_strings_and_version():
    L = _lib.lib()
    assert L.lsh_version() >= 100
    assert L.lsh_status_string(0) == b"ok"
    assert b"unsupported" in L.lsh_status_string(2)
    assert L.lsh_status_string(99) == b"unknown status"


def _prob(**kw):
    base = dict(batch=1, heads=2, seq_len=256, head_dim=64, n_hashes=2, n_buckets=16, chunk_len=32)
    base.update(kw)
    return lsh.problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(n_buckets=15), 1), (dict(n_buckets=0), 1), (dict(chunk_len=48), 1), (dict(seq_len=-256), 1),
    (dict(batch=-1), 1), (dict(chunk_len=0), 1),
    (dict(head_dim=48), 2), (dict(seq_len=65536 * 2, chunk_len=64), 2), (dict(n_hashes=17), 2),
    (dict(batch=4096, heads=8, n_hashes=2, seq_len=64), 2),
    (dict(n_buckets=8192), 2),
])
def test_invalid_problems_rejected_before_launch(kw, status):
    p = _prob(**kw)
    L = _lib.lib()
    dummy = ctypes.c_void_p(256)
    assert L.lsh_hash(ctypes.byref(p), dummy, dummy, dummy, None) == status
    assert L.lsh_workspace_bytes(ctypes.byref(p), 0) == 0


@pytest.mark.parametrize("kw", [dict(seq_len=0), dict(batch=0), dict(heads=0)])
def test_empty_problems_are_no_ops(kw):
    # null pointers and a null workspace are fine: nothing is read or launched
    p = _prob(**kw)
    L = _lib.lib()
    for k in (0, 1, 2, 3, 4):
        assert L.lsh_workspace_bytes(ctypes.byref(p), k) == 0
    n = None
    assert L.lsh_hash(ctypes.byref(p), n, n, n, n) == 0
    assert L.lsh_sort(ctypes.byref(p), n, n, n, n, n, ctypes.c_size_t(0), n) == 0
    assert L.lsh_attn_fwd(ctypes.byref(p), n, n, n, n, n, n, n, n, ctypes.c_size_t(0), n) == 0
    assert L.lsh_combine(ctypes.byref(p), n, n, n, n, n, n, n) == 0
    assert L.lsh_attn_bwd(ctypes.byref(p), n, n, n, n, n, n, n, n, n, n, n, ctypes.c_size_t(0), n) == 0
    assert L.lsh_attn_bwd_saved(ctypes.byref(p), n, n, n, n, n, n, n, n, ctypes.c_size_t(0), n) == 0
    assert L.lsh_attn_bwd_rehash(ctypes.byref(p), n, n, n, n, n, n, n, n, n, ctypes.c_size_t(0), n) == 0
    # an empty problem is still validated: a bad head size is reported
    bad = _prob(head_dim=48, **kw)
    assert L.lsh_hash(ctypes.byref(bad), n, n, n, n) == 2


def test_causal_flag_values():
    # 1 (causal) and 0 (non-causal) are valid; anything else is malformed and
    # rejected before any pointer is looked at
    L = _lib.lib()
    p = _prob()
    p.causal = 2
    dummy = ctypes.c_void_p(256)
    assert L.lsh_hash(ctypes.byref(p), dummy, dummy, dummy, None) == 1
    assert L.lsh_workspace_bytes(ctypes.byref(p), 1) == 0
    c, n = _prob(), _prob()
    n.causal = 0
    # the non-causal forward keeps one more 32-bit record per (token, round)
    rnd = c.batch * c.heads * c.seq_len * c.n_hashes
    extra = (rnd * 4 + 255) // 256 * 256
    for kind in (1, 2, 3):
        assert L.lsh_workspace_bytes(ctypes.byref(n), kind) == L.lsh_workspace_bytes(ctypes.byref(c), kind) + extra
    assert L.lsh_workspace_bytes(ctypes.byref(n), 0) == L.lsh_workspace_bytes(ctypes.byref(c), 0)


def test_flags_values():
    L = _lib.lib()
    dummy = ctypes.c_void_p(256)
    for bad in (4, 3, -1):           # an unknown bit; both set flags together
        p = _prob()
        p.flags = bad
        assert L.lsh_hash(ctypes.byref(p), dummy, dummy, dummy, None) == 1
        assert L.lsh_workspace_bytes(ctypes.byref(p), 1) == 0
    c = _prob()
    rnd = c.batch * c.heads * c.seq_len * c.n_hashes
    a256 = lambda x: (x + 255) // 256 * 256
    # without the bucket condition: window records, and for causal problems
    # also the lone flags (one byte per token-round) and per-chunk minima
    nbc = _prob(bucket_mask=False)
    extra = a256(rnd * 4) + a256(rnd) + a256(rnd // c.chunk_len * 4)
    nbn = _prob(bucket_mask=False, causal=False)
    # duplicates counted over buckets: the bucket-run starts per token-round
    # and one scratch word per 1024 sorted rows of each (b, h, round)
    dup = _prob(dup_by_bucket=True)
    segs = c.batch * c.heads * c.n_hashes
    for kind in (1, 2, 3):
        base = L.lsh_workspace_bytes(ctypes.byref(c), kind)
        assert L.lsh_workspace_bytes(ctypes.byref(nbc), kind) == base + extra
        assert L.lsh_workspace_bytes(ctypes.byref(nbn), kind) == base + a256(rnd * 4)
        assert L.lsh_workspace_bytes(ctypes.byref(dup), kind) == (
            base + a256(rnd * 4) + a256(segs * ((c.seq_len + 1023) // 1024) * 4))


def test_null_and_misaligned_pointers_rejected():
    p = _prob()
    L = _lib.lib()
    ok = ctypes.c_void_p(1 << 20)
    assert L.lsh_hash(ctypes.byref(p), None, ok, ok, None) == 1
    assert L.lsh_hash(ctypes.byref(p), ctypes.c_void_p((1 << 20) + 2), ok, ok, None) == 1
    ws = L.lsh_workspace_bytes(ctypes.byref(p), _lib.LSH_WS_SORT)
    assert ws > 0
    # too small a workspace, or one that is not 256-byte aligned
    assert L.lsh_sort(ctypes.byref(p), ok, ok, ok, ok, ok, ctypes.c_size_t(ws - 1), None) == 1
    assert L.lsh_sort(ctypes.byref(p), ok, ok, ok, ok, ctypes.c_void_p((1 << 20) + 16), ctypes.c_size_t(ws),
                      None) == 1
    assert L.lsh_attn_fwd(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, None, ctypes.c_size_t(0), None) == 1
    assert L.lsh_attn_bwd(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, ctypes.c_size_t(1),
                          None) == 1
    assert L.lsh_combine(ctypes.byref(p), ok, ok, None, ok, ok, ok, None) == 1
    assert L.lsh_attn_fwd(None, ok, ok, ok, ok, ok, ok, ok, ok, ctypes.c_size_t(1 << 30), None) == 1


def test_saved_backward_workspace_and_arguments():
    # the shared workspace holds the forward's records at the forward's offsets and the backward's scratch
    p = _prob()
    L = _lib.lib()
    fwd = lsh.workspace_bytes(p, _lib.LSH_WS_FWD)
    train = lsh.workspace_bytes(p, _lib.LSH_WS_TRAIN)
    assert train == lsh.workspace_bytes(p, _lib.LSH_WS_BWD) and train > fwd > 0
    assert L.lsh_workspace_bytes(ctypes.byref(p), 5) == 0
    ok = ctypes.c_void_p(1 << 20)
    args = [ok] * 7
    assert L.lsh_attn_bwd_saved(ctypes.byref(p), *args, ok, ctypes.c_size_t(train - 1), None) == 1
    assert L.lsh_attn_bwd_saved(ctypes.byref(p), *args, None, ctypes.c_size_t(train), None) == 1
    assert L.lsh_attn_bwd_saved(ctypes.byref(p), *args, ctypes.c_void_p((1 << 20) + 128), ctypes.c_size_t(train),
                                None) == 1
    assert L.lsh_attn_bwd_saved(ctypes.byref(p), None, *args[1:], ok, ctypes.c_size_t(train), None) == 1
    assert L.lsh_attn_bwd_saved(None, *args, ok, ctypes.c_size_t(train), None) == 1
    # the standalone backward still wants the sort's outputs
    assert L.lsh_attn_bwd(ctypes.byref(p), ok, ok, ok, ok, ok, None, ok, ok, ok, ok, ok, ctypes.c_size_t(train),
                          None) == 1


def test_rehash_backward_workspace_and_arguments():
    # the rehash workspace holds the backward's, the recomputed sort outputs and the sort's scratch
    p = _prob()
    L = _lib.lib()
    rehash = lsh.workspace_bytes(p, _lib.LSH_WS_REHASH)
    rnd = p.batch * p.heads * p.n_hashes * p.seq_len
    assert rehash >= lsh.workspace_bytes(p, _lib.LSH_WS_BWD) + 4 * rnd * 4 + lsh.workspace_bytes(p, _lib.LSH_WS_SORT)
    ok = ctypes.c_void_p(1 << 20)
    args = [ok] * 8   # q, v, rot, out, dout, lse, dq, dv
    sz = ctypes.c_size_t(rehash)
    assert L.lsh_attn_bwd_rehash(ctypes.byref(p), *args, ok, ctypes.c_size_t(rehash - 1), None) == 1
    assert L.lsh_attn_bwd_rehash(ctypes.byref(p), *args, None, sz, None) == 1
    assert L.lsh_attn_bwd_rehash(ctypes.byref(p), *args, ctypes.c_void_p((1 << 20) + 64), sz, None) == 1
    assert L.lsh_attn_bwd_rehash(ctypes.byref(p), ok, ok, None, *args[3:], ok, sz, None) == 1          # rot
    assert L.lsh_attn_bwd_rehash(ctypes.byref(p), ok, ok, ctypes.c_void_p((1 << 20) + 2), *args[3:], ok, sz,
                                 None) == 1
    assert L.lsh_attn_bwd_rehash(ctypes.byref(p), *args[:6], None, ok, ok, sz, None) == 1                # dq
    bad = _prob(head_dim=48)
    assert L.lsh_attn_bwd_rehash(ctypes.byref(bad), *args, ok, sz, None) == 2


def test_workspace_sizes_grow_with_problem():
    small = _prob()
    big = _prob(batch=4)
    for k in (0, 1, 2, 3, 4):
        assert 0 < lsh.workspace_bytes(small, k) < lsh.workspace_bytes(big, k)
        assert lsh.workspace_bytes(small, k) % 256 == 0


def test_kernel_names_and_profile_hook():
    L = _lib.lib()
    names = [L.lsh_kernel_name(k).decode() for k in range(len(_lib.KERNELS))]
    assert tuple(names) == _lib.KERNELS
    assert L.lsh_kernel_name(len(_lib.KERNELS)) is None
    assert L.lsh_profile_kernel(len(_lib.KERNELS), None, None) == 1
    assert L.lsh_profile_kernel(0, None, None) == 0      # clearing needs no GPU


def test_ff_descriptions_validated_without_launching():
    L = _lib.lib()
    dummy = ctypes.c_void_p(256)
    ok = lsh.ff_problem(100, 64, 256, 2)
    assert L.lsh_ff_workspace_bytes(ctypes.byref(ok), 0) > 0
    assert L.lsh_ff_workspace_bytes(ctypes.byref(ok), 1) > L.lsh_ff_workspace_bytes(ctypes.byref(ok), 0)
    for bad, status in ((lsh.ff_problem(100, 60, 256, 2), 1), (lsh.ff_problem(100, 64, 250, 2), 1),
                        (lsh.ff_problem(100, 64, 256, 0), 1), (lsh.ff_problem(-1, 64, 256, 1), 1)):
        assert L.lsh_ff_workspace_bytes(ctypes.byref(bad), 0) == 0
        assert L.lsh_ff_fwd(ctypes.byref(bad), dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                            ctypes.c_size_t(1 << 30), None) == status
    f32 = lsh.ff_problem(100, 64, 256, 2)
    f32.dtype = 0
    assert L.lsh_ff_fwd(ctypes.byref(f32), dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                        ctypes.c_size_t(1 << 30), None) == 2
    # null pointers and a short workspace are rejected before anything runs
    assert L.lsh_ff_fwd(ctypes.byref(ok), None, dummy, dummy, dummy, dummy, dummy, dummy,
                        ctypes.c_size_t(1 << 30), None) == 1
    assert L.lsh_ff_fwd(ctypes.byref(ok), dummy, dummy, dummy, dummy, dummy, dummy, dummy, ctypes.c_size_t(16),
                        None) == 1
    empty = lsh.ff_problem(0, 64, 256, 2)
    assert L.lsh_ff_workspace_bytes(ctypes.byref(empty), 1) == 0
    assert L.lsh_ff_bwd(ctypes.byref(empty), None, None, None, None, None, None, None, None, None, None, None,
                        ctypes.c_size_t(0), None) == 0


def test_sort_noalloc_arguments_and_limit():
    # lsh_sort_noalloc validates like lsh_sort and rejects problems whose count
    # matrix exceeds the static scratch, all before anything is launched
    L = _lib.lib()
    ok = ctypes.c_void_p(1 << 20)
    p = _prob()
    assert L.lsh_sort_noalloc(ctypes.byref(p), None, ok, ok, ok, None) == _lib.LSH_ERR_INVALID
    assert L.lsh_sort_noalloc(ctypes.byref(p), ok, ok, None, ok, None) == _lib.LSH_ERR_INVALID
    assert L.lsh_sort_noalloc(None, ok, ok, ok, ok, None) == _lib.LSH_ERR_INVALID
    empty = lsh.problem(1, 2, 0, 64, 2, 16, 32, dtype="bf16")
    assert L.lsh_sort_noalloc(ctypes.byref(empty), None, None, None, None, None) == _lib.LSH_OK
    # 8 x 16 x 8 segments of 16 tiles x 4096 buckets x 2 bytes = 128 MiB of counts
    big = lsh.problem(8, 16, 65536, 64, 8, 4096, 128, dtype="bf16")
    assert L.lsh_workspace_bytes(ctypes.byref(big), _lib.LSH_WS_SORT) > _lib.LSH_SORT_NOALLOC_MAX_BYTES
    assert L.lsh_sort_noalloc(ctypes.byref(big), ok, ok, ok, ok, None) == _lib.LSH_ERR_UNSUPPORTED
    # the text-shaped problem fits
    text = lsh.problem(1, 8, 65536, 128, 4, 1024, 128, dtype="bf16")
    assert 0 < L.lsh_workspace_bytes(ctypes.byref(text), _lib.LSH_WS_SORT) <= _lib.LSH_SORT_NOALLOC_MAX_BYTES
