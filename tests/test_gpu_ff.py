"""GPU parity of the chunked feed-forward layer (lsh_ff_fwd / lsh_ff_bwd,
through the C ABI) against the fp64 oracle (oracle/ff_oracle.py).

Inputs lie on the exact grid of inputs.generate_ff, so the ReLU decisions of
the kernels and the oracle agree.  Tolerance, elementwise, from the
arithmetic: the kernels round the hidden activation h (and its gradient dh)
and each output to bf16 once and accumulate in fp32, so every output stays
within 2^-8 (S + |exact|) of the exact value, S being the sum of the
absolute values of the terms it adds up (ff_oracle.abs_sums).  Chunking must
not change the forward output or dx at all (each row is computed the same
way whatever its chunk); the fp32 weight gradients, summed chunk by chunk,
agree to fp32 rounding."""
import numpy as np
import pytest
import torch

import lsh_sparse_attention_amd as lsh
from lsh_sparse_attention_amd import inputs as gen
from oracle import ff_oracle as ffo
import gpu_util as gu

pytestmark = pytest.mark.gpu


def _close(name, got, want, s):
    err = np.abs(got - want)
    bound = 2.0 ** -8 * (s + np.abs(want)) + 1e-6
    bad = err > bound
    assert not bad.any(), (f"{name}: {bad.sum()} of {bad.size} outside the rounding bound; worst err/bound "
                           f"{(err / bound).max():.2f} at {np.argwhere(bad)[:3].tolist()}")


def _dev(d):
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return {"x": bf(d["x"]), "w1": bf(d["w1"]), "w2": bf(d["w2"]), "dy": bf(d["dy"]),
            "b1": torch.from_numpy(d["b1"]).cuda(), "b2": torch.from_numpy(d["b2"]).cuda()}


def _f64(d):
    f = lambda a: gen.bf16_bits_to_f32(a).astype(np.float64)
    return f(d["x"]), f(d["w1"]), d["b1"].astype(np.float64), f(d["w2"]), d["b2"].astype(np.float64), f(d["dy"])


def _run(d, chunks, backward=True):
    n, dm, dff = d["n"], d["d_model"], d["d_ff"]
    t = _dev(d)
    ff = lsh.ff_problem(n, dm, dff, chunks)
    y = torch.empty((n, dm), dtype=torch.bfloat16, device="cuda")
    lsh.lsh_ff_fwd(ff, t["x"], t["w1"], t["b1"], t["w2"], t["b2"], y)
    res = {"y": y}
    if backward:
        dx = torch.empty_like(y)
        dw1 = torch.empty((dm, dff), dtype=torch.float32, device="cuda")
        dw2 = torch.empty((dff, dm), dtype=torch.float32, device="cuda")
        db1 = torch.empty(dff, dtype=torch.float32, device="cuda")
        db2 = torch.empty(dm, dtype=torch.float32, device="cuda")
        lsh.lsh_ff_bwd(ff, t["x"], t["w1"], t["b1"], t["w2"], t["dy"], dx, dw1, db1, dw2, db2)
        res.update(dx=dx, dw1=dw1, db1=db1, dw2=dw2, db2=db2)
    torch.cuda.synchronize()
    return res


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


# n, d_model, d_ff, chunks: tiles of 128 with ragged row, column and K tails,
# one chunk and many, a chunk count that does not divide n
SMALL = [(1000, 64, 256, 3), (257, 128, 512, 1), (130, 64, 192, 7), (2048, 256, 1024, 4), (1, 8, 8, 1),
         (96, 1024, 4096, 2), (5, 16, 24, 9), (1100, 40, 136, 2)]


@pytest.mark.parametrize("n,dm,dff,c", SMALL)
def test_ff_small_shapes_match_oracle(n, dm, dff, c):
    gu.say(f"[gpu] ff n={n} d_model={dm} d_ff={dff} chunks={c}")
    d = gen.generate_ff(n, dm, dff, seed=900 + n)
    res = _run(d, c)
    x, w1, b1, w2, b2, dy = _f64(d)
    s = ffo.abs_sums(x, w1, b1, w2, dy)
    _close("y", _np(res["y"]), ffo.forward(x, w1, b1, w2, b2), s["y"])
    g = ffo.backward(x, w1, b1, w2, b2, dy)
    for k in ("dx", "dw1", "db1", "dw2", "db2"):
        _close(k, _np(res[k]), g[k], s[k])


def test_ff_chunking_changes_no_row():
    d = gen.generate_ff(1500, 128, 512, seed=950)
    one, many = _run(d, 1), _run(d, 6)
    for k in ("y", "dx"):
        assert torch.equal(one[k].view(torch.int16), many[k].view(torch.int16)), k
    for k in ("dw1", "db1", "dw2", "db2"):
        gu.assert_close(k, _np(many[k]), _np(one[k]), 1e-5)


def test_ff_paper_shape_full_size_sampled():
    # 65536 positions (the text workload's B * L) through the ablation layer
    # d_model = 1024, d_ff = 4096 in 8 chunks; the oracle checks sampled rows
    # of y and dx and sampled hidden units of the weight gradients
    n, dm, dff = 65536, gen.FF_SHAPE["d_model"], gen.FF_SHAPE["d_ff"]
    gu.say("[gpu] ff full size: generating")
    d = gen.generate_ff(n, dm, dff, seed=960)
    gu.say("[gpu] ff full size: running the library")
    res = _run(d, 8)
    x, w1, b1, w2, b2, dy = _f64(d)
    rows = [0, 1, 8191, 8192, 40000, 65535]
    gu.say("[gpu] ff full size: oracle on sampled rows and hidden units")
    cols = [0, 1, 777, 2048, 4095]
    s = ffo.abs_sums(x, w1, b1, w2, dy, rows=rows, cols=cols)
    _close("y rows", _np(res["y"])[rows], ffo.forward(x[rows], w1, b1, w2, b2), s["y"])
    _close("dx rows", _np(res["dx"])[rows], ffo.dx_rows(x, w1, b1, w2, dy, rows), s["dx"])
    c = ffo.weight_grad_columns(x, w1, b1, w2, dy, cols)
    _close("dw1 cols", _np(res["dw1"])[:, cols], c["dw1"], s["dw1"])
    _close("db1 cols", _np(res["db1"])[cols], c["db1"], s["db1"])
    _close("dw2 rows", _np(res["dw2"])[cols], c["dw2"], s["dw2"])
    _close("db2", _np(res["db2"]), dy.sum(axis=0), s["db2"])


def test_ff_empty_is_a_no_op():
    ff = lsh.ff_problem(0, 64, 256, 2)
    assert lsh.ff_workspace_bytes(ff, False) == 0
    z = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w1 = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((256, 64), dtype=torch.bfloat16, device="cuda")
    b1 = torch.zeros(256, device="cuda")
    b2 = torch.zeros(64, device="cuda")
    lsh.lsh_ff_fwd(ff, z, w1, b1, w2, b2, z, ws=torch.empty(1, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
