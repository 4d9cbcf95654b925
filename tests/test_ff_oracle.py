"""Pins of the feed-forward oracle (oracle/ff_oracle.py) against facts fixed
outside it: torch fp64 autograd of the same layer, central differences, and
closed forms."""
import numpy as np
import pytest
import torch

from oracle import ff_oracle as ffo


def _problem(seed, n, dm, dff):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, dm)), rng.standard_normal((dm, dff)) / np.sqrt(dm),
            rng.standard_normal(dff) * 0.1, rng.standard_normal((dff, dm)) / np.sqrt(dff),
            rng.standard_normal(dm) * 0.1, rng.standard_normal((n, dm)))


@pytest.mark.parametrize("seed,n,dm,dff", [(1, 37, 16, 48), (2, 128, 64, 256)])
def test_ff_matches_torch_autograd(seed, n, dm, dff):
    x, w1, b1, w2, b2, dy = _problem(seed, n, dm, dff)
    ts = [torch.tensor(a, requires_grad=True) for a in (x, w1, b1, w2, b2)]
    y = torch.relu(ts[0] @ ts[1] + ts[2]) @ ts[3] + ts[4]
    (y * torch.from_numpy(dy)).sum().backward()
    np.testing.assert_allclose(ffo.forward(x, w1, b1, w2, b2), y.detach().numpy(), rtol=1e-12, atol=1e-12)
    g = ffo.backward(x, w1, b1, w2, b2, dy)
    for name, t in zip(("dx", "dw1", "db1", "dw2", "db2"), ts):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-11, atol=1e-11, err_msg=name)


def test_ff_finite_differences():
    x, w1, b1, w2, b2, dy = _problem(3, 9, 6, 10)
    g = ffo.backward(x, w1, b1, w2, b2, dy)
    args = [x, w1, b1, w2, b2]
    h = 1e-6
    rng = np.random.default_rng(3)
    for k, name in enumerate(("dx", "dw1", "db1", "dw2", "db2")):
        a = args[k]
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in a.shape)
            ap, am = a.copy(), a.copy()
            ap[idx] += h
            am[idx] -= h
            fp = (ffo.forward(*[ap if j == k else args[j] for j in range(5)]) * dy).sum()
            fm = (ffo.forward(*[am if j == k else args[j] for j in range(5)]) * dy).sum()
            assert (fp - fm) / (2 * h) == pytest.approx(g[name][idx], rel=1e-6, abs=1e-7), name


def test_ff_closed_forms():
    # positive pre-activations everywhere: the layer is affine, y = x w1 w2 +
    # b1 w2 + b2; all negative: y = b2 and no gradient reaches x, w1 or b1
    rng = np.random.default_rng(4)
    n, dm, dff = 12, 5, 7
    x = np.abs(rng.standard_normal((n, dm)))
    w1 = np.abs(rng.standard_normal((dm, dff)))
    b1 = np.ones(dff)
    w2, b2 = rng.standard_normal((dff, dm)), rng.standard_normal(dm)
    np.testing.assert_allclose(ffo.forward(x, w1, b1, w2, b2), x @ w1 @ w2 + b1 @ w2 + b2, rtol=1e-13)
    y = ffo.forward(x, -w1, -b1, w2, b2)
    np.testing.assert_array_equal(y, np.broadcast_to(b2, y.shape))
    g = ffo.backward(x, -w1, -b1, w2, b2, rng.standard_normal((n, dm)))
    for name in ("dx", "dw1", "db1", "dw2"):
        assert not np.any(g[name]), name


def test_ff_row_and_column_restrictions_agree_with_full_backward():
    x, w1, b1, w2, b2, dy = _problem(5, 40, 16, 24)
    g = ffo.backward(x, w1, b1, w2, b2, dy)
    rows, cols = [0, 7, 39], [1, 5, 23]
    np.testing.assert_allclose(ffo.dx_rows(x, w1, b1, w2, dy, rows), g["dx"][rows], rtol=1e-13, atol=1e-13)
    c = ffo.weight_grad_columns(x, w1, b1, w2, dy, cols)
    np.testing.assert_allclose(c["dw1"], g["dw1"][:, cols], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(c["db1"], g["db1"][cols], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(c["dw2"], g["dw2"][cols], rtol=1e-13, atol=1e-13)


def test_ff_abs_sums_bound_the_terms():
    # the absolute-sum companions dominate the outputs and restrict like them
    x, w1, b1, w2, b2, dy = _problem(6, 30, 12, 20)
    g = ffo.backward(x, w1, b1, w2, b2, dy)
    s = ffo.abs_sums(x, w1, b1, w2, dy)
    assert np.all(s["y"] + np.abs(b2) >= np.abs(ffo.forward(x, w1, b1, w2, b2)) - 1e-12)
    for k in ("dx", "dw1", "db1", "dw2", "db2"):
        assert np.all(s[k] >= np.abs(g[k]) - 1e-12), k
    r = ffo.abs_sums(x, w1, b1, w2, dy, rows=[2, 5], cols=[3, 19])
    np.testing.assert_allclose(r["dx"], s["dx"][[2, 5]], rtol=1e-13)
    np.testing.assert_allclose(r["dw1"], s["dw1"][:, [3, 19]], rtol=1e-13)
    np.testing.assert_allclose(r["dw2"], s["dw2"][[3, 19]], rtol=1e-13)
