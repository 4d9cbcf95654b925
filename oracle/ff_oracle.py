"""Plain fp64 oracle of the chunked feed-forward layer.

TEST INFRASTRUCTURE ONLY: imported by the tests and the benchmark's CPU leg;
the library never uses it and shares nothing with it.

Source: "Reformer: The Efficient Transformer", §3 (Reversible Transformer):
the feed-forward computation is independent across sequence positions, so
it is split into c chunks of positions, forward and backward alike; chunking
changes the memory held at once, not the result.  The pages do not print the
layer itself; the reading here is the standard Transformer feed-forward
layer, FF(x) = relu(x W1 + b1) W2 + b2, applied to each position (row) x.
The oracle therefore computes the unchunked definition, in fp64 on the exact
input values, with NumPy matrix products as the only library steps.

Shapes: x [n, d_model], w1 [d_model, d_ff], b1 [d_ff], w2 [d_ff, d_model],
b2 [d_model]; dy like the output.
"""
import numpy as np


def forward(x, w1, b1, w2, b2):
    """y = relu(x w1 + b1) w2 + b2."""
    pre = x @ w1 + b1
    return np.maximum(pre, 0.0) @ w2 + b2


def backward(x, w1, b1, w2, b2, dy):
    """Gradients of sum(y * dy): dx, dw1, db1, dw2, db2.  relu'(p) = 1 for
    p > 0, else 0."""
    pre = x @ w1 + b1
    h = np.maximum(pre, 0.0)
    dh = (dy @ w2.T) * (pre > 0)
    return {"dx": dh @ w1.T, "dw1": x.T @ dh, "db1": dh.sum(axis=0), "dw2": h.T @ dy, "db2": dy.sum(axis=0)}


def dx_rows(x, w1, b1, w2, dy, rows):
    """Rows of dx only (each row of dx depends on that row of x and dy)."""
    pre = x[rows] @ w1 + b1
    return ((dy[rows] @ w2.T) * (pre > 0)) @ w1.T


def weight_grad_columns(x, w1, b1, w2, dy, cols):
    """Hidden units ``cols`` only: columns of dw1, entries of db1 and rows of
    dw2 (each depends on that hidden unit's column over all rows)."""
    pre = x @ w1[:, cols] + b1[cols]                  # [n, len(cols)]
    dh = (dy @ w2[cols].T) * (pre > 0)
    return {"dw1": x.T @ dh, "db1": dh.sum(axis=0), "dw2": np.maximum(pre, 0.0).T @ dy}


def abs_sums(x, w1, b1, w2, dy, rows=None, cols=None):
    """For each output, the sum of the absolute values of the terms it adds
    up (the scale of its rounding error): y <- |h| |w2|, dx <- |dh| |w1|^T,
    dw1 <- |x|^T |dh|, db1 <- sum |dh|, dw2 <- |h|^T |dy|, db2 <- sum |dy|.
    A kernel that rounds the hidden activation h (and dh) and its outputs to
    bf16 once each and accumulates in fp32 stays within
    2^-8 (abs_sum + |exact|) of the exact value (2^-9 per rounding of the
    intermediate and of the result; fp32 accumulation over K <= 2^12 terms
    adds at most 2^-12 abs_sum).  ``rows`` / ``cols`` restrict y, dx to those
    rows and the weight gradients to those hidden units, as in dx_rows and
    weight_grad_columns."""
    xr, dyr = (x, dy) if rows is None else (x[rows], dy[rows])
    pre_r = xr @ w1 + b1
    h_r, dh_r = np.maximum(pre_r, 0.0), (dyr @ w2.T) * (pre_r > 0)
    out = {"y": np.abs(h_r) @ np.abs(w2), "dx": np.abs(dh_r) @ np.abs(w1).T}
    c = slice(None) if cols is None else cols
    pre = x @ w1[:, c] + b1[c]
    h, dh = np.maximum(pre, 0.0), (dy @ w2[c].T) * (pre > 0)
    out.update(dw1=np.abs(x).T @ np.abs(dh), db1=np.abs(dh).sum(axis=0), dw2=np.abs(h).T @ np.abs(dy),
               db2=np.abs(dy).sum(axis=0))
    return out
