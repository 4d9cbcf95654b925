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
