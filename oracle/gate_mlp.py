"""fp64 oracle of the gate prologue: hidden states -> gate logits.

TEST INFRASTRUCTURE, like the rest of this package: only the tests,
``__graft_entry__.smoke()`` and the CPU baseline leg of ``bench.py`` may use
it; the GPU library shares no code with it.

The pages say a two-layer MLP followed by a sigmoid gives each head its
three branch gates (paper summary page, "Method"; model card, "Model
Architecture": learnable per-head gates). Reading (their width and activation
are not given, so both are parameters of the call): the input is the token's
hidden state x (d_model values); logits = W2 . act(W1 . x + b1) + b2 with
W1 [d_hidden, d_model], W2 [3 Hq, d_hidden] (row 3 h + c is head h's logit
for branch c: compression, selection, window), optional biases; the sigmoid
is applied where the gates are used (the branch epilogues). Activations:
"silu" x * sigmoid(x), "gelu_tanh" 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715
x^3))), "relu" max(x, 0) -- each written out from its definition here.
"""
from __future__ import annotations

import math

import numpy as np

ACTIVATIONS = ("silu", "gelu_tanh", "relu")


def activation(h: np.ndarray, act: str) -> np.ndarray:
    h = np.asarray(h, dtype=np.float64)
    if act == "silu":
        return h / (1.0 + np.exp(-h))
    if act == "gelu_tanh":
        c = math.sqrt(2.0 / math.pi)
        return 0.5 * h * (1.0 + np.tanh(c * (h + 0.044715 * h ** 3)))
    if act == "relu":
        return np.maximum(h, 0.0)
    raise ValueError(f"unknown activation {act}")


def hidden(x, w1, b1, act: str) -> np.ndarray:
    """act(W1 x + b1) for every token: x [N, d_model] -> [N, d_hidden], fp64."""
    x = np.asarray(x, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    pre = x @ w1.T
    if b1 is not None:
        pre = pre + np.asarray(b1, dtype=np.float64)[None, :]
    return activation(pre, act)


def gate_logits(x, w1, b1, w2, b2, act: str, n_q_heads: int) -> np.ndarray:
    """Gate logits [N, Hq, 3] (fp64) of tokens x [N, d_model]."""
    h = hidden(x, w1, b1, act)
    out = h @ np.asarray(w2, dtype=np.float64).T
    if b2 is not None:
        out = out + np.asarray(b2, dtype=np.float64)[None, :]
    return out.reshape(out.shape[0], n_q_heads, 3)
