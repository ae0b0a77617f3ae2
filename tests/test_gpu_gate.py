"""GPU parity of the gate prologue (nsa_gate_logits: hidden states -> gate
logits through the two-layer MLP) against the fp64 oracle, through the C ABI.

Bar, per logit o of token t (derived from the kernels' arithmetic): the
hidden layer multiplies bf16 values exactly and sums d_model products in
fp32, is activated (slope at most 1.1 for these activations) and stored in
fp16 (relative rounding 2^-11); the output layer converts W2 to fp16 (exact
above 2^-14 in magnitude, absolute error below 2^-25 under it) and sums
d_hidden exact products in fp32. So
    |gpu - ref| <= 2^-10 * sum_j |W2_oj| (|h_j| + 1.1 d_model 2^-24 sum_k |W1_jk x_k|)
                   + 2^-24 sum_j |h_j| + 1e-6,
with h the fp64 hidden layer; the layer's own output bar (max |d| <= 1e-2,
mean |d| <= 1e-3) is checked on the logits as well. Each case prints its
name and shape before touching the GPU.
"""
import numpy as np
import pytest
import torch

from oracle import gate_mlp
from sparse_attention_long_nsa_amd import binding
from sparse_attention_long_nsa_amd.inputs import make_gate_inputs

pytestmark = pytest.mark.gpu


def upload(g, dev="cuda:0"):
    out = {}
    for key in ("x", "w1", "w2"):
        out[key] = torch.from_numpy(g[key]).to(dev).to(torch.bfloat16).contiguous()
    for key in ("b1", "b2"):
        out[key] = None if g[key] is None else torch.from_numpy(g[key]).to(dev)
    return out


def bound(g, rows, act):
    x = np.asarray(g["x"][rows], np.float64)
    w1 = np.asarray(g["w1"], np.float64)
    w2 = np.abs(np.asarray(g["w2"], np.float64))
    h = np.abs(gate_mlp.hidden(x, w1, g["b1"], act))
    s1 = np.abs(x) @ np.abs(w1).T                      # sum_k |W1_jk x_k|
    dm = x.shape[1]
    per_h = h + 1.1 * dm * 2.0 ** -24 * s1
    return 2.0 ** -10 * (per_h @ w2.T) + 2.0 ** -24 * h.sum(axis=1, keepdims=True) + 1e-6


def check(g, got, rows, act, label):
    ref = gate_mlp.gate_logits(g["x"][rows], g["w1"], g["b1"], g["w2"], g["b2"], act,
                               g["n_q_heads"]).reshape(len(rows), -1)
    got = np.asarray(got, np.float64).reshape(len(rows), -1)
    assert np.all(np.isfinite(got)), label
    err = np.abs(got - ref)
    tol = bound(g, rows, act)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), f"{label}: |d| {err[worst]:.3e} > {tol[worst]:.3e} at {worst}"
    assert err.max() <= 1e-2 and err.mean() <= 1e-3, f"{label}: max {err.max():.3e} mean {err.mean():.3e}"


CASES = [
    # (n, d_model, d_hidden, Hq, act, bias): ragged token counts against the
    # 256-token tile and the 64-token wave; 3 Hq = 84 (ragged), 96 (full), 3
    (300, 256, 256, 28, "silu", True),
    (300, 256, 256, 28, "gelu_tanh", True),
    (300, 256, 256, 28, "relu", False),
    (1, 64, 128, 28, "silu", True),
    (17, 128, 256, 32, "silu", True),
    (129, 192, 384, 1, "gelu_tanh", True),
    (1000, 3584, 1024, 28, "silu", True),
]


@pytest.mark.parametrize("n,dm,dh,hq,act,bias", CASES)
def test_gate_parity(n, dm, dh, hq, act, bias):
    label = f"gate n={n} d_model={dm} d_hidden={dh} Hq={hq} {act} bias={bias}"
    print(label, flush=True)
    g = make_gate_inputs(n, dm, dh, hq, seed=n + dh, bias=bias)
    d = upload(g)
    out = binding.gate_logits(d["x"], d["w1"], d["b1"], d["w2"], d["b2"], hq, act)
    torch.cuda.synchronize()
    check(g, out.cpu().numpy(), np.arange(n), act, label)


def test_gate_full_size_sampled_rows():
    """The bench's workload (131,584 tokens of a 3,584-wide model, 1,024
    hidden units, 28 heads): 512 sampled tokens, the first and last included,
    against the oracle one by one; then a second call into a reused output and
    workspace gives identical bits."""
    n, dm, dh, hq = 131072 + 512, 3584, 1024, 28
    print(f"gate full size n={n}", flush=True)
    g = make_gate_inputs(n, dm, dh, hq, seed=7)
    d = upload(g)
    out = binding.gate_logits(d["x"], d["w1"], d["b1"], d["w2"], d["b2"], hq, "silu")
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 510)]))
    got = out.cpu().numpy()
    check(g, got[rows], rows, "silu", "full size")
    again = binding.gate_logits(d["x"], d["w1"], d["b1"], d["w2"], d["b2"], hq, "silu", out=out)
    torch.cuda.synchronize()
    assert np.array_equal(again.cpu().numpy(), got)


def test_gate_feeds_the_layer():
    """Gate logits made on the device are the layer's gate_logits argument:
    the layer run on them equals the layer run on the same logits copied
    through the host."""
    from gpu_util import run_prefill, upload as upload_layer
    from sparse_attention_long_nsa_amd.inputs import PrefillShape, make_prefill_inputs
    s = PrefillShape(1024, 64, 64, 28, 4, 128, 64, 8, 256, "bf16")
    inp = make_prefill_inputs(s, seed=3)
    n = s.n_tokens
    print(f"gate -> layer n={n}", flush=True)
    g = make_gate_inputs(n, 256, 256, s.n_q_heads, seed=5)
    d = upload(g)
    logits = binding.gate_logits(d["x"], d["w1"], d["b1"], d["w2"], d["b2"], s.n_q_heads, "silu")
    torch.cuda.synchronize()
    host = logits.cpu().numpy()
    dev = upload_layer(inp)
    dev["gates"] = logits
    a = run_prefill(inp, dev=dev)
    inp2 = dict(inp, gates=host)
    b = run_prefill(inp2)
    assert np.array_equal(a["out"], b["out"])
