"""GPU parity of the backward pass (nsa_prefill_backward) against the fp64
autograd oracle (oracle/backward.py), through the C ABI.

Both sides take the C oracle's own block selection, so the comparison is
free of selection ties. Bar, from the arithmetic: the kernels work in fp32
(unit roundoff u = 2^-24) on bf16 inputs that are exact in fp32; every
gradient entry is a sum over at most N keys of products that are themselves
d-term dot products of O(1) values, so its relative error is about
(N + d) u, below 1e-4 for the sizes here. Each array must agree within 1e-3
of its largest magnitude (max |d| <= 1e-3 max |ref|) and on average within
1e-5 of it. Each case prints its name and shape before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as bwd
from sparse_attention_long_nsa_amd import binding
from sparse_attention_long_nsa_amd.inputs import PrefillShape, make_output_grad, make_prefill_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # n_vis, before, after, Hq, Hkv, d, k, w: partial last block, text on
    # both sides, a window wider than the vision run, no text, d 64 and 128
    PrefillShape(300, 5, 7, 4, 2, 64, 64, 3, 50, "bf16"),
    PrefillShape(200, 0, 0, 4, 1, 64, 64, 2, 400, "bf16"),
    PrefillShape(1045, 16, 48, 28, 4, 128, 64, 8, 256, "bf16"),
]


def run(inp, sel, dout):
    s = inp["shape"]
    dev = {n: torch.from_numpy(np.ascontiguousarray(inp[n])).to("cuda:0").to(torch.bfloat16).contiguous()
           for n in ("q", "k", "v", "w_k", "w_v")}
    gates = torch.from_numpy(np.ascontiguousarray(inp["gates"])).to("cuda:0")
    sel_d = torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).to("cuda:0")
    dout_d = torch.from_numpy(dout).to("cuda:0")
    r = binding.prefill_backward(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"], dev["w_v"], gates,
                                 sel_d, dout_d, s.top_k, s.window, block=s.block)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy().astype(np.float64) for n, t in r.items()}


@pytest.mark.parametrize("shape", CASES, ids=lambda s: f"nv{s.n_vis}_t{s.n_text}_h{s.n_q_heads}_d{s.head_dim}")
def test_backward_parity(shape):
    print(f"backward {shape}", flush=True)
    inp = make_prefill_inputs(shape, seed=11)
    vis = np.asarray(inp["is_vision"]).astype(bool)
    sel = oracle.prefill(inp, want=("out", "sel"))["sel"][vis]
    dout = make_output_grad((shape.n_tokens, shape.n_q_heads, shape.head_dim), seed=12)
    ref = bwd.gradients(inp, sel, dout)
    got = run(inp, sel, dout)
    pairs = (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dw_cmp_k", "w_k"), ("dw_cmp_v", "w_v"), ("dgate", "gates"))
    for gname, rname in pairs:
        g, rf = got[gname], ref[rname]
        assert np.all(np.isfinite(g)), gname
        big = np.abs(rf).max()
        err = np.abs(g - rf)
        assert err.max() <= 1e-3 * big, f"{gname}: max |d| {err.max():.3e} vs {big:.3e}"
        assert err.mean() <= 1e-5 * big, f"{gname}: mean |d| {err.mean():.3e} vs {big:.3e}"
