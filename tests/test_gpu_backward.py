"""GPU parity of the backward pass (nsa_prefill_backward) against the fp64
autograd oracle (oracle/backward.py), through the C ABI.

Both sides take the same block selection (the C oracle's own, or the GPU
forward's handed over as a caller would), so the comparison is free of
selection ties. Bar, from the arithmetic: the kernels multiply fp16 operands
on the matrix cores with fp32 accumulation. q, k and v are bf16 and convert
to fp16 exactly; dout, the probabilities P, the score gradients dS and the
compressed keys / values are rounded to fp16 (unit roundoff u = 2^-11). A
gradient element is a sum of products of two such operands, one of them
(dS) itself carrying the rounding of dP = dout . v and of P, so each term's
relative error is a few u and the element's error a few u times the sum of
its terms' magnitudes, which for these inputs is within a small factor of
the array's largest element. Each array must agree within 8 u of its
largest magnitude (max |d| <= 8 u max |ref|, 3.9e-3) and on average within
4 u of its mean magnitude (mean |d| <= 4 u mean |ref|, 2.0e-3), each plus
1e-6 absolute for arrays whose reference cancels to zero; measured on these
cases: at most 7.0e-4 and 6.5e-4. D = dout . o is formed from dout rounded to
fp16, as in the products that give dP, so that dP - D cancels exactly where
a row's probability sits on one key. Each case prints its name and shape
before touching the GPU.
"""
import math

U16 = 2.0 ** -11  # fp16 unit roundoff
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
    # both sides, a window wider than the vision run, no text, d 64 and 128,
    # one and eight query heads per KV head
    PrefillShape(300, 5, 7, 4, 2, 64, 64, 3, 50, "bf16"),
    PrefillShape(200, 0, 0, 4, 1, 64, 64, 2, 400, "bf16"),
    PrefillShape(1045, 16, 48, 28, 4, 128, 64, 8, 256, "bf16"),
    PrefillShape(333, 3, 9, 3, 3, 64, 64, 4, 90, "bf16"),
    PrefillShape(400, 0, 20, 16, 2, 64, 64, 5, 128, "bf16"),
    # edge cases: no complete block (no compressed keys), text only (no vision
    # rows at all), exactly one block (one compressed key, seen by one token)
    PrefillShape(40, 10, 5, 4, 2, 64, 64, 2, 16, "bf16"),
    PrefillShape(0, 70, 0, 4, 2, 64, 64, 2, 16, "bf16"),
    PrefillShape(64, 0, 0, 8, 1, 64, 64, 3, 64, "bf16"),
]


def run(inp, sel, dout):
    s = inp["shape"]
    dev = {n: torch.from_numpy(np.ascontiguousarray(inp[n])).to("cuda:0").to(torch.bfloat16).contiguous()
           for n in ("q", "k", "v", "w_k", "w_v")}
    gates = torch.from_numpy(np.ascontiguousarray(inp["gates"])).to("cuda:0")
    sel_d = torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).to("cuda:0") if len(sel) else None
    dout_d = torch.from_numpy(dout).to("cuda:0")
    r = binding.prefill_backward(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"], dev["w_v"], gates,
                                 sel_d, dout_d, s.top_k, s.window, block=s.block)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy().astype(np.float64) for n, t in r.items()}


def check_bar(gname, g, rf):
    assert np.all(np.isfinite(g)), gname
    big, avg = np.abs(rf).max(), np.abs(rf).mean()
    err = np.abs(g - rf)
    print(f"  {gname}: max |d| {err.max():.3e} (max |ref| {big:.3e}), "
          f"mean |d| {err.mean():.3e} (mean |ref| {avg:.3e})", flush=True)
    # plus 1e-6 absolute: where the reference cancels to exactly zero (a
    # compressed key seen by a single query, whose dS is P (dP - D) with one
    # probability of 1), the fp32 sums leave residues of order 2^-24 times
    # the terms' magnitude
    assert err.max() <= 8 * U16 * big + 1e-6, f"{gname}: max |d| {err.max():.3e} vs {big:.3e}"
    assert err.mean() <= 4 * U16 * avg + 1e-6, f"{gname}: mean |d| {err.mean():.3e} vs mean |ref| {avg:.3e}"


@pytest.mark.parametrize("shape", CASES, ids=lambda s: f"nv{s.n_vis}_t{s.n_text}_h{s.n_q_heads}_d{s.head_dim}")
def test_backward_parity(shape):
    print(f"backward {shape}", flush=True)
    inp = make_prefill_inputs(shape, seed=11)
    vis = np.asarray(inp["is_vision"]).astype(bool)
    if vis.any():
        sel = oracle.prefill(inp, want=("out", "sel"))["sel"][vis]
    else:
        sel = np.zeros((0, shape.n_kv_heads, shape.top_k), np.int32)
    dout = make_output_grad((shape.n_tokens, shape.n_q_heads, shape.head_dim), seed=12)
    ref = bwd.gradients(inp, sel, dout)
    got = run(inp, sel, dout)
    pairs = (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dw_cmp_k", "w_k"), ("dw_cmp_v", "w_v"), ("dgate", "gates"))
    for gname, rname in pairs:
        check_bar(gname, got[gname], ref[rname])


def upload(inp):
    dev = {n: torch.from_numpy(np.ascontiguousarray(inp[n])).to("cuda:0").to(torch.bfloat16).contiguous()
           for n in ("q", "k", "v", "w_k", "w_v")}
    dev["gates"] = torch.from_numpy(np.ascontiguousarray(inp["gates"])).to("cuda:0")
    return dev


def sample_rows(inp, n_vis_rows, n_text_rows, seed=0):
    isv = np.asarray(inp["is_vision"]).astype(bool)
    V, T = np.nonzero(isv)[0], np.nonzero(~isv)[0]
    rng = np.random.default_rng(seed)
    picks = [V[:3], V[[63, 64, 65, 127, 128]], V[-3:], rng.choice(V, n_vis_rows, replace=False)]
    if len(T):
        picks += [T[[0, -1]], rng.choice(T, n_text_rows, replace=False)]
    return np.unique(np.concatenate(picks))


# The benchmarked backward (4,096 vision + 512 text tokens, k 32, w 256) and
# the pages' training length (36,864 + 512, k 16, w 512; model card,
# "Training Details"), on sampled rows: the upstream gradient is zero outside
# the sample, so the oracle needs only those queries (its row-restricted
# form), while the GPU runs the whole layer. The selection is the GPU
# forward's own sel_idx, handed to the backward as a caller would.
@pytest.mark.parametrize("shape,n_vis_rows,n_text_rows", [
    (PrefillShape(4096, 0, 512, 28, 4, 128, 64, 32, 256, "bf16"), 160, 24),
    (PrefillShape(36864, 0, 512, 28, 4, 128, 64, 16, 512, "bf16"), 64, 8),
], ids=["bench_4k_k32_w256", "train_36k_k16_w512"])
def test_backward_parity_sampled_rows_on_the_forwards_selection(shape, n_vis_rows, n_text_rows):
    print(f"backward sampled rows {shape}", flush=True)
    inp = make_prefill_inputs(shape, seed=13)
    dev = upload(inp)
    fwd = binding.prefill(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"], dev["w_v"], dev["gates"],
                          shape.top_k, shape.window, want_sel=True)
    torch.cuda.synchronize()
    sel = fwd["sel_idx"].cpu().numpy()
    rows = sample_rows(inp, n_vis_rows, n_text_rows)
    dout = np.zeros((shape.n_tokens, shape.n_q_heads, shape.head_dim), np.float32)
    dout[rows] = make_output_grad((len(rows), shape.n_q_heads, shape.head_dim), seed=14)
    got = binding.prefill_backward(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"], dev["w_v"],
                                   dev["gates"], fwd["sel_idx"], torch.from_numpy(dout).to("cuda:0"),
                                   shape.top_k, shape.window, block=shape.block)
    torch.cuda.synchronize()
    got = {n: t.cpu().numpy().astype(np.float64) for n, t in got.items()}
    print(f"  {len(rows)} rows, oracle ...", flush=True)
    ref = bwd.gradients(inp, sel, dout, rows=rows)
    others = np.setdiff1d(np.arange(shape.n_tokens), rows)
    assert np.all(got["dq"][others] == 0) and np.all(got["dgate"][others] == 0)
    pairs = (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dw_cmp_k", "w_k"), ("dw_cmp_v", "w_v"), ("dgate", "gates"))
    for gname, rname in pairs:
        check_bar(gname, got[gname], ref[rname])


def test_backward_hostile_selection_lists_stay_in_bounds():
    """Selection entries far outside the valid range (negative, beyond the
    query's own block, 2^25, INT32_MAX) are clamped before any index
    arithmetic: the call completes with finite gradients."""
    shape = PrefillShape(640, 4, 8, 8, 2, 64, 64, 4, 100, "bf16")
    print(f"backward hostile lists {shape}", flush=True)
    inp = make_prefill_inputs(shape, seed=15)
    dev = upload(inp)
    nv = shape.n_vis
    rng = np.random.default_rng(16)
    bad = rng.choice(np.array([-7, -1, 0, 3, 9, 1 << 25, (1 << 31) - 1], np.int64), size=(nv, 2, 4)).astype(np.int32)
    dout = make_output_grad((shape.n_tokens, shape.n_q_heads, shape.head_dim), seed=17)
    got = binding.prefill_backward(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"], dev["w_v"],
                                   dev["gates"], torch.from_numpy(bad).to("cuda:0"),
                                   torch.from_numpy(dout).to("cuda:0"), shape.top_k, shape.window, block=shape.block)
    torch.cuda.synchronize()
    for n, t in got.items():
        assert torch.isfinite(t).all(), n


def test_backward_is_bitwise_repeatable():
    """Every gradient element is written by one thread in a fixed order (no
    atomics): two calls give identical bits."""
    shape = PrefillShape(1045, 16, 48, 28, 4, 128, 64, 8, 256, "bf16")
    print(f"backward repeatability {shape}", flush=True)
    inp = make_prefill_inputs(shape, seed=18)
    vis = np.asarray(inp["is_vision"]).astype(bool)
    sel = oracle.prefill(inp, want=("sel",))["sel"][vis]
    dout = make_output_grad((shape.n_tokens, shape.n_q_heads, shape.head_dim), seed=19)
    a, b = run(inp, sel, dout), run(inp, sel, dout)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
