"""GPU parity of the Dense-NSA mode (nsa_prefill_dense: dense causal GQA over
every token) against the fp64 oracle, through the C ABI.

Bar: outputs max |d| <= 1e-2, mean |d| <= 1e-3 (the output bar of the NSA
path); lse within 2e-2 of the fp64 log-sum-exp. Each case prints its name
and shape before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
from sparse_attention_long_nsa_amd import binding
from sparse_attention_long_nsa_amd.inputs import PREFILL_PRESETS, PrefillShape, make_prefill_inputs

from gpu_util import upload

pytestmark = pytest.mark.gpu


def run_dense(inp, dev=None, lse=False):
    if dev is None:
        dev = upload(inp)
    r = binding.prefill_dense(dev["q"], dev["k"], dev["v"], want_lse=lse)
    torch.cuda.synchronize()
    out = {"out": r["out"].cpu().numpy()}
    if lse:
        out["lse"] = r["lse"].cpu().numpy()
    return out


def lse_fp64(inp, rows):
    """log-sum-exp of the scaled causal logits, fp64, per (row, head)."""
    q = np.asarray(inp["q"], np.float64)
    k = np.asarray(inp["k"], np.float64)
    hq, d = q.shape[1], q.shape[2]
    G = hq // k.shape[1]
    res = np.empty((len(rows), hq))
    for i, r in enumerate(rows):
        for h in range(hq):
            s = k[: r + 1, h // G] @ q[r, h] / math.sqrt(d)
            m = s.max()
            res[i, h] = m + math.log(np.exp(s - m).sum())
    return res


@pytest.mark.parametrize("shape", [
    PrefillShape(1000, 0, 77, 28, 4, 128, 64, 16, 512, "bf16"),   # vision + text, ragged tail
    PrefillShape(640, 30, 0, 8, 2, 64, 64, 4, 64, "bf16"),
    PrefillShape(300, 0, 0, 4, 1, 64, 64, 4, 128, "fp32"),
    PrefillShape(64, 0, 0, 28, 4, 128, 64, 16, 512, "bf16"),      # one whole block
    PrefillShape(65, 0, 0, 28, 4, 128, 64, 16, 512, "bf16"),      # one key past a block
    PrefillShape(1, 0, 0, 28, 4, 128, 64, 16, 512, "bf16"),       # a single token
])
def test_dense_all_rows(shape):
    print(f"\n[case] dense_all_rows: {shape}", flush=True)
    inp = make_prefill_inputs(shape, seed=21)
    gpu = run_dense(inp, lse=True)
    ref = oracle.dense(inp)
    rep = parity.compare(gpu["out"], ref)
    print(rep, flush=True)
    assert rep.ok(), rep
    rows = np.unique(np.linspace(0, shape.n_tokens - 1, 24).astype(np.int64))
    assert np.abs(gpu["lse"][rows] - lse_fp64(inp, rows)).max() < 2e-2


def test_dense_is_deterministic_and_matches_the_nsa_text_rows():
    s = PrefillShape(700, 100, 50, 28, 4, 128, 64, 16, 512, "bf16")
    print(f"\n[case] dense_vs_nsa_text_rows: {s}", flush=True)
    inp = make_prefill_inputs(s, seed=22)
    dev = upload(inp)
    a = run_dense(inp, dev=dev)["out"]
    b = run_dense(inp, dev=dev)["out"]
    assert np.array_equal(a, b)
    # the NSA path's text rows are dense causal too: close to the dense mode
    r = binding.prefill(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"], dev["w_v"],
                        dev["gates"], s.top_k, s.window)
    torch.cuda.synchronize()
    text = np.nonzero(inp["is_vision"] == 0)[0]
    assert np.abs(r["out"].cpu().numpy()[text] - a[text]).max() < 1e-2


def test_dense_full_size_sampled_rows():
    s = PREFILL_PRESETS["qwen_128k_k32_w256"]
    print(f"\n[case] dense qwen_128k: {s}", flush=True)
    inp = make_prefill_inputs(s, seed=0)
    gpu = run_dense(inp)
    rng = np.random.default_rng(3)
    n = s.n_tokens
    rows = np.unique(np.concatenate([np.arange(70), np.arange(n - 40, n),
                                     rng.choice(n, size=48, replace=False)]))
    ref = oracle.dense(inp, rows=rows)
    rep = parity.compare(gpu["out"][rows], ref)
    print(rep, flush=True)
    assert rep.ok(), rep
