"""GPU parity with several vision runs in one sequence (row maps), through the C ABI.

The vision tokens lie in several runs with text between them; the NSA
branches take the vision tokens in position order and text tokens attend to
every earlier token. Same bar as the one-run parity tests: selected indices
exact except near-ties (oracle score gap <= 1e-3), outputs max |d| <= 1e-2,
mean |d| <= 1e-3. Each case prints its name and shape before touching the GPU.
"""
import numpy as np
import pytest

from oracle import parity
from sparse_attention_long_nsa_amd.inputs import (
    PREFILL_PRESETS, SPAN_LAYOUTS, PrefillShape, make_prefill_inputs, mask_from_runs, relayout)

from gpu_util import run_prefill, upload

pytestmark = pytest.mark.gpu


def spans_inputs(runs, hq, hkv, d, k, w, dtype="bf16", seed=11):
    m = mask_from_runs(runs)
    nv = int(m.sum())
    base = make_prefill_inputs(PrefillShape(nv, 0, len(m) - nv, hq, hkv, d, 64, k, w, dtype), seed)
    return base, relayout(base, m)


def announce(name, runs, extra=""):
    short = runs if len(runs) <= 12 else f"{len(runs)} runs"
    print(f"\n[case] {name}: {short} {extra}", flush=True)


def check(inp, rows):
    gpu = run_prefill(inp)
    rep, orep, _ = parity.check_prefill(inp, gpu, rows)
    print(rep, "|", orep, flush=True)
    if rep is not None:
        assert rep.counted == 0, rep
    assert orep.ok(), orep
    return gpu


CASES = [
    # runs, hq, hkv, d, k, w, dtype
    ([("t", 40), ("v", 1000), ("t", 3), ("v", 777), ("t", 100), ("v", 1300), ("t", 60)],
     28, 4, 128, 16, 512, "bf16"),
    # blocks straddling runs, 1-token text runs
    ([("v", 100), ("t", 1), ("v", 28), ("t", 1), ("v", 64 * 20 + 5)], 28, 4, 128, 8, 100, "bf16"),
    ([("t", 5), ("v", 300), ("t", 64), ("v", 64), ("t", 1), ("v", 900)], 8, 2, 64, 4, 64, "bf16"),
    ([("v", 100), ("t", 10), ("v", 200), ("t", 3)], 4, 1, 64, 4, 128, "fp32"),
    # a text token after every 50 vision tokens
    ([("v", 50), ("t", 1)] * 40, 28, 4, 128, 4, 256, "bf16"),
]


@pytest.mark.parametrize("case", CASES)
def test_several_vision_runs_all_rows(case):
    runs, hq, hkv, d, k, w, dt = case
    announce("spans_all_rows", runs, f"hq {hq} hkv {hkv} d {d} k {k} w {w} {dt}")
    _, inp = spans_inputs(runs, hq, hkv, d, k, w, dt)
    check(inp, np.arange(len(inp["is_vision"])))


def test_runs_across_mask_slices_sampled_rows():
    # longer than one 16,384-position slice of the mask: maps built by
    # several launches, runs crossing slice boundaries
    runs = [("t", 100), ("v", 16000), ("t", 300), ("v", 20000), ("t", 50), ("v", 3000), ("t", 7)]
    announce("spans_slices", runs)
    _, inp = spans_inputs(runs, 28, 4, 128, 16, 512)
    rows = parity.sample_rows(inp, n_random=192, n_text=48)
    T = np.nonzero(inp["is_vision"] == 0)[0]
    V = np.nonzero(inp["is_vision"])[0]
    # the rows on both sides of every run boundary
    edges = np.nonzero(np.diff(inp["is_vision"].astype(np.int8)))[0]
    rows = np.unique(np.concatenate([rows, edges, edges + 1, T[:: max(1, len(T) // 64)], V[16000 - 70:16000 + 70]]))
    check(inp, rows)


def test_vision_rows_equal_the_one_run_layout_bitwise():
    # the vision rows depend only on the vision tokens in order, so the GPU
    # gives them bit for bit what it gives the one-run layout
    runs = [("v", 2000), ("t", 30), ("v", 1500), ("t", 1), ("v", 700), ("t", 90)]
    announce("spans_vs_one_run", runs)
    base, inp = spans_inputs(runs, 28, 4, 128, 16, 512)
    a = run_prefill(base)
    b = run_prefill(inp)
    va = np.nonzero(base["is_vision"])[0]
    vb = np.nonzero(inp["is_vision"])[0]
    assert np.array_equal(a["sel"], b["sel"])
    assert np.array_equal(a["out"][va], b["out"][vb])


def test_full_size_eight_clips_sampled_rows():
    s = PREFILL_PRESETS["qwen_128k_k32_w256"]
    runs = SPAN_LAYOUTS["8clips"]
    announce("qwen_128k_k32_w256 8clips", runs)
    m = mask_from_runs(runs)
    base = make_prefill_inputs(s.replace(n_text_before=0, n_text_after=len(m) - s.n_vis), seed=0)
    inp = relayout(base, m)
    del base
    dev = upload(inp)
    gpu = run_prefill(inp, dev=dev)
    del dev
    rows = parity.sample_rows(inp, n_random=256, n_text=64)
    edges = np.nonzero(np.diff(inp["is_vision"].astype(np.int8)))[0]
    rows = np.unique(np.concatenate([rows, edges, edges + 1]))
    rep, orep, _ = parity.check_prefill(inp, gpu, rows)
    print(rep, "|", orep, flush=True)
    assert rep.counted == 0, rep
    assert orep.ok(), orep
