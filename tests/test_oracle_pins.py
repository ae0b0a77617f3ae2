"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names the pin it checks:
  P1/P2/P11  special cases that reduce to dense causal attention (torch fp64 SDPA)
  P3         one-hot gates isolate a single branch (exact)
  P4         C oracle == independent numpy masked-dense formulation (brute.py)
  P5         per-row attended-pair counts == closed forms; budget vs the pages
  P6         top-k == numpy.lexsort ranking of the oracle's own scores
  P7         pooled keys == reshape-mean-matmul
  P8         constant frames with W = I: closed-form compressed keys and o_cmp
  P9         all-equal keys: every score ties, lowest indices win
  P10        decode at the last cache slot == prefill's last row
  P12        linearity in v, invariance to a common key shift
  P13        permuting KV groups with their query heads permutes the output
  P14        one head per group: score == that head's compression probability
  P16        Dense-NSA mode: every row == torch fp64 SDPA causal
  P17        gate prologue: activations == their library forms, identity layers,
             a hand-worked example, affinity in the second layer
  P15        several vision runs: vision rows see only the vision tokens in
             position order (equal to the one-run layout), text rows dense causal
  P18        backward oracle: its forward == the C oracle's output and branch
             outputs; its gradients == finite differences (gradcheck); the gate
             gradient == the closed form from the C oracle's branch outputs
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from sparse_attention_long_nsa_amd.inputs import (
    DecodeShape, PrefillShape, make_decode_inputs, make_prefill_inputs, mask_from_runs, relayout)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small(n_vis=300, before=0, after=0, hq=4, hkv=1, d=16, k=4, w=100, B=64, dtype="fp32", seed=0):
    return make_prefill_inputs(PrefillShape(n_vis, before, after, hq, hkv, d, B, k, w, dtype), seed)


def sdpa_causal(q, k, v, hq, hkv):
    """Dense causal GQA with torch's fp64 CPU routine. q [n,Hq,d], k/v [n,Hkv,d]."""
    G = hq // hkv
    qt = torch.from_numpy(np.asarray(q, np.float64)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(np.asarray(k, np.float64)).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.asarray(v, np.float64)).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    return o[0].permute(1, 0, 2).numpy()


# ---------------------------------------------------------------- P1, P2, P11

def test_p1_selection_covering_all_blocks_is_dense_causal():
    inp = small(n_vis=300, hq=6, hkv=2, k=64)
    r = oracle.prefill(inp)
    ref = sdpa_causal(inp["q"], inp["k"], inp["v"], 6, 2)
    np.testing.assert_allclose(r["osel"], ref, rtol=0, atol=1e-12)


def test_p2_window_covering_sequence_is_dense_causal():
    inp = small(n_vis=300, hq=6, hkv=2, w=300)
    r = oracle.prefill(inp)
    ref = sdpa_causal(inp["q"], inp["k"], inp["v"], 6, 2)
    np.testing.assert_allclose(r["oswa"], ref, rtol=0, atol=1e-12)


def test_p11_text_rows_are_dense_causal_over_all_positions():
    inp = small(n_vis=256, before=40, after=70, hq=6, hkv=2)
    r = oracle.prefill(inp)
    ref = sdpa_causal(inp["q"], inp["k"], inp["v"], 6, 2)
    text = np.nonzero(inp["is_vision"] == 0)[0]
    np.testing.assert_allclose(r["out"][text], ref[text], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------- P3

@pytest.mark.parametrize("branch", [0, 1, 2])
def test_p3_one_hot_gates_isolate_a_branch(branch):
    inp = small(n_vis=200, hq=4, hkv=2)
    g = np.full_like(inp["gates"], -np.inf)
    g[..., branch] = np.inf
    inp["gates"] = g
    r = oracle.prefill(inp)
    name = ("ocmp", "osel", "oswa")[branch]
    np.testing.assert_array_equal(r["out"], r[name])


def test_p3_all_open_gates_sum_the_branches():
    inp = small(n_vis=200, hq=4, hkv=2)
    inp["gates"] = np.full_like(inp["gates"], np.inf)
    r = oracle.prefill(inp)
    np.testing.assert_allclose(r["out"], r["ocmp"] + r["osel"] + r["oswa"], rtol=0, atol=1e-15)


# ----------------------------------------------------------------------- P4

BRUTE_CASES = [
    # n_vis, before, after, hq, hkv, d, k, w
    (300, 0, 0, 4, 1, 16, 4, 100),
    (300, 0, 0, 4, 1, 16, 1, 1),
    (320, 0, 0, 4, 1, 16, 2, 64),
    (257, 30, 45, 6, 2, 16, 4, 64),
    (512, 0, 20, 6, 2, 8, 4, 100),
    (130, 5, 0, 4, 4, 16, 2, 1),
    (40, 3, 4, 4, 1, 16, 4, 100),  # no complete block at all
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_p4_oracle_equals_brute_force(case):
    n_vis, before, after, hq, hkv, d, k, w = case
    inp = small(n_vis, before, after, hq, hkv, d, k, w, seed=sum(case))
    r = oracle.prefill(inp, want=("lse", "sel", "ocmp", "osel", "oswa", "kcmp", "scores"))
    b = brute.layer(inp)
    V = b["vis"]
    np.testing.assert_allclose(r["out"], b["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["kcmp"], b["kcmp"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["vcmp"], b["vcmp"], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(r["sel"][V], b["sel"])
    np.testing.assert_array_equal(np.isinf(r["lse"][V]), np.isinf(b["lse"]))
    fin = np.isfinite(b["lse"])
    np.testing.assert_allclose(r["lse"][V][fin], b["lse"][fin], rtol=0, atol=1e-12)
    for name in ("ocmp", "osel", "oswa"):
        np.testing.assert_allclose(r[name][V], b[name], rtol=0, atol=1e-12)
    # scores: only the visible blocks are defined
    nb = b["scores"].shape[-1]
    t = np.arange(len(V))
    vis = (np.arange(nb)[None, :] + 1) * inp["shape"].block <= t[:, None] + 1
    np.testing.assert_allclose(r["scores"][V][np.broadcast_to(vis[:, None, :], b["scores"].shape)],
                               b["scores"][np.broadcast_to(vis[:, None, :], b["scores"].shape)],
                               rtol=0, atol=1e-12)


# ----------------------------------------------------------------------- P5

def closed_form_counts(n_vis, B, k, w):
    t = np.arange(n_vis, dtype=np.int64)
    cur = t // B
    n_cmp = (t + 1) // B
    n_sel = (np.minimum(k, cur + 1) - 1) * B + (t - cur * B + 1)
    n_swa = np.minimum(w, t + 1)
    return n_cmp, n_sel, n_swa


@pytest.mark.parametrize("k,w", [(4, 100), (1, 1), (8, 700)])
def test_p5_pair_counts_match_closed_form(k, w):
    inp = small(n_vis=650, hq=4, hkv=2, k=k, w=w, d=8)
    r = oracle.prefill(inp, want=("counts",))
    n_cmp, n_sel, n_swa = closed_form_counts(650, 64, k, w)
    np.testing.assert_array_equal(r["counts"][:, 0], n_cmp)
    np.testing.assert_array_equal(r["counts"][:, 1], n_sel)
    np.testing.assert_array_equal(r["counts"][:, 2], n_swa)


def attended_fraction(n_vis, B, k, w):
    """Fine-grained (selection + window) keys over dense causal pairs."""
    _, n_sel, n_swa = closed_form_counts(n_vis, B, k, w)
    dense = n_vis * (n_vis + 1) // 2
    return (int(n_sel.sum()) + int(n_swa.sum())) / dense


def test_p5_budget_fraction_against_the_pages():
    with open(os.path.join(GOLDEN, "pages_budget.json")) as f:
        g = json.load(f)
    B, k, w = g["block"], g["top_k"], g["window"]
    # The pages print 3.6% at "128K" without the accounting. The nominal
    # budget -- k blocks of B plus w window keys per query over the mean
    # causal length N/2 -- lands on it exactly when 128K means 128,000.
    nominal = 100 * (k * B + w) / (128000 / 2)
    assert round(nominal, 2) == g["budget_fraction_percent"]
    # The exact attended fraction of the oracle's key sets (partial current
    # block, short early rows) is a little lower; it must stay close.
    frac_131072 = 100 * attended_fraction(131072, B, k, w)
    frac_128000 = 100 * attended_fraction(128000, B, k, w)
    assert round(frac_131072, 2) == 3.44
    assert abs(frac_128000 - g["budget_fraction_percent"]) < 0.1
    assert abs(frac_131072 - g["budget_fraction_percent"]) < 0.2


def test_p5_preset_matches_pages_defaults():
    from sparse_attention_long_nsa_amd.inputs import PREFILL_PRESETS
    with open(os.path.join(GOLDEN, "pages_budget.json")) as f:
        g = json.load(f)
    s = PREFILL_PRESETS["qwen_128k_k32_w256"]
    assert (s.n_q_heads, s.n_kv_heads, s.block, s.top_k, s.window) == (
        g["n_q_heads"], g["n_kv_heads"], g["block"], g["top_k"], g["window"])


# ----------------------------------------------------------------------- P6

def test_p6_topk_equals_lexsort_of_scores():
    inp = small(n_vis=1024, hq=8, hkv=2, k=5, d=16)
    r = oracle.prefill(inp, want=("sel", "scores"))
    B, k = 64, 5
    for t in range(0, 1024, 7):
        cur, nc = t // B, (t + 1) // B
        cand = np.array([b for b in range(nc) if b != cur], dtype=np.int64)
        for g in range(2):
            if len(cand):
                sc = r["scores"][t, g, cand]
                chosen = cand[np.lexsort((cand, -sc))[: k - 1]]
            else:
                chosen = cand
            S = np.sort(np.concatenate([[cur], chosen]))
            exp = np.full(k, -1)
            exp[: len(S)] = S
            np.testing.assert_array_equal(r["sel"][t, g], exp)


# ----------------------------------------------------------------------- P7

def test_p7_pooling_is_reshape_mean_matmul():
    inp = small(n_vis=330, before=10, after=5, hq=4, hkv=2, d=16)
    r = oracle.prefill(inp, rows=np.array([0], np.int64), want=("kcmp",))
    V = np.nonzero(inp["is_vision"])[0]
    nb = len(V) // 64
    for x, wname, key in (("k", "w_k", "kcmp"), ("v", "w_v", "vcmp")):
        xs = inp[x][V][: nb * 64].astype(np.float64).reshape(nb, 64, 2, 16).mean(axis=1)
        ref = xs @ inp[wname].astype(np.float64).T
        np.testing.assert_allclose(r[key], ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.cmp_pool(inp["k"][V], inp["w_k"], 64), r["kcmp"], rtol=0, atol=0)


# ----------------------------------------------------------------------- P8

def test_p8_constant_frames_identity_map_closed_form():
    inp = small(n_vis=448, hq=4, hkv=1, d=16)
    rng = np.random.default_rng(5)
    kf = rng.standard_normal((7, 1, 16)).astype(np.float32)
    inp["k"] = np.repeat(kf, 64, axis=0)
    inp["w_k"] = np.eye(16, dtype=np.float32)
    inp["w_v"] = np.eye(16, dtype=np.float32)
    r = oracle.prefill(inp)
    np.testing.assert_array_equal(r["kcmp"], kf.astype(np.float64))
    vmean = inp["v"].astype(np.float64).reshape(7, 64, 1, 16).mean(axis=1)
    scale = 1 / math.sqrt(16)
    for t in (63, 64, 200, 447):
        nc = (t + 1) // 64
        for h in range(4):
            s = scale * (kf[:nc, 0].astype(np.float64) @ inp["q"][t, h].astype(np.float64))
            p = np.exp(s - s.max())
            p /= p.sum()
            np.testing.assert_allclose(r["ocmp"][t, h], p @ vmean[:nc, 0], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------- P9

def test_p9_all_equal_keys_tie_and_lowest_indices_win():
    inp = small(n_vis=640, hq=4, hkv=1, k=4, d=16)
    inp["k"][:] = inp["k"][0]
    r = oracle.prefill(inp, want=("sel",))
    for t in range(640):
        cur = t // 64
        S = sorted({cur} | set(range(min(3, cur))))
        exp = np.full(4, -1)
        exp[: len(S)] = S
        np.testing.assert_array_equal(r["sel"][t, 0], exp)


# ---------------------------------------------------------------------- P10

@pytest.mark.parametrize("L,k,w", [(640, 4, 100), (640, 16, 512), (641, 4, 100), (703, 6, 64), (63, 4, 30),
                                   (64, 2, 64), (129, 3, 200)])
def test_p10_decode_equals_prefill_last_row(L, k, w):
    # any cache length: when 64 does not divide L the query's own block is
    # the partial one after the L // 64 compressed blocks
    inp = small(n_vis=L, hq=6, hkv=2, d=16, k=k, w=w)
    r = oracle.prefill(inp, rows=np.array([L - 1], np.int64), want=("sel", "lse", "kcmp"))
    dec = dict(q=inp["q"][L - 1][None], k_cache=inp["k"][None], v_cache=inp["v"][None],
               gates=inp["gates"][L - 1][None],
               shape=DecodeShape(1, L, 6, 2, 16, 64, k, w, "fp32"))
    d = oracle.decode(dec, r["kcmp"].astype(np.float32)[None], r["vcmp"].astype(np.float32)[None])
    np.testing.assert_array_equal(d["sel"], r["sel"])
    np.testing.assert_allclose(d["out"], r["out"], rtol=0, atol=1e-5)
    np.testing.assert_allclose(d["lse"], r["lse"], rtol=0, atol=1e-5)


def test_p10_decode_inputs_end_at_the_last_frame():
    s = DecodeShape(2, 256, 4, 1, 16, 64, 2, 64, "fp32")
    inp = make_decode_inputs(s, seed=3)
    kc = np.stack([oracle.cmp_pool(inp["k_cache"][b], inp["w_k"], 64) for b in range(2)])
    vc = np.stack([oracle.cmp_pool(inp["v_cache"][b], inp["w_v"], 64) for b in range(2)])
    d = oracle.decode(inp, kc.astype(np.float32), vc.astype(np.float32))
    assert np.all(d["sel"][:, :, -1] == 3)  # own block is the last of the four
    assert d["counts"][0, 0] == 4 and d["counts"][0, 2] == 64


# ---------------------------------------------------------------------- P12

def test_p12_linear_in_values():
    inp = small(n_vis=300, before=9, after=11, hq=4, hkv=2)
    r1 = oracle.prefill(inp, want=("sel",))
    inp2 = dict(inp, v=inp["v"] * np.float32(2.0))
    r2 = oracle.prefill(inp2, want=("sel",))
    np.testing.assert_array_equal(r1["sel"], r2["sel"])
    np.testing.assert_allclose(r2["out"], 2.0 * r1["out"], rtol=1e-14, atol=1e-14)


def test_p12_common_key_shift_changes_nothing():
    inp = small(n_vis=300, before=9, after=11, hq=4, hkv=2)
    r1 = oracle.prefill(inp, want=("sel",))
    c = np.random.default_rng(9).standard_normal((1, 2, 16)).astype(np.float32)
    inp2 = dict(inp, k=(inp["k"] + c).astype(np.float32))
    r2 = oracle.prefill(inp2, want=("sel",))
    np.testing.assert_array_equal(r1["sel"], r2["sel"])
    np.testing.assert_allclose(r2["out"], r1["out"], rtol=0, atol=1e-6)


# ---------------------------------------------------------------------- P13

def test_p13_group_permutation_equivariance():
    hq, hkv, G = 6, 3, 2
    inp = small(n_vis=260, before=4, after=6, hq=hq, hkv=hkv)
    perm = np.array([2, 0, 1])
    qperm = np.concatenate([np.arange(p * G, (p + 1) * G) for p in perm])
    inp2 = dict(inp, q=inp["q"][:, qperm], k=inp["k"][:, perm], v=inp["v"][:, perm],
                gates=inp["gates"][:, qperm])
    r1 = oracle.prefill(inp, want=("sel",))
    r2 = oracle.prefill(inp2, want=("sel",))
    np.testing.assert_allclose(r2["out"], r1["out"][:, qperm], rtol=0, atol=1e-13)
    np.testing.assert_array_equal(r2["sel"], r1["sel"][:, perm])


# ---------------------------------------------------------------------- P14

def test_p14_single_head_group_score_is_its_probability():
    inp = small(n_vis=400, hq=2, hkv=2, d=16)
    r = oracle.prefill(inp, want=("scores", "kcmp", "lse"))
    scale = 1 / math.sqrt(16)
    for t in (63, 100, 399):
        nc = (t + 1) // 64
        for g in range(2):
            s = scale * (r["kcmp"][:nc, g] @ inp["q"][t, g].astype(np.float64))
            p = np.exp(s - s.max())
            p /= p.sum()
            np.testing.assert_allclose(r["scores"][t, g, :nc], p, rtol=0, atol=1e-14)
            assert np.all(r["scores"][t, g, nc:] == -1.0)


# ------------------------------------------------------------ input recipe

def test_generator_is_seeded_and_frame_correlated():
    s = PrefillShape(256, 2, 3, 4, 1, 16, 64, 4, 64, "bf16")
    a = make_prefill_inputs(s, seed=1)
    b = make_prefill_inputs(s, seed=1)
    for key in ("q", "k", "v", "gates", "w_k"):
        np.testing.assert_array_equal(a[key], b[key])
    # bf16-exact values
    assert not np.any(a["q"].view(np.uint32) & 0xFFFF)
    # tokens of one frame share a vector: within-frame spread ~0.5, across frames ~1.1
    vis = a["k"][2:258, 0]
    within = vis[:64].std(axis=0).mean()
    across = vis[::64].std(axis=0).mean()
    assert within < 0.7 < across


# ---------------------------------------------------------------------- P15

# Several vision runs in one sequence (paper summary page, "Method": tokens
# are split into vision and text sets by position; the NSA branches take the
# vision set). Runs straddle block boundaries, text runs are 1..many tokens.
SPAN_RUNS = [
    [("v", 100), ("t", 7), ("v", 120), ("t", 30)],
    [("t", 3), ("v", 64), ("t", 1), ("v", 64), ("t", 5), ("v", 92), ("t", 9)],
    [("v", 1), ("t", 2), ("v", 150), ("t", 40), ("v", 105)],
    [("t", 20), ("v", 70), ("t", 1), ("v", 1), ("t", 1), ("v", 184)],
]


def _spans_case(runs, hq=4, hkv=2, d=16, k=3, w=50, seed=5):
    m = mask_from_runs(runs)
    nv = int(m.sum())
    base = small(n_vis=nv, before=0, after=len(m) - nv, hq=hq, hkv=hkv, d=d, k=k, w=w, seed=seed)
    return base, relayout(base, m)


@pytest.mark.parametrize("runs", SPAN_RUNS)
def test_p15_vision_rows_see_the_vision_tokens_in_order(runs):
    base, inp = _spans_case(runs)
    a = oracle.prefill(base, want=("lse", "sel", "ocmp", "osel", "oswa"))
    b = oracle.prefill(inp, want=("lse", "sel", "ocmp", "osel", "oswa"))
    va = np.nonzero(base["is_vision"])[0]
    vb = np.nonzero(inp["is_vision"])[0]
    for name in ("out", "lse", "sel", "ocmp", "osel", "oswa"):
        np.testing.assert_array_equal(a[name][va], b[name][vb], err_msg=name)


@pytest.mark.parametrize("runs", SPAN_RUNS)
def test_p15_text_rows_dense_causal_with_several_vision_runs(runs):
    _, inp = _spans_case(runs)
    r = oracle.prefill(inp)
    ref = sdpa_causal(inp["q"], inp["k"], inp["v"], 4, 2)
    text = np.nonzero(inp["is_vision"] == 0)[0]
    np.testing.assert_allclose(r["out"][text], ref[text], rtol=0, atol=1e-12)


@pytest.mark.parametrize("runs", SPAN_RUNS[:2])
def test_p15_oracle_equals_brute_force_with_several_vision_runs(runs):
    _, inp = _spans_case(runs)
    r = oracle.prefill(inp, want=("sel", "ocmp", "osel", "oswa"))
    b = brute.layer(inp)
    V = b["vis"]
    np.testing.assert_allclose(r["out"], b["out"], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(r["sel"][V], b["sel"])
    for name in ("ocmp", "osel", "oswa"):
        np.testing.assert_allclose(r[name][V], b[name], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------- P16

@pytest.mark.parametrize("n,hq,hkv", [(300, 6, 2), (129, 4, 1), (1, 4, 4)])
def test_p16_dense_mode_is_dense_causal_on_every_row(n, hq, hkv):
    inp = small(n_vis=n, hq=hq, hkv=hkv)
    out = oracle.dense(inp)
    ref = sdpa_causal(inp["q"], inp["k"], inp["v"], hq, hkv)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------- P17

from oracle import gate_mlp  # noqa: E402


@pytest.mark.parametrize("act", gate_mlp.ACTIVATIONS)
def test_p17_activations_match_their_library_forms(act):
    x = np.linspace(-6.0, 6.0, 2001)
    t = torch.from_numpy(x)
    ref = {"silu": torch.nn.functional.silu(t),
           "gelu_tanh": torch.nn.functional.gelu(t, approximate="tanh"),
           "relu": torch.relu(t)}[act].numpy()
    np.testing.assert_allclose(gate_mlp.activation(x, act), ref, rtol=0, atol=1e-14)


def test_p17_identity_layers_give_the_activation_of_the_input():
    # W1 = I, no biases, W2 = I: the logits are act(x), laid out head-major
    rng = np.random.default_rng(7)
    hq = 4
    x = rng.standard_normal((5, 3 * hq))
    eye = np.eye(3 * hq)
    for act in gate_mlp.ACTIVATIONS:
        out = gate_mlp.gate_logits(x, eye, None, eye, None, act, hq)
        np.testing.assert_allclose(out, gate_mlp.activation(x, act).reshape(5, hq, 3), rtol=0, atol=0)


def test_p17_hand_worked_example():
    # d_model 2, d_hidden 2, one head: W1 = [[1, 2], [0, -1]], b1 = [0.5, 0],
    # x = [1, -1]: pre = [1 - 2 + 0.5, 0 + 1] = [-0.5, 1]; relu -> [0, 1];
    # W2 rows [1, 1], [2, 0], [0, -3], b2 = [0, 1, 2]: logits = [1, 1, -1]
    x = np.array([[1.0, -1.0]])
    w1 = np.array([[1.0, 2.0], [0.0, -1.0]])
    w2 = np.array([[1.0, 1.0], [2.0, 0.0], [0.0, -3.0]])
    out = gate_mlp.gate_logits(x, w1, [0.5, 0.0], w2, [0.0, 1.0, 2.0], "relu", 1)
    np.testing.assert_array_equal(out, [[[1.0, 1.0, -1.0]]])


def test_p17_logits_are_affine_in_the_second_layer():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((6, 16))
    w1, b1 = rng.standard_normal((8, 16)), rng.standard_normal(8)
    w2a, w2b = rng.standard_normal((6, 8)), rng.standard_normal((6, 8))
    ga = gate_mlp.gate_logits(x, w1, b1, w2a, None, "silu", 2)
    gb = gate_mlp.gate_logits(x, w1, b1, w2b, None, "silu", 2)
    gab = gate_mlp.gate_logits(x, w1, b1, w2a + 2 * w2b, None, "silu", 2)
    np.testing.assert_allclose(gab, ga + 2 * gb, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------- P18

from oracle import backward as bwd  # noqa: E402


def _vision_sel(inp):
    r = oracle.prefill(inp)
    return r, r["sel"][np.asarray(inp["is_vision"]).astype(bool)]


@pytest.mark.parametrize("case", [dict(n_vis=300, before=5, after=7, hq=4, hkv=2, d=16, k=3, w=50),
                                  dict(n_vis=260, before=0, after=0, hq=6, hkv=3, d=8, k=2, w=70)])
def test_p18_backward_oracle_forward_equals_the_c_oracle(case):
    inp = small(**case)
    r, sel = _vision_sel(inp)
    t = {n: torch.tensor(np.asarray(inp[n], dtype=np.float64)) for n in ("q", "k", "v", "w_k", "w_v", "gates")}
    out, (oc, os_, ow) = bwd.forward(t["q"], t["k"], t["v"], t["w_k"], t["w_v"], t["gates"], inp["is_vision"],
                                     sel, 64, case["w"], 1.0 / math.sqrt(case["d"]), branches=True)
    np.testing.assert_allclose(out.numpy(), r["out"], rtol=0, atol=1e-12)
    vis = np.asarray(inp["is_vision"]).astype(bool)
    for mine, ref in ((oc, r["ocmp"]), (os_, r["osel"]), (ow, r["oswa"])):
        np.testing.assert_allclose(mine.numpy(), ref[vis], rtol=0, atol=1e-12)


def test_p18_gradients_match_finite_differences():
    # tiny layout: 2 text tokens, 14 vision tokens in blocks of 4 (one partial),
    # 2 query heads on 1 KV head, d 3; every input is perturbed numerically
    rng = np.random.default_rng(3)
    N, hq, hkv, d, B, w = 18, 2, 1, 3, 4, 5
    isv = np.array([0] + [1] * 9 + [0] + [1] * 5 + [0, 0], dtype=np.uint8)[:N]
    nv = int(isv.sum())
    sel = np.full((nv, hkv, 2), -1, dtype=np.int32)
    for t in range(nv):  # own block plus the earliest complete one, as a fixed choice
        cur = t // B
        sel[t, 0, 0] = 0 if cur > 0 else cur
        sel[t, 0, 1] = cur if cur > 0 else -1
    args = [torch.tensor(rng.standard_normal(sh), dtype=torch.float64, requires_grad=True)
            for sh in ((N, hq, d), (N, hkv, d), (N, hkv, d), (d, d), (d, d), (N, hq, 3))]
    fn = lambda *a: bwd.forward(*a, isv, sel, B, w, 0.7)  # noqa: E731
    assert torch.autograd.gradcheck(fn, args, eps=1e-6, atol=1e-7, rtol=1e-5)


def test_p18_gate_gradient_closed_form():
    inp = small(n_vis=200, before=3, after=4, hq=4, hkv=2, d=8, k=2, w=40)
    r, sel = _vision_sel(inp)
    dout = np.random.default_rng(5).standard_normal(r["out"].shape)
    g = bwd.gradients(inp, sel, dout)
    vis = np.asarray(inp["is_vision"]).astype(bool)
    sig = 1.0 / (1.0 + np.exp(-np.asarray(inp["gates"], np.float64)[vis]))
    for c, name in enumerate(("ocmp", "osel", "oswa")):
        ref = (dout[vis] * r[name][vis]).sum(-1) * sig[..., c] * (1 - sig[..., c])
        np.testing.assert_allclose(g["gates"][vis][..., c], ref, rtol=0, atol=1e-12)
    assert np.all(g["gates"][~vis] == 0)


def test_p18_row_restricted_form_equals_the_full_form():
    """The row-restricted backward oracle (queries limited to a sample of
    rows) gives exactly the full form's rows, and its gradients equal the full
    form's gradients when dout is zero outside the sample; the restriction
    changes which queries are evaluated, not any formula."""
    inp = small(n_vis=300, before=5, after=7, hq=4, hkv=2, d=16, k=3, w=50)
    _, sel = _vision_sel(inp)
    N = inp["q"].shape[0]
    rows = np.array([0, 3, 5, 6, 70, 127, 128, 200, 304, 305, N - 2, N - 1])
    t = {n: torch.tensor(np.asarray(inp[n], dtype=np.float64)) for n in ("q", "k", "v", "w_k", "w_v", "gates")}
    args = (t["q"], t["k"], t["v"], t["w_k"], t["w_v"], t["gates"], inp["is_vision"], sel, 64, 50, 0.25)
    full = bwd.forward(*args).numpy()
    part = bwd.forward(*args, rows=rows).numpy()
    np.testing.assert_array_equal(part, full[rows])
    dout = np.random.default_rng(6).standard_normal(full.shape)
    dz = np.zeros_like(dout)
    dz[rows] = dout[rows]
    g_full = bwd.gradients(inp, sel, dz, scale=0.25)
    g_part = bwd.gradients(inp, sel, dout, scale=0.25, rows=rows)
    for n in g_full:
        np.testing.assert_allclose(g_part[n], g_full[n], rtol=0, atol=1e-12, err_msg=n)
    # and a restriction that drops a row drops exactly its contribution
    assert np.abs(g_part["q"][np.setdiff1d(np.arange(N), rows)]).max() == 0
