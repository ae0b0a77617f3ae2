"""Pins of the parity checker itself (``oracle/parity.py``) and of the
oracle's selection-injection path, on the CPU.

Every GPU parity claim goes through these two pieces: ``index_parity``
decides which selection differences are near-ties (exempt) and which count,
and the oracle re-evaluates exempt rows on the GPU's selection
(``inject_sel``). A bug in either would weaken every claim without a visible
failure, so each is tested here on cases whose right answer is known by
construction.
"""
import numpy as np
import pytest

import oracle
from oracle import parity
from sparse_attention_long_nsa_amd.inputs import PrefillShape, make_prefill_inputs


# ------------------------------------------------------------ index parity
def scores_for(rows_scores):
    """scores_fn over a fixed [n, hkv, n_blk] array."""
    return lambda idx: rows_scores[idx]


def one_row(sel_gpu, sel_ora, scores, cur):
    g = np.asarray(sel_gpu, np.int32)[None, None]
    o = np.asarray(sel_ora, np.int32)[None, None]
    sc = np.asarray(scores, np.float64)[None, None]
    return parity.index_parity(g, o, scores_for(sc), np.array([cur]))


def test_identical_selection_is_exact():
    rep = one_row([0, 3, 5], [0, 3, 5], [0.5, 0.1, 0.1, 0.4, 0.1, 0.9], 5)
    assert (rep.exact, rep.exempt, rep.counted) == (1, 0, 0)


def test_near_tie_swap_is_exempt():
    # oracle takes block 3 (score 0.4000), GPU takes block 1 (0.3995): gap 5e-4
    sc = [0.5, 0.3995, 0.1, 0.4, 0.1, 0.9]
    rep = one_row([0, 1, 5], [0, 3, 5], sc, 5)
    assert (rep.exact, rep.exempt, rep.counted) == (0, 1, 0)
    assert rep.max_exempt_gap == pytest.approx(5e-4)
    assert rep.exempt_rows.tolist() == [0]


def test_gap_at_the_tolerance_is_exempt_and_above_it_counts():
    base = [0.5, 0.0, 0.1, 0.4, 0.1, 0.9]
    at = list(base); at[1] = 0.4 - 0.999 * parity.TIE_TOL
    above = list(base); above[1] = 0.4 - 2 * parity.TIE_TOL
    assert one_row([0, 1, 5], [0, 3, 5], at, 5).exempt == 1
    rep = one_row([0, 1, 5], [0, 3, 5], above, 5)
    assert (rep.exempt, rep.counted) == (0, 1)
    assert rep.exempt_rows.size == 0


def test_large_gap_swap_counts():
    rep = one_row([0, 2, 5], [0, 3, 5], [0.5, 0.1, 0.1, 0.4, 0.1, 0.9], 5)
    assert rep.counted == 1


def test_missing_own_block_counts():
    # GPU list lacks the own block 5 even though the swapped scores tie
    rep = one_row([0, 3, 4], [0, 3, 5], [0.5, 0.1, 0.1, 0.4, 0.4, 0.4], 5)
    assert rep.counted == 1


def test_padding_mismatch_counts():
    rep = one_row([0, 5, -1], [0, 3, 5], [0.5, 0.1, 0.1, 0.4, 0.1, 0.9], 5)
    assert rep.counted == 1


def test_block_after_own_counts():
    # a block after the query's own can never be selected
    rep = one_row([0, 5, 6], [0, 3, 5], [0.5, 0.1, 0.1, 0.4, 0.1, 0.9, 0.4], 5)
    assert rep.counted == 1


def test_two_swaps_pair_by_rank_and_every_pair_must_be_a_tie():
    # oracle {1, 2} vs GPU {3, 4}: pairs (best of each side) = (1, 3) gap 1e-4
    # and (2, 4) gap 0.2 -> counted; with (2, 4) close as well -> exempt
    sc = np.array([0.9, 0.5, 0.4, 0.4999, 0.2, 0.0, 0.8])
    assert one_row([0, 3, 4, 6], [0, 1, 2, 6], sc, 6).counted == 1
    sc2 = sc.copy(); sc2[4] = 0.3995
    rep = one_row([0, 3, 4, 6], [0, 1, 2, 6], sc2, 6)
    assert (rep.exempt, rep.counted) == (1, 0)


def test_only_failing_groups_of_a_row_are_judged_and_rows_report_once():
    g = np.array([[[0, 5], [1, 5]], [[0, 5], [2, 5]]], np.int32)   # 2 rows x 2 groups
    o = np.array([[[0, 5], [1, 5]], [[0, 5], [3, 5]]], np.int32)
    sc = np.zeros((2, 2, 6))
    sc[1, 1, 2], sc[1, 1, 3] = 0.3, 0.3001
    # scores_fn is called with the indices of the differing rows only
    called = []

    def fn(idx):
        called.append(list(idx))
        return sc[idx]

    rep = parity.index_parity(g, o, fn, np.array([5, 5]))
    assert called == [[1]]
    assert (rep.rows, rep.exact, rep.exempt, rep.counted) == (4, 3, 1, 0)
    assert rep.exempt_rows.tolist() == [1]


# ------------------------------------------------------- index injection
@pytest.fixture(scope="module")
def small():
    s = PrefillShape(640 + 13, 9, 20, 8, 2, 32, 64, 4, 100, "bf16")
    return make_prefill_inputs(s, seed=11)


def test_injecting_the_oracles_own_selection_reproduces_its_output_bit_for_bit(small):
    V = np.nonzero(small["is_vision"])[0]
    ref = oracle.prefill(small, rows=V, want=("sel",))
    inj = oracle.prefill(small, rows=V, inject_sel=ref["sel"], want=())
    assert np.array_equal(inj["out"], ref["out"])


def test_injected_selection_is_what_the_branch_attends(small):
    V = np.nonzero(small["is_vision"])[0]
    ref = oracle.prefill(small, rows=V, want=("sel", "osel"))
    sel = ref["sel"].copy()
    # exchange the two KV groups' lists on rows with two different lists:
    # the selection branch must then follow the swapped lists
    differ = np.nonzero(np.any(sel[:, 0] != sel[:, 1], axis=1))[0]
    assert differ.size > 50
    swapped = sel.copy()
    swapped[:, [0, 1]] = sel[:, [1, 0]]
    inj = oracle.prefill(small, rows=V, inject_sel=swapped, want=("osel", "ocmp", "oswa"))
    assert not np.allclose(inj["osel"][differ], ref["osel"][differ])
    # rows whose two lists agree, and the other branches, are unchanged
    same = np.setdiff1d(np.arange(len(V)), differ)
    assert np.array_equal(inj["osel"][same], ref["osel"][same])
    again = oracle.prefill(small, rows=V, want=("ocmp", "oswa"))
    assert np.array_equal(inj["ocmp"], again["ocmp"]) and np.array_equal(inj["oswa"], again["oswa"])
    # and it equals the branch evaluated from scratch on those key sets
    # (brute-force restatement: softmax over the keys of the injected blocks)
    q = small["q"].astype(np.float64)
    k = small["k"].astype(np.float64)
    v = small["v"].astype(np.float64)
    G = q.shape[1] // k.shape[1]
    scale = 1.0 / np.sqrt(q.shape[2])
    for r in differ[:5]:
        t = r  # vision-local index (vision rows start the sequence after the text prefix)
        pos = V[t]
        for h in range(q.shape[1]):
            g = h // G
            keys = [V[j] for b in swapped[r, g] if b >= 0 for j in range(64 * b, min(64 * b + 64, t + 1))]
            s_ = scale * k[keys, g] @ q[pos, h]
            p = np.exp(s_ - s_.max())
            o = (p / p.sum()) @ v[keys, g]
            assert np.allclose(inj["osel"][r, h], o, atol=1e-12, rtol=1e-12)


def test_check_prefill_injects_gpu_selection_on_exempt_rows_only(small):
    """A 'GPU' result that is the oracle's own except one near-tie swap on one
    row: the checker must exempt it, inject it, and pass; the same swap with a
    wrong output must fail."""
    s = small["shape"]
    V = np.nonzero(small["is_vision"])[0]
    ref = oracle.prefill(small, rows=np.arange(s.n_tokens), want=("sel", "scores"))
    vloc = np.cumsum(small["is_vision"]) - 1
    sel = ref["sel"][V].copy()
    sc = ref["scores"][V]
    # find a vision row and group where the k-th and (k+1)-th candidates are close
    best = None
    for t in range(len(V)):
        cur = t // 64
        for g in range(sel.shape[1]):
            row = sc[t, g]
            cand = [b for b in range(cur) if b not in set(sel[t, g])]
            if not cand or (sel[t, g] >= 0).sum() < 2:
                continue
            chosen = [b for b in sel[t, g] if b >= 0 and b != cur]
            if not chosen:
                continue
            worst = min(chosen, key=lambda b: (row[b], -b))
            alt = max(cand, key=lambda b: (row[b], -b))
            gap = row[worst] - row[alt]
            if best is None or gap < best[0]:
                best = (gap, t, g, worst, alt)
    gap, t, g, worst, alt = best
    assert gap <= parity.TIE_TOL, "no near-tie in this small layout"
    gsel = sel.copy()
    lst = [b for b in gsel[t, g] if b >= 0 and b != worst] + [alt]
    gsel[t, g] = sorted(lst) + [-1] * (s.top_k - len(lst))
    # the 'GPU' output for that row is the oracle evaluated on the swapped list
    inj = oracle.prefill(small, rows=V[[t]], inject_sel=gsel[[t]], want=())
    out = ref["out"].copy()
    out[V[t]] = inj["out"][0]
    gpu = {"out": out.astype(np.float32), "sel": gsel}
    rep, orep, _ = parity.check_prefill(small, gpu, np.arange(s.n_tokens))
    assert rep.counted == 0 and rep.exempt == 1 and orep.ok(), (rep, orep)
    # without injection the swapped row would differ from the oracle's own output
    assert np.abs(inj["out"][0] - ref["out"][V[t]]).max() > 0
    # a wrong output on that row is caught
    bad = dict(gpu)
    bad["out"] = gpu["out"].copy()
    bad["out"][V[t]] += 0.05
    _, orep2, _ = parity.check_prefill(small, bad, np.arange(s.n_tokens))
    assert not orep2.ok()
    assert vloc[V[t]] == t


def test_selection_only_evaluation_equals_the_full_one(small):
    """The oracle's selection-only mode (no attention outputs) gives the very
    same selection, lse, scores and counts as a full evaluation."""
    rows = np.arange(small["shape"].n_tokens)
    full = oracle.prefill(small, rows=rows, want=("sel", "lse", "scores", "counts"))
    part = oracle.prefill(small, rows=rows, want=("sel", "lse", "scores", "counts"), outputs=False)
    assert "out" not in part
    for key in ("sel", "scores", "counts"):
        assert np.array_equal(part[key], full[key]), key
    assert np.array_equal(np.isnan(part["lse"]), np.isnan(full["lse"]))
    m = ~np.isnan(full["lse"])
    assert np.array_equal(part["lse"][m], full["lse"][m])
