"""GPU parity of the varlen batch (nsa_prefill_varlen): several independent
sequences in one call, each checked against the fp64 oracle on that sequence
alone and against a separate nsa_prefill call (bit for bit). Same bar as the
single-sequence tests. Each case prints its name before touching the GPU."""
import numpy as np
import pytest
import torch

from oracle import parity
from sparse_attention_long_nsa_amd import binding
from sparse_attention_long_nsa_amd.inputs import PrefillShape, make_prefill_inputs, mask_from_runs, relayout

from gpu_util import run_prefill, upload

pytestmark = pytest.mark.gpu


def sequences(hq, hkv, d, k, w, dtype="bf16"):
    """Four sequences of one layer (shared compression maps): text around a
    vision run, whole blocks of vision only, text only, several vision runs."""
    specs = [(PrefillShape(700, 20, 30, hq, hkv, d, 64, k, w, dtype), None),
             (PrefillShape(64 * 5, 0, 0, hq, hkv, d, 64, k, w, dtype), None),
             (PrefillShape(0, 50, 0, hq, hkv, d, 64, k, w, dtype), None),
             (PrefillShape(800, 0, 15, hq, hkv, d, 64, k, w, dtype),
              [("v", 300), ("t", 5), ("v", 500), ("t", 10)])]
    seqs = []
    for i, (s, runs) in enumerate(specs):
        inp = make_prefill_inputs(s, seed=40 + i)
        if runs is not None:
            inp = relayout(inp, mask_from_runs(runs))
        if seqs:
            inp["w_k"], inp["w_v"] = seqs[0]["w_k"], seqs[0]["w_v"]
        seqs.append(inp)
    return seqs


def concat(seqs):
    cat = {x: np.concatenate([s[x] for s in seqs]) for x in ("q", "k", "v", "gates", "is_vision")}
    cat.update(w_k=seqs[0]["w_k"], w_v=seqs[0]["w_v"], shape=seqs[0]["shape"])
    cu = np.cumsum([0] + [len(s["is_vision"]) for s in seqs]).astype(np.int64)
    return cat, cu


@pytest.mark.parametrize("cfg", [(28, 4, 128, 8, 128, "bf16"), (8, 2, 64, 4, 64, "bf16"), (4, 1, 64, 3, 100, "fp32")])
def test_varlen_matches_each_sequence(cfg):
    hq, hkv, d, k, w, dt = cfg
    print(f"\n[case] varlen: hq {hq} hkv {hkv} d {d} k {k} w {w} {dt}", flush=True)
    seqs = sequences(hq, hkv, d, k, w, dt)
    cat, cu = concat(seqs)
    dev = upload(cat)
    r = binding.prefill_varlen(dev["q"], dev["k"], dev["v"], cu, cat["is_vision"], dev["w_k"], dev["w_v"],
                               dev["gates"], k, w, want_sel=True, want_kcmp=True, want_lse=True)
    torch.cuda.synchronize()
    out = r["out"].cpu().numpy()
    sel = r["sel_idx"].cpu().numpy()
    kcmp = r["k_cmp"].cpu().numpy()
    lse = r["lse"].cpu().numpy()
    vis0 = blk0 = 0
    for i, s in enumerate(seqs):
        a, b = cu[i], cu[i + 1]
        nv = int(s["is_vision"].sum())
        nb = nv // 64
        gpu = {"out": out[a:b], "sel": sel[vis0:vis0 + nv]}
        rep, orep, _ = parity.check_prefill(s, gpu, np.arange(b - a))
        print(i, rep, "|", orep, flush=True)
        if rep is not None:
            assert rep.counted == 0, (i, rep)
        assert orep.ok(), (i, orep)
        one = run_prefill(s, kcmp=True, lse=True)  # the same sequence alone
        assert np.array_equal(one["out"], gpu["out"]), i
        assert np.array_equal(one["sel"], gpu["sel"]), i
        assert np.array_equal(one["kcmp"], kcmp[blk0:blk0 + nb]), i
        assert np.array_equal(one["lse"], lse[vis0:vis0 + nv]), i
        vis0 += nv
        blk0 += nb
