"""GPU decode (nsa_decode) parity against the fp64 oracle through the C ABI.

Both sides consume the same compressed caches (pooled by the oracle, rounded
to bf16). Tolerances as for prefill: indices exact up to near-ties with an
oracle score gap <= 1e-3; outputs max |d| <= 1e-2, mean |d| <= 1e-3."""
import numpy as np
import pytest
import torch

from oracle import parity
from sparse_attention_long_nsa_amd import binding
from sparse_attention_long_nsa_amd.inputs import (
    DECODE_PRESETS, DecodeShape, PrefillShape, make_decode_inputs, make_prefill_inputs, round_to_bf16)

pytestmark = pytest.mark.gpu


def bf(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(torch.bfloat16)


def run_decode(inp, kc, vc):
    s = inp["shape"]
    r = binding.decode(bf(inp["q"]), bf(inp["k_cache"]), bf(inp["v_cache"]), bf(kc), bf(vc),
                       torch.from_numpy(inp["gates"]).cuda(), s.top_k, s.window, block=s.block,
                       want_sel=True, want_lse=True)
    torch.cuda.synchronize()
    return r["out"].cpu().numpy(), r["sel_idx"].cpu().numpy(), r["lse"].cpu().numpy()


def check(inp, name):
    print(f"\n[case] {name}: {inp['shape']}", flush=True)
    kc, vc = parity.decode_inputs_cmp(inp, round_to_bf16)
    out, sel, lse = run_decode(inp, kc, vc)
    rep, orep, ref = parity.check_decode(inp, kc, vc, out, sel)
    print(rep, "|", orep, flush=True)
    assert rep.counted == 0, rep
    assert orep.ok(), orep
    np.testing.assert_allclose(lse, ref["lse"], rtol=0, atol=2e-3)
    return out, sel


@pytest.mark.parametrize("shape", [
    DecodeShape(3, 4096, 28, 4, 128, 64, 16, 512),
    DecodeShape(2, 640, 4, 1, 64, 64, 4, 100),
    DecodeShape(2, 1024, 8, 2, 128, 64, 32, 1024),   # k covers every block, window = cache
    DecodeShape(1, 128, 6, 3, 64, 64, 5, 1),         # fewer blocks than k
    DecodeShape(4, 8192 + 64, 16, 2, 128, 64, 8, 96),
    DecodeShape(1, 2100 * 64, 8, 2, 128, 64, 16, 512),  # > 2048 candidates per row
])
def test_decode_small(shape):
    check(make_decode_inputs(shape, seed=11), "decode_small")


def test_decode_full_size_preset():
    check(make_decode_inputs(DECODE_PRESETS["decode_16x128k"], seed=0), "decode_16x128k")


def test_decode_equals_prefill_last_row_on_gpu():
    L = 4096
    s = PrefillShape(L, 0, 0, 28, 4, 128, 64, 16, 512, "bf16")
    inp = make_prefill_inputs(s, seed=12)
    print(f"\n[case] decode_vs_prefill: {s}", flush=True)
    dev = {k: bf(inp[k]) for k in ("q", "k", "v", "w_k", "w_v")}
    g = torch.from_numpy(inp["gates"]).cuda()
    pre = binding.prefill(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"], dev["w_v"], g,
                          16, 512, want_kcmp=True, want_sel=True)
    torch.cuda.synchronize()
    kc = round_to_bf16(pre["k_cmp"].cpu().numpy())[None]
    vc = round_to_bf16(pre["v_cmp"].cpu().numpy())[None]
    dinp = dict(q=inp["q"][L - 1][None], k_cache=inp["k"][None], v_cache=inp["v"][None],
                gates=inp["gates"][L - 1][None], shape=DecodeShape(1, L, 28, 4, 128, 64, 16, 512))
    out, sel, _ = run_decode(dinp, kc, vc)
    p_out = pre["out"][L - 1].cpu().numpy()
    p_sel = pre["sel_idx"][L - 1].cpu().numpy()
    assert np.array_equal(sel[0], p_sel), (sel[0], p_sel)
    rep = parity.compare(out[0], p_out)
    print(rep, flush=True)
    assert rep.ok(), rep
