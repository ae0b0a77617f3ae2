"""Every entry point reads only workspace it wrote in the same call: each
runs with a workspace filled with 0xFF bytes (NaN as fp32, -1 as int32) and
must give exactly what it gives with a zeroed workspace, at oracle parity.
Each case prints its name before touching the GPU."""
import numpy as np
import pytest
import torch

from oracle import parity
from sparse_attention_long_nsa_amd import binding
from sparse_attention_long_nsa_amd.inputs import (
    DecodeShape, PrefillShape, make_decode_inputs, make_prefill_inputs, mask_from_runs, relayout, round_to_bf16)

from gpu_util import upload

pytestmark = pytest.mark.gpu

BIG = 1 << 28  # bytes, more than any case here needs


def filled(byte):
    return torch.full((BIG,), byte, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("runs", [None, [("t", 9), ("v", 500), ("t", 3), ("v", 700), ("t", 20)]])
def test_prefill_workspace_contents_do_not_matter(runs):
    s = PrefillShape(1200, 9, 23, 28, 4, 128, 64, 16, 200, "bf16")
    print(f"\n[case] prefill workspace: {s} {runs}", flush=True)
    inp = make_prefill_inputs(s, seed=61)
    if runs is not None:
        inp = relayout(inp, mask_from_runs(runs))
    dev = upload(inp)
    res = []
    for byte in (0, 255):
        r = binding.prefill(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"], dev["w_v"], dev["gates"],
                            s.top_k, s.window, want_sel=True, want_lse=True, workspace=filled(byte))
        torch.cuda.synchronize()
        res.append({k: r[k].cpu().numpy() for k in ("out", "sel_idx", "lse")})
    for k in ("out", "sel_idx", "lse"):
        assert np.array_equal(res[0][k], res[1][k]), k
    rep, orep, _ = parity.check_prefill(inp, {"out": res[1]["out"], "sel": res[1]["sel_idx"]},
                                        np.arange(len(inp["is_vision"])))
    assert rep.counted == 0 and orep.ok(), (rep, orep)


@pytest.mark.parametrize("shape", [
    DecodeShape(2, 1024, 8, 2, 128, 64, 32, 1024),   # k above the block count: unused selection slots
    DecodeShape(3, 64 * 9 + 5, 28, 4, 128, 64, 16, 100),
])
def test_decode_workspace_contents_do_not_matter(shape):
    print(f"\n[case] decode workspace: {shape}", flush=True)
    inp = make_decode_inputs(shape, seed=62)
    kc, vc = parity.decode_inputs_cmp(inp, round_to_bf16)
    L, cap = shape.cache_len, -(-shape.cache_len // 64) * 64

    def dv(x, rows):
        buf = np.zeros((x.shape[0], rows) + x.shape[2:], dtype=np.float32)
        buf[:, : x.shape[1]] = x
        return torch.from_numpy(buf).cuda().to(torch.bfloat16)

    q = torch.from_numpy(np.ascontiguousarray(inp["q"])).cuda().to(torch.bfloat16)
    args = (q, dv(inp["k_cache"], cap), dv(inp["v_cache"], cap), dv(kc, cap // 64), dv(vc, cap // 64),
            torch.from_numpy(inp["gates"]).cuda(), shape.top_k, shape.window)
    res = []
    for byte in (0, 255):
        r = binding.decode(*args, want_sel=True, want_lse=True, cache_len=L, workspace=filled(byte))
        torch.cuda.synchronize()
        res.append({k: r[k].cpu().numpy() for k in ("out", "sel_idx", "lse")})
    for k in ("out", "sel_idx", "lse"):
        assert np.array_equal(res[0][k], res[1][k]), k
    rep, orep, _ = parity.check_decode(inp, kc, vc, res[1]["out"], res[1]["sel_idx"])
    assert rep.counted == 0 and orep.ok(), (rep, orep)


def test_dense_and_varlen_workspace_contents_do_not_matter():
    s = PrefillShape(700, 5, 30, 28, 4, 128, 64, 8, 100, "bf16")
    print(f"\n[case] dense/varlen workspace: {s}", flush=True)
    inp = make_prefill_inputs(s, seed=63)
    dev = upload(inp)
    outs = []
    for byte in (0, 255):
        a = binding.prefill_dense(dev["q"], dev["k"], dev["v"], want_lse=True, workspace=filled(byte))
        cu = np.array([0, 300, len(inp["is_vision"])], np.int64)
        b = binding.prefill_varlen(dev["q"], dev["k"], dev["v"], cu, inp["is_vision"], dev["w_k"], dev["w_v"],
                                   dev["gates"], s.top_k, s.window, want_sel=True, workspace=filled(byte))
        torch.cuda.synchronize()
        outs.append([a["out"].cpu().numpy(), a["lse"].cpu().numpy(), b["out"].cpu().numpy(),
                     b["sel_idx"].cpu().numpy()])
    for x, y in zip(*outs):
        assert np.array_equal(x, y)
