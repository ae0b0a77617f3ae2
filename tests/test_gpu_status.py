"""The prefill workspace's status word, through the C ABI on the GPU.

* A bounded wait that gives up is reported: with the spin limit forced down
  from the host (a test aid of the library), the selection kernel's waits give
  up at once, every kernel still ends normally, the outputs are invalid (NaN)
  and nsa_workspace_status reports NSA_ERR_KERNEL with bit 0 set; with the
  default limit restored the same workspace reports success and the outputs
  are at oracle parity again.
* fp16 range (queries, values and compressed keys/values are used in fp16):
  values scaled by 2^10 stay in range -- no flag, and the output scales
  exactly with v (linearity in v), so out / 2^10 is at parity with the
  oracle on the unscaled inputs; values past 65504 set bit 1. The
  backward's workspace carries the same word: dout or keys past 65504 set
  bit 1 there too.
"""
import numpy as np
import pytest
import torch

from oracle import parity
from sparse_attention_long_nsa_amd import binding
from sparse_attention_long_nsa_amd.inputs import PrefillShape, make_prefill_inputs

from gpu_util import upload

pytestmark = pytest.mark.gpu

SHAPE = PrefillShape(2048 + 19, 16, 48, 28, 4, 128, 64, 16, 256, "bf16")


def run(inp, dev, workspace=None):
    s = inp["shape"]
    r = binding.prefill(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"], dev["w_v"], dev["gates"],
                        s.top_k, s.window, want_sel=True, workspace=workspace)
    torch.cuda.synchronize()
    return r


def test_forced_give_up_is_reported_and_recovers():
    inp = make_prefill_inputs(SHAPE, seed=21)
    print(f"\n[case] forced give-up: {SHAPE}", flush=True)
    dev = upload(inp)
    try:
        binding.set_spin_limit(1)
        r = run(inp, dev)
        flags = binding.workspace_status(r["workspace"])
        print("status word with spin limit 1:", flags, flush=True)
        assert flags & 1
        V = np.nonzero(inp["is_vision"])[0]
        assert not np.all(np.isfinite(r["out"].cpu().numpy()[V]))
    finally:
        binding.set_spin_limit(0)
    r2 = run(inp, dev, workspace=r["workspace"])
    assert binding.workspace_status(r2["workspace"]) == 0
    gpu = {"out": r2["out"].cpu().numpy(), "sel": r2["sel_idx"].cpu().numpy()}
    rep, orep, _ = parity.check_prefill(inp, gpu, parity.sample_rows(inp, n_random=128, n_text=8))
    print(rep, "|", orep, flush=True)
    assert rep.counted == 0 and orep.ok(), (rep, orep)


def test_large_values_in_range_scale_exactly():
    inp = make_prefill_inputs(SHAPE, seed=22)
    print(f"\n[case] v x 2^10: {SHAPE}", flush=True)
    big = dict(inp)
    big["v"] = inp["v"] * 1024.0  # exact in bf16; |v| stays far below 65504
    dev = upload(big)
    r = run(big, dev)
    assert binding.workspace_status(r["workspace"]) == 0
    gpu = {"out": r["out"].cpu().numpy() / 1024.0, "sel": r["sel_idx"].cpu().numpy()}
    rep, orep, _ = parity.check_prefill(inp, gpu, parity.sample_rows(inp, n_random=128, n_text=8))
    print(rep, "|", orep, flush=True)
    assert rep.counted == 0 and orep.ok(), (rep, orep)


@pytest.mark.parametrize("what", ["v", "q"])
def test_values_past_fp16_range_are_flagged(what):
    inp = make_prefill_inputs(SHAPE, seed=23)
    print(f"\n[case] {what} past fp16 range: {SHAPE}", flush=True)
    bad = dict(inp)
    x = np.array(inp[what], copy=True)
    V = np.nonzero(inp["is_vision"])[0]
    x[V[700:710]] *= 2.0 ** 17  # a few vision rows beyond 65504
    bad[what] = x
    dev = upload(bad)
    r = run(bad, dev)
    flags = binding.workspace_status(r["workspace"])
    print("status word:", flags, flush=True)
    assert flags & 2


BWD_SHAPE = PrefillShape(700, 8, 24, 28, 4, 128, 64, 8, 128, "bf16")


@pytest.mark.parametrize("what", ["none", "dout", "k"])
def test_backward_flags_values_past_fp16_range(what):
    """The backward's workspace carries the same status word: inputs in range
    leave it 0; dout or keys scaled past 65504 (converted to fp16 for the
    matrix cores) set bit 1."""
    from sparse_attention_long_nsa_amd.inputs import make_output_grad
    import oracle
    inp = make_prefill_inputs(BWD_SHAPE, seed=24)
    print(f"\n[case] backward, {what} past fp16 range: {BWD_SHAPE}", flush=True)
    vis = np.asarray(inp["is_vision"]).astype(bool)
    sel = oracle.prefill(inp, want=("sel",))["sel"][vis]
    dout = make_output_grad((BWD_SHAPE.n_tokens, BWD_SHAPE.n_q_heads, BWD_SHAPE.head_dim), seed=25)
    bad = dict(inp)
    if what == "dout":
        dout[100:104] *= 2.0 ** 17
    elif what == "k":
        x = np.array(inp["k"], copy=True)
        x[300:302] *= 2.0 ** 17
        bad["k"] = x
    dev = upload(bad)
    ws = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    binding.prefill_backward(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"], dev["w_v"], dev["gates"],
                             torch.from_numpy(sel).to("cuda:0"), torch.from_numpy(dout).to("cuda:0"),
                             BWD_SHAPE.top_k, BWD_SHAPE.window, workspace=ws)
    flags = binding.workspace_status(ws)
    print("status word:", flags, flush=True)
    assert (flags & 2) == (0 if what == "none" else 2)


def test_backward_forced_give_up_is_reported_and_recovers():
    """The backward's query-side selection ring waits are bounded too: with
    the spin limit forced down they give up, every kernel still ends, bit 0
    of the status word is set and dq holds NaN; with the default limit the
    next call is clean and bitwise equal to a call that never gave up."""
    from sparse_attention_long_nsa_amd.inputs import make_output_grad
    import oracle
    inp = make_prefill_inputs(BWD_SHAPE, seed=26)
    print(f"\n[case] backward forced give-up: {BWD_SHAPE}", flush=True)
    vis = np.asarray(inp["is_vision"]).astype(bool)
    sel = torch.from_numpy(oracle.prefill(inp, want=("sel",))["sel"][vis]).to("cuda:0")
    dout = torch.from_numpy(make_output_grad((BWD_SHAPE.n_tokens, BWD_SHAPE.n_q_heads, BWD_SHAPE.head_dim),
                                             seed=27)).to("cuda:0")
    dev = upload(inp)
    ws = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")

    def call():
        return binding.prefill_backward(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"], dev["w_v"],
                                        dev["gates"], sel, dout, BWD_SHAPE.top_k, BWD_SHAPE.window, workspace=ws)

    clean = {n: t.cpu().numpy() for n, t in call().items()}
    assert binding.workspace_status(ws) == 0
    try:
        binding.set_spin_limit(1)
        r = call()
        flags = binding.workspace_status(ws)
        print("status word with spin limit 1:", flags, flush=True)
        assert flags & 1
        assert not np.all(np.isfinite(r["dq"].cpu().numpy()))
    finally:
        binding.set_spin_limit(0)
    again = {n: t.cpu().numpy() for n, t in call().items()}
    assert binding.workspace_status(ws) == 0
    for n in clean:
        assert np.array_equal(clean[n], again[n]), n
