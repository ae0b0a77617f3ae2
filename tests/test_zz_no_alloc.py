"""GPU test of nsa_decode_noalloc (decode with the library's fixed device
scratch, for callers that cannot allocate), through the C ABI: on two calls
in a row, the second with a smaller input, its outputs equal those of
nsa_decode on the same inputs bit for bit (same kernels, same order of
arithmetic), and a step too large for the scratch is refused."""
import numpy as np
import pytest
import torch

from oracle import parity
from sparse_attention_long_nsa_amd import binding
from sparse_attention_long_nsa_amd.inputs import DecodeShape, make_decode_inputs, round_to_bf16

pytestmark = pytest.mark.gpu


def bf(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(torch.bfloat16)


def device_inputs(shape, seed):
    inp = make_decode_inputs(shape, seed=seed)
    kc, vc = parity.decode_inputs_cmp(inp, round_to_bf16)
    return dict(q=bf(inp["q"]), k_cache=bf(inp["k_cache"]), v_cache=bf(inp["v_cache"]), k_cmp=bf(kc),
                v_cmp=bf(vc), gate_logits=torch.from_numpy(inp["gates"]).cuda())


def test_noalloc_decode_equals_decode_on_two_calls_the_second_smaller():
    shapes = [DecodeShape(8, 65536 + 37, 28, 4, 128, 64, 16, 512),   # partial own block
              DecodeShape(3, 4096, 28, 4, 128, 64, 16, 512)]
    for i, s in enumerate(shapes):
        print(f"\n[case] noalloc call {i}: {s}", flush=True)
        dev = device_inputs(s, seed=40 + i)
        # the second workload fits in a prefix of the cache buffers: capacity
        # stays the array's row count, cache_len the used rows
        ref = binding.decode(**dev, top_k=s.top_k, window=s.window, want_sel=True, want_lse=True)
        out = torch.full((s.batch, 28, 128), float("nan"), device="cuda")
        sel = torch.full((s.batch, 4, s.top_k), -7, dtype=torch.int32, device="cuda")
        lse = torch.full((s.batch, 28), float("nan"), device="cuda")
        got = binding.decode_noalloc(**dev, top_k=s.top_k, window=s.window, out=out, sel_idx=sel, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(got["out"], ref["out"]), i
        assert torch.equal(got["sel_idx"], ref["sel_idx"]), i
        assert torch.equal(got["lse"], ref["lse"]), i
        assert torch.isfinite(got["out"]).all()


def test_noalloc_decode_refuses_a_step_beyond_its_scratch():
    # 64 sequences of 524,288 tokens need about 117 MB of scratch: refused
    # before anything is launched (the caches are never read)
    s = DecodeShape(64, 524288, 28, 4, 128, 64, 16, 512)
    desc = binding.DecodeDesc(s.batch, s.cache_len, 28, 4, 128, 64, 16, 512, 0.0, 0, 0)
    assert binding.decode_workspace_size(desc) > binding.DECODE_NOALLOC_SCRATCH_BYTES
    fake = torch.empty(16, dtype=torch.uint8, device="cuda")
    p = fake.data_ptr()
    st = binding.lib().nsa_decode_noalloc(__import__("ctypes").byref(desc), p, p, p, p, p, p, p, None, None, None)
    assert st == binding.NSA_ERR_WORKSPACE
