"""Every supported head shape on the GPU: head_dim 64 with 1..8 query heads
per KV head and head_dim 128 with 1..7 (each is its own kernel instance),
through prefill (all rows), decode and the dense mode, against the fp64
oracle at the usual bar. Each case prints its shape before touching the GPU."""
import numpy as np
import pytest
import torch

import oracle
from oracle import parity
from sparse_attention_long_nsa_amd import binding
from sparse_attention_long_nsa_amd.inputs import DecodeShape, PrefillShape, make_decode_inputs, make_prefill_inputs, round_to_bf16

from gpu_util import run_prefill, upload

pytestmark = pytest.mark.gpu

HEADS = [(64, g) for g in range(1, 9)] + [(128, g) for g in range(1, 8)]


@pytest.mark.parametrize("d,G", HEADS)
def test_prefill_every_head_shape(d, G):
    s = PrefillShape(700, 13, 40, 2 * G, 2, d, 64, 4, 100, "bf16")
    print(f"\n[case] prefill heads: {s}", flush=True)
    inp = make_prefill_inputs(s, seed=100 + d + G)
    gpu = run_prefill(inp)
    rep, orep, _ = parity.check_prefill(inp, gpu, np.arange(s.n_tokens))
    print(rep, "|", orep, flush=True)
    assert rep.counted == 0, rep
    assert orep.ok(), orep


@pytest.mark.parametrize("d,G", HEADS)
def test_decode_every_head_shape(d, G):
    s = DecodeShape(2, 64 * 11 + 9, 2 * G, 2, d, 64, 5, 90)
    print(f"\n[case] decode heads: {s}", flush=True)
    inp = make_decode_inputs(s, seed=200 + d + G)
    kc, vc = parity.decode_inputs_cmp(inp, round_to_bf16)
    L, cap = s.cache_len, 64 * 12

    def dev(x, rows):
        buf = np.zeros((x.shape[0], rows) + x.shape[2:], dtype=np.float32)
        buf[:, : x.shape[1]] = x
        return torch.from_numpy(buf).cuda().to(torch.bfloat16)

    q = torch.from_numpy(np.ascontiguousarray(inp["q"])).cuda().to(torch.bfloat16)
    r = binding.decode(q, dev(inp["k_cache"], cap), dev(inp["v_cache"], cap),
                       dev(kc, cap // 64), dev(vc, cap // 64), torch.from_numpy(inp["gates"]).cuda(), s.top_k,
                       s.window, want_sel=True, cache_len=L)
    torch.cuda.synchronize()
    rep, orep, _ = parity.check_decode(inp, kc, vc, r["out"].cpu().numpy(), r["sel_idx"].cpu().numpy())
    print(rep, "|", orep, flush=True)
    assert rep.counted == 0, rep
    assert orep.ok(), orep


@pytest.mark.parametrize("d,G", HEADS)
def test_dense_every_head_shape(d, G):
    s = PrefillShape(300, 0, 37, 2 * G, 2, d, 64, 4, 100, "bf16")
    print(f"\n[case] dense heads: {s}", flush=True)
    inp = make_prefill_inputs(s, seed=300 + d + G)
    dv = upload(inp)
    r = binding.prefill_dense(dv["q"], dv["k"], dv["v"])
    torch.cuda.synchronize()
    rep = parity.compare(r["out"].cpu().numpy(), oracle.dense(inp))
    print(rep, flush=True)
    assert rep.ok(), rep


# fp32 inputs: split-bf16 block scores need G * d <= 512
HEADS_FP32 = [(64, g) for g in range(1, 9)] + [(128, g) for g in range(1, 5)]


@pytest.mark.parametrize("d,G", HEADS_FP32)
def test_prefill_fp32_every_head_shape(d, G):
    s = PrefillShape(650, 7, 21, 2 * G, 2, d, 64, 4, 100, "fp32")
    print(f"\n[case] prefill fp32 heads: {s}", flush=True)
    inp = make_prefill_inputs(s, seed=400 + d + G)
    gpu = run_prefill(inp)
    rep, orep, _ = parity.check_prefill(inp, gpu, np.arange(s.n_tokens))
    print(rep, "|", orep, flush=True)
    assert rep.counted == 0, rep
    assert orep.ok(), orep
