#!/usr/bin/env python3
"""Benchmark of the VideoNSA attention layer forward pass (nsa_prefill) on one
MI355X, at 131,072 vision + 512 text tokens (Qwen2.5-VL-7B layer shape: 28
query heads, 4 KV heads, d = 128, bf16), top-32 blocks of 64 and a 256-token
window -- the paper's own defaults (VideoNSA paper summary page, "Method").

One step = one nsa_prefill call over the whole sequence with inputs resident
in HBM. Prints one JSON line on stdout; everything else goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NSA attention tokens/s/layer at 128K vision tokens; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector peak
SWEEP = ((8, 1024), (16, 512))  # fixed-budget trade of blocks against window


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def closed_form_work(shape, n_text_positions):
    """Algorithmic work per kernel (flops for matrix kernels, bytes for
    streaming ones) of one layer call, from the per-query key counts."""
    s = shape
    B, d, hq, hkv, k, w = s.block, s.head_dim, s.n_q_heads, s.n_kv_heads, s.top_k, s.window
    t = np.arange(s.n_vis, dtype=np.int64)
    cur = t // B
    n_cmp = (t + 1) // B
    n_sel = (np.minimum(k, cur + 1) - 1) * B + (t - cur * B + 1)
    n_swa = np.minimum(w, t + 1)
    text_keys = np.asarray(n_text_positions, dtype=np.int64) + 1
    n_blk = s.n_vis // B
    n_frames = -(-s.n_vis // B)
    f4 = 4.0 * d * hq
    kv_block = 2 * B * d
    return {
        # the maps: block means in (fp32), each result out twice in fp16 (plain
        # and packed); the means themselves come out of pack_kv's read of the rows
        "cmp_pool": ("bytes", 2.0 * n_blk * hkv * d * 4 + 2.0 * n_blk * hkv * d * 2 * 2),
        "cmp_attn": ("flops", f4 * float(n_cmp.sum())),
        "blk_score_topk": ("bytes", 4.0 * hkv * float(cur.sum()) + 4.0 * s.n_vis * hkv * k),
        "swa_attn": ("flops", f4 * float(n_swa.sum())),
        "pack_kv": ("bytes", 4.0 * s.n_vis * hkv * d + 2.0 * n_frames * hkv * kv_block + 8.0 * n_blk * hkv * d),
        "pack_cmp": ("bytes", 4.0 * n_blk * hkv * d + 2.0 * (-(-n_blk // B)) * hkv * kv_block),
        "pack_text": ("bytes", 4.0 * len(text_keys) * hkv * d + 2.0 * (-(-len(text_keys) // B)) * hkv * kv_block),
        "sel_attn": ("flops", f4 * float(n_sel.sum())),
        "text_attn": ("flops", f4 * float(text_keys.sum())),
    }


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def pmc_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary for
    this kernel and workload, or None when the kernel source changed since."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src) or source_digest(src) != rec["source_sha256_16"]:
        return None
    return float(rec["hbm_bytes_per_launch"])


def run_gpu(inp, dev, top_k, window, steps, warmup, per_kernel):
    import torch
    from sparse_attention_long_nsa_amd import binding
    s = inp["shape"]

    def call(out, ws):
        return binding.prefill(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"],
                               dev["w_v"], dev["gates"], top_k, window, block=s.block,
                               out=out, workspace=ws)

    r = call(None, None)
    out, ws = r["out"], r["workspace"]
    for _ in range(warmup):
        call(out, ws)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call(out, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kernels = None
    if per_kernel:
        binding.timing_reset()
        binding.timing_enable(True)
        for _ in range(steps):
            call(out, ws)
        torch.cuda.synchronize()
        kernels = {n: (tot / cnt, cnt) for n, (tot, cnt) in binding.timing_read().items()}
        binding.timing_enable(False)
        binding.timing_reset()
    return ms, kernels, out


def run_spans_bench(inp, shape, steps, warmup, one_run_ms):
    """The same tokens with the vision tokens in several runs: 8 clips of
    16,384 vision tokens, each after 64 of the text tokens (row maps)."""
    import torch
    from sparse_attention_long_nsa_amd.inputs import SPAN_LAYOUTS, mask_from_runs, relayout
    m = mask_from_runs(SPAN_LAYOUTS["8clips"])
    if len(m) != shape.n_tokens or int(m.sum()) != shape.n_vis:
        return None
    mi = relayout(inp, m)
    dev = {k: torch.from_numpy(mi[k]).to("cuda:0").to(torch.bfloat16).contiguous()
           for k in ("q", "k", "v", "w_k", "w_v")}
    dev["gates"] = torch.from_numpy(mi["gates"]).to("cuda:0")
    ms, kern, _ = run_gpu(mi, dev, shape.top_k, shape.window, steps, warmup, True)
    log(f"8 clips: {ms:.3f} ms/step ({ms / one_run_ms:.4f} x one run)")

    # the same rows as 8 independent sequences of one clip each (varlen batch)
    from sparse_attention_long_nsa_amd import binding
    per = len(m) // 8
    cu = np.arange(9, dtype=np.int64) * per

    def call(out, ws):
        return binding.prefill_varlen(dev["q"], dev["k"], dev["v"], cu, m, dev["w_k"], dev["w_v"],
                                      dev["gates"], shape.top_k, shape.window, out=out, workspace=ws)

    r = call(None, None)
    out, ws = r["out"], r["workspace"]
    for _ in range(warmup):
        call(out, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call(out, ws)
    e1.record()
    torch.cuda.synchronize()
    vms = e0.elapsed_time(e1) / steps
    del dev, out, ws, r
    log(f"varlen 8 x {per}: {vms:.3f} ms/step")
    return {"layout": "8 clips of 16,384 vision tokens, 64 text tokens before each",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(shape.n_tokens / (ms * 1e-3), 1),
            "vs_one_run": round(ms / one_run_ms, 4),
            "kernels_ms": {n: round(t, 4) for n, (t, _) in sorted(kern.items(), key=lambda x: -x[1][0])},
            "varlen_8_sequences": {"sequence": f"{per} tokens (64 text, then 16,384 vision)",
                                   "ms_per_step": round(vms, 4),
                                   "tokens_per_s": round(shape.n_tokens / (vms * 1e-3), 1)}}


def run_dense_bench(dev, shape, steps, warmup, nsa_ms):
    """Dense-NSA mode on the same tokens: dense causal GQA over all of them."""
    import torch
    from sparse_attention_long_nsa_amd import binding
    r = binding.prefill_dense(dev["q"], dev["k"], dev["v"])
    out, ws = r["out"], r["workspace"]
    for _ in range(warmup):
        binding.prefill_dense(dev["q"], dev["k"], dev["v"], out=out, workspace=ws)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        binding.prefill_dense(dev["q"], dev["k"], dev["v"], out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    binding.timing_reset()
    binding.timing_enable(True)
    for _ in range(steps):
        binding.prefill_dense(dev["q"], dev["k"], dev["v"], out=out, workspace=ws)
    torch.cuda.synchronize()
    kern = {k: {"avg_ms": round(tot / cnt, 4), "launches": cnt}
            for k, (tot, cnt) in binding.timing_read().items()}
    binding.timing_enable(False)
    binding.timing_reset()
    n = shape.n_tokens
    flops = 4.0 * shape.head_dim * shape.n_q_heads * n * (n + 1) / 2
    tf = flops / (ms * 1e-3) / 1e12
    log(f"dense: {ms:.3f} ms/step, {tf:.1f} TF/s ({nsa_ms / ms:.4f} of its time for NSA)")
    return {"ms_per_step": round(ms, 3), "tokens_per_s": round(n / (ms * 1e-3), 1),
            "algorithmic_tflop": round(flops / 1e12, 3), "tflops": round(tf, 1),
            "mfma_peak_frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "nsa_speedup": round(ms / nsa_ms, 2), "steps": steps, "kernels": kern}


GATE_D_MODEL, GATE_D_HIDDEN = 3584, 1024  # Qwen2.5-VL-7B width; the MLP width is not given


def run_gate_bench(shape, steps, warmup):
    """Gate prologue on the layer's tokens: hidden states [N, 3584] -> gate
    logits [N, Hq, 3] through a 1,024-unit SiLU MLP."""
    import torch
    from sparse_attention_long_nsa_amd import binding
    from sparse_attention_long_nsa_amd.inputs import make_gate_inputs
    n, hq = shape.n_tokens, shape.n_q_heads
    g = make_gate_inputs(n, GATE_D_MODEL, GATE_D_HIDDEN, hq, seed=0)
    d = {k: torch.from_numpy(g[k]).to("cuda:0").to(torch.bfloat16).contiguous() for k in ("x", "w1", "w2")}
    b1, b2 = torch.from_numpy(g["b1"]).to("cuda:0"), torch.from_numpy(g["b2"]).to("cuda:0")
    del g

    def call(out=None, ws=None):
        return binding.gate_logits(d["x"], d["w1"], b1, d["w2"], b2, hq, "silu", out=out, workspace=ws)
    out = call()
    ws = torch.empty(binding.gate_workspace_size(binding.GateDesc(n, GATE_D_MODEL, GATE_D_HIDDEN, hq, 0, 0)),
                     dtype=torch.uint8, device="cuda:0")
    for _ in range(warmup):
        call(out, ws)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call(out, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    binding.timing_reset()
    binding.timing_enable(True)
    for _ in range(steps):
        call(out, ws)
    torch.cuda.synchronize()
    kern = {k: round(tot / cnt, 4) for k, (tot, cnt) in binding.timing_read().items()}
    binding.timing_enable(False)
    binding.timing_reset()
    flops_h = 2.0 * n * GATE_D_MODEL * GATE_D_HIDDEN
    bytes_o = 2.0 * n * GATE_D_HIDDEN + 4.0 * n * 3 * hq  # read the fp16 hidden layer, write the logits
    res = {"ms_per_step": round(ms, 4), "n_tokens": n, "d_model": GATE_D_MODEL, "d_hidden": GATE_D_HIDDEN,
           "activation": "silu", "steps": steps, "kernels": kern}
    if "gate_hidden" in kern:
        tf = flops_h / (kern["gate_hidden"] * 1e-3) / 1e12
        res["gate_hidden"] = {"tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    if "gate_out" in kern:
        gbs = bytes_o / (kern["gate_out"] * 1e-3) / 1e9
        res["gate_out"] = {"gbs": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
    log(f"gate prologue: {res}")
    return res


BWD_SHAPE = dict(n_vis=4096, n_text_after=512)  # a short context with the headline's heads, k and w


def run_backward_bench(shape, steps, warmup):
    """Backward pass (training) of the layer, reusing the forward's
    selection; reports time per call and the rate of algorithmic flops."""
    import torch
    from sparse_attention_long_nsa_amd import binding
    from sparse_attention_long_nsa_amd.inputs import make_output_grad, make_prefill_inputs
    s = shape
    inp = make_prefill_inputs(s, seed=0)
    dev = {k: torch.from_numpy(inp[k]).to("cuda:0").to(torch.bfloat16).contiguous()
           for k in ("q", "k", "v", "w_k", "w_v")}
    gates = torch.from_numpy(inp["gates"]).to("cuda:0")
    fwd = binding.prefill(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"], dev["w_v"], gates,
                          s.top_k, s.window, want_sel=True)
    vis = np.asarray(inp["is_vision"]).astype(bool)
    sel = fwd["sel_idx"]  # [N_v, Hkv, k]: the forward's choice is reused
    dout = torch.from_numpy(make_output_grad((s.n_tokens, s.n_q_heads, s.head_dim), seed=1)).to("cuda:0")

    def call():
        return binding.prefill_backward(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"], dev["w_v"],
                                        gates, sel, dout, s.top_k, s.window)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    binding.timing_reset()
    binding.timing_enable(True)
    call()
    torch.cuda.synchronize()
    kern = {k: round(tot / cnt, 4) for k, (tot, cnt) in binding.timing_read().items()}
    binding.timing_enable(False)
    binding.timing_reset()
    # algorithmic flops: per attended (query, head, key) pair the backward
    # recomputes nothing in principle and does dV, dP, dQ, dK: 4 products of
    # 2 d flops each (the forward's two are not counted)
    text_pos = np.nonzero(~vis)[0]
    work = closed_form_work(s, text_pos)
    fwd_flops = sum(v for kind, v in work.values() if kind == "flops")
    flops = 2.0 * fwd_flops
    tf = flops / (ms * 1e-3) / 1e12
    # the kernels multiply fp16 operands on the matrix cores: priced against
    # the dense fp16 peak (the same figure as bf16)
    res = {"ms_per_step": round(ms, 3), "n_vision": s.n_vis, "n_text": s.n_text, "top_k": s.top_k,
           "window": s.window, "algorithmic_tflop": round(flops / 1e12, 4), "tflops": round(tf, 2),
           "mfma_peak_frac": round(tf / PEAK_BF16_TFLOPS, 4), "kernels": kern, "steps": steps}
    log(f"backward: {res}")
    return res


def run_scaling_bench(shape, steps, warmup):
    """Step time against context length at the workload's k and w: 16K to
    512K vision tokens (the largest the kernels take) plus its text tokens."""
    import torch
    from sparse_attention_long_nsa_amd.inputs import make_prefill_inputs
    rows = []
    for n_vis in (16384, 32768, 65536, 131072, 262144, 524288):
        s = shape.replace(n_vis=n_vis)
        inp = make_prefill_inputs(s, seed=0)
        dev = {k: torch.from_numpy(inp[k]).to("cuda:0").to(torch.bfloat16).contiguous()
               for k in ("q", "k", "v", "w_k", "w_v")}
        dev["gates"] = torch.from_numpy(inp["gates"]).to("cuda:0")
        ms, kern, out = run_gpu(inp, dev, s.top_k, s.window, steps, warmup, True)
        del dev, out, inp
        torch.cuda.empty_cache()

        def ms_of(*names):
            return round(sum(kern.get(n, (0.0, 0))[0] for n in names), 4)

        row = {"n_vision": n_vis, "n_tokens": s.n_tokens, "ms_per_step": round(ms, 4),
               "tokens_per_s": round(s.n_tokens / (ms * 1e-3), 1),
               "branch_ms": {"cmp": ms_of("cmp_pool", "pack_cmp", "cmp_attn"), "topk": ms_of("blk_score_topk"),
                             "sel": ms_of("pack_kv", "sel_attn"), "swa": ms_of("swa_attn"),
                             "text": ms_of("pack_text", "text_attn", "text_merge")}}
        rows.append(row)
        log(f"scaling {n_vis}: {ms:.3f} ms {row['branch_ms']}")
    return rows


def run_context_bench(presets, steps, warmup):
    """Step time and per-branch split of other prefill workloads (each its
    own k and w)."""
    import torch
    from sparse_attention_long_nsa_amd.inputs import PREFILL_PRESETS, make_prefill_inputs
    rows = []
    for name in presets:
        s = PREFILL_PRESETS[name]
        inp = make_prefill_inputs(s, seed=0)
        dev = {k: torch.from_numpy(inp[k]).to("cuda:0").to(torch.bfloat16).contiguous()
               for k in ("q", "k", "v", "w_k", "w_v")}
        dev["gates"] = torch.from_numpy(inp["gates"]).to("cuda:0")
        ms, kern, out = run_gpu(inp, dev, s.top_k, s.window, steps, warmup, True)
        text_pos = np.nonzero(inp["is_vision"] == 0)[0]
        fl = sum(v for kind, v in closed_form_work(s, text_pos).values() if kind == "flops")
        del dev, out, inp
        torch.cuda.empty_cache()

        def ms_of(*names):
            return round(sum(kern.get(n, (0.0, 0))[0] for n in names), 4)

        row = {"workload": name, "n_vision": s.n_vis, "n_text": s.n_text, "top_k": s.top_k, "window": s.window,
               "ms_per_step": round(ms, 4), "tokens_per_s": round(s.n_tokens / (ms * 1e-3), 1),
               "mfma_peak_frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
               "branch_ms": {"cmp": ms_of("cmp_pool", "pack_cmp", "cmp_attn"), "topk": ms_of("blk_score_topk"),
                             "sel": ms_of("pack_kv", "sel_attn"), "swa": ms_of("swa_attn"),
                             "text": ms_of("pack_text", "text_attn", "text_merge")},
               "kernels_ms": {k: round(v[0], 4) for k, v in sorted(kern.items(), key=lambda x: -x[1][0])}}
        rows.append(row)
        log(f"context {name}: {ms:.3f} ms {row['branch_ms']}")
    return rows


def cpu_baseline(inp, n_vis_rows, n_text_rows):
    """The fp64 oracle, as it stands, on a bounded row sample of the same
    workload; per-row times extrapolated to the whole sequence."""
    import oracle
    s = inp["shape"]
    isv = inp["is_vision"].astype(bool)
    V, T = np.nonzero(isv)[0], np.nonzero(~isv)[0]
    rng = np.random.default_rng(1)
    rv = np.sort(rng.choice(V, size=min(n_vis_rows, len(V)), replace=False))
    t0 = time.perf_counter()
    oracle.prefill(inp, rows=rv, want=())
    tv = time.perf_counter() - t0
    tt, rt = 0.0, np.zeros(0, dtype=np.int64)
    if len(T):
        rt = np.sort(rng.choice(T, size=min(n_text_rows, len(T)), replace=False))
        t0 = time.perf_counter()
        oracle.prefill(inp, rows=rt, want=())
        tt = time.perf_counter() - t0
    est = tv / len(rv) * len(V) + (tt / len(rt) * len(T) if len(rt) else 0.0)
    return {
        "value": s.n_tokens / est,
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"{len(rv)} random vision rows ({tv:.1f} s) + {len(rt)} random text rows "
                   f"({tt:.1f} s) of the same workload, per-row time extrapolated to all "
                   f"{s.n_tokens} rows"),
    }


def decode_bytes(s):
    """Algorithmic HBM bytes of one decode step: per (sequence, KV group) the
    compressed K/V cache, the k selected blocks' K/V and the window's K/V
    (bf16), plus queries, gates and outputs."""
    kv = 2 * 2 * s.head_dim  # K and V, bf16
    n_blk = s.cache_len // s.block
    per_group = n_blk * kv + min(s.top_k, n_blk) * s.block * kv + min(s.window, s.cache_len) * kv
    other = s.batch * s.n_q_heads * (s.head_dim * 2 + 3 * 4 + s.head_dim * 4)
    return float(s.batch * s.n_kv_heads * per_group + other)


def run_decode_bench(steps, warmup):
    """One nsa_decode step over 16 sequences with 131,072-token caches
    (compressed caches pooled on the GPU beforehand, outside the timed
    region); per-kernel event times as for prefill."""
    import torch
    from sparse_attention_long_nsa_amd import binding
    from sparse_attention_long_nsa_amd.inputs import DECODE_PRESETS, make_decode_inputs
    name = "decode_16x128k"
    s = DECODE_PRESETS[name]
    t0 = time.time()
    inp = make_decode_inputs(s, seed=0)
    log(f"inputs {name}: {time.time() - t0:.1f} s")

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0").to(torch.bfloat16)

    q, kcache, vcache = bf(inp["q"]), bf(inp["k_cache"]), bf(inp["v_cache"])
    del inp["k_cache"], inp["v_cache"]
    wk, wv = bf(inp["w_k"]), bf(inp["w_v"])
    gates = torch.from_numpy(inp["gates"]).to("cuda:0")
    kc = torch.stack([binding.cmp_pool(kcache[b], wk, s.block)["bf16"] for b in range(s.batch)])
    vc = torch.stack([binding.cmp_pool(vcache[b], wv, s.block)["bf16"] for b in range(s.batch)])

    def call(out, ws):
        return binding.decode(q, kcache, vcache, kc, vc, gates, s.top_k, s.window, block=s.block,
                              out=out, workspace=ws)

    r = call(None, None)
    out, ws = r["out"], r["workspace"]
    for _ in range(warmup):
        call(out, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call(out, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    binding.timing_reset()
    binding.timing_enable(True)
    for _ in range(steps):
        call(out, ws)
    torch.cuda.synchronize()
    kern = binding.timing_read()
    binding.timing_enable(False)
    binding.timing_reset()

    # cache maintenance per generated token: nsa_cache_append rewriting the
    # cache's own last rows (so the caches stay as they are), without and
    # with the pooling of a block the token completes
    def append_us(L, n=50):
        kn, vn = kcache[:, L - 1].contiguous(), vcache[:, L - 1].contiguous()
        binding.cache_append(kn, vn, kcache, vcache, wk, wv, kc, vc, L)
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(n):
            binding.cache_append(kn, vn, kcache, vcache, wk, wv, kc, vc, L)
        a1.record()
        torch.cuda.synchronize()
        binding.timing_reset()
        binding.timing_enable(True)
        for _ in range(n):
            binding.cache_append(kn, vn, kcache, vcache, wk, wv, kc, vc, L)
        torch.cuda.synchronize()
        kt = {k: round(v[0] / v[1] * 1e3, 2) for k, v in binding.timing_read().items()}
        binding.timing_enable(False)
        binding.timing_reset()
        return {"us_per_call": round(a0.elapsed_time(a1) / n * 1e3, 2), "kernel_us": kt}

    # us_per_call includes the host's per-call cost (back-to-back calls)
    append = {"row": append_us(s.cache_len - 1), "row_and_block_pool": append_us(s.cache_len)}
    nbytes = decode_bytes(s)
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": name, "batch": s.batch, "cache_len": s.cache_len, "top_k": s.top_k,
           "window": s.window, "us_per_step": round(ms * 1e3, 2),
           "sequences_per_s": round(s.batch / (ms * 1e-3), 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "algorithmic_bytes": nbytes},
           "kernels": {k: {"avg_us": round(v[0] / v[1] * 1e3, 2), "launches": v[1]} for k, v in kern.items()},
           "cache_append": append}
    log(f"decode {name}: {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s algorithmic")
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen_128k_k32_w256")
    ap.add_argument("--cpu-vision-rows", type=int, default=15000)
    ap.add_argument("--cpu-text-rows", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-spans", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-gate", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--backward-workload", choices=("both", "short", "qwen_36k"), default="both",
                    help="backward legs: 4,096 + 512 tokens, the 36,864 + 512 training length, or both")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the 36K / 64K per-branch legs (for profiler runs of the headline workload)")
    ap.add_argument("--scaling", action="store_true",
                    help="also time 16K..512K vision tokens (about a minute more, mostly input generation)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this layer library runs on a single MI355X and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_long_nsa_amd import binding
    from sparse_attention_long_nsa_amd.inputs import PREFILL_PRESETS, make_prefill_inputs
    binding.lib()  # fail loudly if the HIP library is missing
    shape = PREFILL_PRESETS[args.workload]
    t0 = time.time()
    inp = make_prefill_inputs(shape, seed=0)
    log(f"inputs {args.workload}: {time.time() - t0:.1f} s")
    dev = {k: torch.from_numpy(inp[k]).to("cuda:0").to(torch.bfloat16).contiguous()
           for k in ("q", "k", "v", "w_k", "w_v")}
    dev["gates"] = torch.from_numpy(inp["gates"]).to("cuda:0")

    ms, kern, _ = run_gpu(inp, dev, shape.top_k, shape.window, args.steps, args.warmup, True)
    tokens = shape.n_tokens
    value = tokens / (ms * 1e-3)
    text_pos = np.nonzero(inp["is_vision"] == 0)[0]
    work = closed_form_work(shape, text_pos)
    layer_flops = sum(v for kind, v in work.values() if kind == "flops")
    log(f"{ms:.3f} ms/step, {value / 1e6:.2f} M tokens/s")

    per_kernel = {}
    for name, (avg_ms, cnt) in sorted(kern.items(), key=lambda x: -x[1][0]):
        kind, amount = work.get(name, (None, None))
        ent = {"avg_ms": round(avg_ms, 4), "launches": cnt}
        if kind == "flops":
            ent["tflops"] = round(amount / (avg_ms * 1e-3) / 1e12, 1)
            ent["frac_of_peak"] = round(ent["tflops"] / PEAK_BF16_TFLOPS, 4)
        elif kind == "bytes":
            ent["gbs"] = round(amount / (avg_ms * 1e-3) / 1e9, 1)
            ent["frac_of_peak"] = round(ent["gbs"] / PEAK_HBM_GBS, 4)
        per_kernel[name] = ent
        log(f"  {name:16s} {avg_ms:8.3f} ms  {ent}")
    dom = max((n for n in kern if n in work), key=lambda n: kern[n][0])
    kind, amount = work[dom]
    avg = kern[dom][0] * 1e-3
    if kind == "flops":
        achieved, peak, unit, bound = amount / avg / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = amount / avg / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    roofline = {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": pmc_traffic(dom, args.workload)}

    def ms_of(*names):
        return round(sum(kern.get(n, (0.0, 0))[0] for n in names), 4)

    branch_ms = {"cmp": ms_of("cmp_pool", "pack_cmp", "cmp_attn"),
                 "sel": ms_of("blk_score_topk", "pack_kv", "sel_attn"),
                 "swa": ms_of("swa_attn"), "text": ms_of("pack_text", "text_attn", "text_merge")}

    sweep = []
    if not args.no_sweep:
        for k, w in SWEEP:
            sms, _, _ = run_gpu(inp, dev, k, w, max(3, args.steps // 2), 1, False)
            sw = closed_form_work(shape.replace(top_k=k, window=w), text_pos)
            fl = sum(v for kd, v in sw.values() if kd == "flops")
            sweep.append({"top_k": k, "window": w, "ms_per_step": round(sms, 3),
                          "tokens_per_s": round(tokens / (sms * 1e-3), 1),
                          "mfma_peak_frac": round(fl / (sms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
            log(f"  sweep k={k} w={w}: {sms:.3f} ms")

    decode = None
    if not args.no_decode:
        decode = run_decode_bench(max(10, args.steps), args.warmup)

    dense = None
    if not args.no_dense:
        dense = run_dense_bench(dev, shape, 3, 1, ms)

    gate = None
    if not args.no_gate:
        gate = run_gate_bench(shape, max(3, args.steps // 2), 1)

    backward = None
    if not args.no_backward:
        short = shape.replace(n_vis=BWD_SHAPE["n_vis"], n_text_before=0, n_text_after=BWD_SHAPE["n_text_after"])
        # the pages' training context (model card, "Training Details": 36K tokens)
        if args.backward_workload == "qwen_36k":
            backward = run_backward_bench(PREFILL_PRESETS["qwen_36k"], 3, 1)
        else:
            backward = run_backward_bench(short, 3, 1)
            if args.backward_workload == "both":
                backward["training_length"] = run_backward_bench(PREFILL_PRESETS["qwen_36k"], 3, 1)

    spans = None
    if not args.no_spans:
        spans = run_spans_bench(inp, shape, max(3, args.steps // 2), 1, ms)

    # the pages' training length and the per-branch split workload (36,864
    # and 65,536 vision + 512 text tokens, k 16, w 512), always; 16K..512K
    # at the headline's k and w on request
    scaling = [] if args.no_context else run_context_bench(("qwen_36k", "qwen_64k"), max(3, args.steps // 2), 1)
    if args.scaling:
        scaling += run_scaling_bench(shape, max(3, args.steps // 2), 1)

    # the published peak checked on this GPU with an MFMA-loop probe
    from sparse_attention_long_nsa_amd.profiling import mfma_peak
    probe = mfma_peak()
    # the fabric rate of the selection kernel's block copies (pseudo-random
    # whole 32 KB blocks) at buffer sizes from L2-resident to far beyond it
    from sparse_attention_long_nsa_amd.profiling import block_stream
    stream_probe = block_stream()
    log(f"block-stream probe: {stream_probe}")
    probe["frac_of_published"] = round(probe["tflops"] / PEAK_BF16_TFLOPS, 4)
    log(f"mfma loop probe: {probe}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_vision_rows, args.cpu_text_rows)
        log(f"cpu baseline: {cpu}")

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "n_vision": shape.n_vis, "n_text": shape.n_text,
                   "n_q_heads": shape.n_q_heads, "n_kv_heads": shape.n_kv_heads,
                   "head_dim": shape.head_dim, "block": shape.block, "top_k": shape.top_k,
                   "window": shape.window, "seq_len": shape.n_tokens, "global_batch": 1,
                   "parallelism": "single GPU"},
        "mfma_peak_frac": round(layer_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "algorithmic_tflop": round(layer_flops / 1e12, 3),
        "mfma_loop_probe": probe,
        "block_stream_probe": stream_probe,
        "roofline": roofline,
        "branch_ms": branch_ms,
        "kernels": per_kernel,
        "sweep": sweep,
        "decode": decode,
        "several_vision_runs": spans,
        "dense_mode": dense,
        "gate_prologue": gate,
        "backward": backward,
        "context_scaling": scaling,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
