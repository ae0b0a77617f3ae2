"""Seeded synthetic inputs for the VideoNSA attention layer.

This module only draws random numbers and lays them out; it contains none of
the layer's arithmetic. Both the fp64 oracle (through the tests) and the HIP
path consume exactly the arrays produced here.

Workload shapes follow the VideoNSA pages: a Qwen2.5-VL-7B decoder layer with
28 query heads and 4 KV heads (paper summary page, "Method"), 64 tokens per
video frame, which is also the compression/selection block (same section),
36K-token training context and 128K-token evaluation context (model card,
"Training Details"; paper summary, §4 Finding 2).

Generator recipe (frame-correlated video tokens):
  * every tensor X in (q, k, v), every head and every 64-token frame gets one
    shared vector s ~ N(0, I_d); each vision token of that frame is
    s + 0.5 * N(0, I_d);
  * text rows are i.i.d. N(0, I_d);
  * gate logits are i.i.d. N(0, 1) per (token, head, branch);
  * the compression maps W_k, W_v are i.i.d. N(0, 1/d);
  * draw order: q/k/v frame vectors, q/k/v token noise, q/k/v text rows,
    gate logits, W_k, W_v; numpy PCG64 seeded with the given seed;
  * for bf16 workloads every array except the gate logits is rounded to the
    nearest bf16 (ties to even); values are returned as float32 arrays that
    hold bf16-exact numbers, plus helpers for the raw 16-bit patterns.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class PrefillShape:
    """One prefill workload: a single sequence laid out as
    [text_before][vision][text_after]."""

    n_vis: int
    n_text_before: int
    n_text_after: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block: int
    top_k: int
    window: int
    dtype: str  # "bf16" or "fp32"

    @property
    def n_tokens(self) -> int:
        return self.n_text_before + self.n_vis + self.n_text_after

    @property
    def n_text(self) -> int:
        return self.n_text_before + self.n_text_after

    def replace(self, **kw) -> "PrefillShape":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class DecodeShape:
    """Decode step: `batch` sequences, each one query (the last cache token)
    against a `cache_len`-token vision K/V cache."""

    batch: int
    cache_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block: int
    top_k: int
    window: int
    dtype: str = "bf16"


# Named workloads. The 128K points trade selected blocks against window width
# at a fixed fine-grained budget (paper summary, §4 Finding 3, Fig. 3); the
# (32, 256) point is the paper's own default (paper summary, "Method").
PREFILL_PRESETS = {
    "tiny_1k_fp32": PrefillShape(1024, 0, 0, 4, 1, 64, 64, 4, 128, "fp32"),
    "qwen_36k": PrefillShape(36864, 0, 512, 28, 4, 128, 64, 16, 512, "bf16"),
    "qwen_64k": PrefillShape(65536, 0, 512, 28, 4, 128, 64, 16, 512, "bf16"),
    "qwen_128k_k32_w256": PrefillShape(131072, 0, 512, 28, 4, 128, 64, 32, 256, "bf16"),
    "qwen_128k_k16_w512": PrefillShape(131072, 0, 512, 28, 4, 128, 64, 16, 512, "bf16"),
    "qwen_128k_k8_w1024": PrefillShape(131072, 0, 512, 28, 4, 128, 64, 8, 1024, "bf16"),
    # longer contexts, up to the largest the kernels take (8,192 blocks of 64)
    "qwen_256k_k32_w256": PrefillShape(262144, 0, 512, 28, 4, 128, 64, 32, 256, "bf16"),
    "qwen_512k_k32_w256": PrefillShape(524288, 0, 512, 28, 4, 128, 64, 32, 256, "bf16"),
}

DECODE_PRESETS = {
    "decode_16x128k": DecodeShape(16, 131072, 28, 4, 128, 64, 16, 512, "bf16"),
    # the longest cache the kernels take (8,192 blocks of 64)
    "decode_2x512k": DecodeShape(2, 524288, 28, 4, 128, 64, 16, 512, "bf16"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) of float32 arrays that hold bf16-exact values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("array holds values that are not bf16-exact")
    return (u >> 16).astype(np.uint16)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _frame_tokens(frames: np.ndarray, noise: np.ndarray, block: int) -> np.ndarray:
    """Vision tokens: each frame vector repeated over its tokens, plus 0.5*noise."""
    n = noise.shape[0]
    out = np.repeat(frames, block, axis=0)[:n]
    out += np.float32(0.5) * noise
    return out


def make_prefill_inputs(shape: PrefillShape, seed: int = 0) -> dict:
    """Draw one prefill workload. Returns float32 numpy arrays:
    q [N,Hq,d], k/v [N,Hkv,d], is_vision uint8 [N], gates [N,Hq,3],
    w_k/w_v [d,d] (y = W x), plus the shape."""
    s = shape
    rng = np.random.Generator(np.random.PCG64(seed))
    d, B = s.head_dim, s.block
    n_frames = -(-s.n_vis // B)
    heads = {"q": s.n_q_heads, "k": s.n_kv_heads, "v": s.n_kv_heads}
    frames = {x: _normal(rng, (n_frames, h, d)) for x, h in heads.items()}
    vis = {}
    for x, h in heads.items():
        vis[x] = _frame_tokens(frames[x], _normal(rng, (s.n_vis, h, d)), B)
        del frames[x]
    text = {x: _normal(rng, (s.n_text, h, d)) for x, h in heads.items()}
    gates = _normal(rng, (s.n_tokens, s.n_q_heads, 3))
    w_scale = np.float32(1.0 / math.sqrt(d))
    w_k = _normal(rng, (d, d)) * w_scale
    w_v = _normal(rng, (d, d)) * w_scale

    out = {}
    a, b = s.n_text_before, s.n_text_before + s.n_vis
    for x, h in heads.items():
        arr = np.empty((s.n_tokens, h, d), dtype=np.float32)
        arr[:a] = text[x][: s.n_text_before]
        arr[a:b] = vis[x]
        arr[b:] = text[x][s.n_text_before:]
        del vis[x]
        out[x] = arr
    is_vision = np.zeros(s.n_tokens, dtype=np.uint8)
    is_vision[a:b] = 1
    out.update(is_vision=is_vision, gates=gates, w_k=w_k, w_v=w_v)
    if s.dtype == "bf16":
        for x in ("q", "k", "v", "w_k", "w_v"):
            out[x] = round_to_bf16(out[x])
    elif s.dtype != "fp32":
        raise ValueError(f"unknown dtype {s.dtype}")
    out["shape"] = s
    return out


def mask_from_runs(runs) -> np.ndarray:
    """Token-kind mask (uint8, 1 = vision) of a sequence written as runs
    [("t", n), ("v", n), ...] in position order."""
    parts = []
    for kind, n in runs:
        if kind not in ("t", "v") or n < 0:
            raise ValueError(f"bad run {(kind, n)}")
        parts.append(np.full(n, 1 if kind == "v" else 0, dtype=np.uint8))
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.uint8)


def relayout(inp: dict, is_vision: np.ndarray) -> dict:
    """The same tokens at new positions: the vision rows of `inp` keep their
    order and move to the positions where `is_vision` is 1, the text rows keep
    theirs and fill the rest; gates travel with their rows."""
    old = np.asarray(inp["is_vision"]).astype(bool)
    new = np.asarray(is_vision).astype(bool)
    if new.shape != old.shape or new.sum() != old.sum():
        raise ValueError("the new mask must hold as many vision tokens as the old one")
    perm = np.empty(old.shape[0], dtype=np.int64)  # new position -> old row
    perm[np.nonzero(new)[0]] = np.nonzero(old)[0]
    perm[np.nonzero(~new)[0]] = np.nonzero(~old)[0]
    out = dict(inp)
    for x in ("q", "k", "v", "gates"):
        out[x] = np.ascontiguousarray(inp[x][perm])
    out["is_vision"] = new.astype(np.uint8)
    return out


# Layouts with several vision runs (several clips or images in one prompt,
# text between them), as run lists over the tokens of a prefill preset.
SPAN_LAYOUTS = {
    # 128K vision tokens as 8 clips of 16,384, each after a 64-token text run
    "8clips": [("t", 64), ("v", 16384)] * 8,
}


def make_gate_inputs(n: int, d_model: int, d_hidden: int, n_q_heads: int, seed: int = 0,
                     bias: bool = True) -> dict:
    """Draw one gate-prologue workload: hidden states x [n, d_model] ~ N(0, 1)
    (a decoder layer's normalised input has unit RMS per token), W1
    [d_hidden, d_model] ~ N(0, 1/d_model), W2 [3 Hq, d_hidden] ~ N(0,
    1/d_hidden), biases b1 [d_hidden], b2 [3 Hq] ~ N(0, 0.1^2) (or None).
    Draw order x, W1, W2, b1, b2; x, W1, W2 are rounded to bf16, the biases
    stay float32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = np.empty((n, d_model), dtype=np.float32)
    step = 8192
    for r0 in range(0, n, step):  # bounded temporaries at long contexts
        x[r0:r0 + step] = round_to_bf16(_normal(rng, (min(step, n - r0), d_model)))
    w1 = round_to_bf16(_normal(rng, (d_hidden, d_model)) * np.float32(1.0 / math.sqrt(d_model)))
    w2 = round_to_bf16(_normal(rng, (3 * n_q_heads, d_hidden)) * np.float32(1.0 / math.sqrt(d_hidden)))
    b1 = _normal(rng, (d_hidden,)) * np.float32(0.1)
    b2 = _normal(rng, (3 * n_q_heads,)) * np.float32(0.1)
    return dict(x=x, w1=w1, w2=w2, b1=b1 if bias else None, b2=b2 if bias else None, n_q_heads=n_q_heads)


def make_output_grad(shape, seed: int = 0) -> np.ndarray:
    """A seeded upstream gradient dL/d(out) for the backward pass: i.i.d.
    N(0, 1) float32 of the given shape."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _normal(rng, tuple(shape))


def make_decode_inputs(shape: DecodeShape, seed: int = 0) -> dict:
    """Draw one decode workload: per sequence a frame-correlated vision K/V
    cache [Bt,L,Hkv,d]; the query is the last cache token, so it is drawn from
    the last frame's q vector plus token noise; gates [Bt,Hq,3]; W_k, W_v for
    whoever pools the compressed cache."""
    s = shape
    rng = np.random.Generator(np.random.PCG64(seed))
    d, B, L = s.head_dim, s.block, s.cache_len
    n_frames = -(-L // B)
    kf = _normal(rng, (s.batch, n_frames, s.n_kv_heads, d))
    vf = _normal(rng, (s.batch, n_frames, s.n_kv_heads, d))
    k = np.empty((s.batch, L, s.n_kv_heads, d), dtype=np.float32)
    v = np.empty_like(k)
    for bi in range(s.batch):
        k[bi] = _frame_tokens(kf[bi], _normal(rng, (L, s.n_kv_heads, d)), B)
    for bi in range(s.batch):
        v[bi] = _frame_tokens(vf[bi], _normal(rng, (L, s.n_kv_heads, d)), B)
    del kf, vf
    qf = _normal(rng, (s.batch, s.n_q_heads, d))
    q = qf + np.float32(0.5) * _normal(rng, (s.batch, s.n_q_heads, d))
    gates = _normal(rng, (s.batch, s.n_q_heads, 3))
    w_scale = np.float32(1.0 / math.sqrt(d))
    w_k = _normal(rng, (d, d)) * w_scale
    w_v = _normal(rng, (d, d)) * w_scale
    out = dict(q=q, k_cache=k, v_cache=v, gates=gates, w_k=w_k, w_v=w_v)
    if s.dtype == "bf16":
        for x in ("q", "k_cache", "v_cache", "w_k", "w_v"):
            out[x] = round_to_bf16(out[x])
    out["shape"] = s
    return out
