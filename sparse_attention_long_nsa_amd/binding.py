"""Thin ctypes binding over libnsa.so (the C ABI declared in include/nsa.h).

Only argument marshalling lives here: torch tensors supply device memory and
the current HIP stream; every step of the layer runs in the library's HIP
kernels. Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnsa.so")

NSA_OK, NSA_ERR_INVALID_ARG, NSA_ERR_UNSUPPORTED, NSA_ERR_WORKSPACE, NSA_ERR_HIP, NSA_ERR_KERNEL = range(6)
NSA_DTYPE_BF16, NSA_DTYPE_FP32 = 0, 1

EXPORTED = (
    "nsa_prefill_workspace_size", "nsa_prefill", "nsa_decode_workspace_size", "nsa_decode",
    "nsa_cmp_pool", "nsa_timing_enable", "nsa_timing_reset", "nsa_timing_read",
    "nsa_status_string", "nsa_version", "nsa_probe_mfma_bf16",
    "nsa_prefill_dense_workspace_size", "nsa_prefill_dense", "nsa_cache_append",
    "nsa_prefill_varlen_workspace_size", "nsa_prefill_varlen",
    "nsa_gate_workspace_size", "nsa_gate_logits",
    "nsa_prefill_backward_workspace_size", "nsa_prefill_backward", "nsa_decode_noalloc",
    "nsa_workspace_status", "nsa_debug_set_spin_limit", "nsa_probe_block_stream",
)

# size of the library's fixed decode scratch (nsa.h NSA_DECODE_NOALLOC_SCRATCH_BYTES)
DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20
NSA_ACTIVATIONS = {"silu": 0, "gelu_tanh": 1, "relu": 2}


class NsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class PrefillDesc(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


class DecodeDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("cache_len", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("cache_capacity", ctypes.c_int32),
    ]


class GateDesc(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64),
        ("d_model", ctypes.c_int32),
        ("d_hidden", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("activation", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if libnsa.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m sparse_attention_long_nsa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.c_size_t
        L.nsa_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillDesc), P, ctypes.POINTER(S)]
        L.nsa_prefill_workspace_size.restype = ctypes.c_int
        L.nsa_prefill.argtypes = [ctypes.POINTER(PrefillDesc)] + [P] * 13 + [S, P]
        L.nsa_prefill.restype = ctypes.c_int
        L.nsa_prefill_dense_workspace_size.argtypes = [ctypes.POINTER(PrefillDesc), ctypes.POINTER(S)]
        L.nsa_prefill_dense_workspace_size.restype = ctypes.c_int
        L.nsa_prefill_dense.argtypes = [ctypes.POINTER(PrefillDesc)] + [P] * 6 + [S, P]
        L.nsa_prefill_dense.restype = ctypes.c_int
        L.nsa_prefill_varlen_workspace_size.argtypes = [ctypes.POINTER(PrefillDesc), ctypes.c_int32, P, P,
                                                        ctypes.POINTER(S)]
        L.nsa_prefill_varlen_workspace_size.restype = ctypes.c_int
        L.nsa_prefill_varlen.argtypes = [ctypes.POINTER(PrefillDesc), ctypes.c_int32] + [P] * 14 + [S, P]
        L.nsa_prefill_varlen.restype = ctypes.c_int
        L.nsa_prefill_backward_workspace_size.argtypes = [ctypes.POINTER(PrefillDesc), P, ctypes.POINTER(S)]
        L.nsa_prefill_backward_workspace_size.restype = ctypes.c_int
        L.nsa_prefill_backward.argtypes = [ctypes.POINTER(PrefillDesc)] + [P] * 16 + [S, P]
        L.nsa_prefill_backward.restype = ctypes.c_int
        L.nsa_gate_workspace_size.argtypes = [ctypes.POINTER(GateDesc), ctypes.POINTER(S)]
        L.nsa_gate_workspace_size.restype = ctypes.c_int
        L.nsa_gate_logits.argtypes = [ctypes.POINTER(GateDesc)] + [P] * 7 + [S, P]
        L.nsa_gate_logits.restype = ctypes.c_int
        L.nsa_cache_append.argtypes = [ctypes.POINTER(DecodeDesc)] + [P] * 9
        L.nsa_cache_append.restype = ctypes.c_int
        L.nsa_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeDesc), ctypes.POINTER(S)]
        L.nsa_decode_workspace_size.restype = ctypes.c_int
        L.nsa_decode.argtypes = [ctypes.POINTER(DecodeDesc)] + [P] * 10 + [S, P]
        L.nsa_decode_noalloc.argtypes = [ctypes.POINTER(DecodeDesc)] + [P] * 10
        L.nsa_decode_noalloc.restype = ctypes.c_int
        L.nsa_workspace_status.argtypes = [P, P, ctypes.POINTER(ctypes.c_int32)]
        L.nsa_workspace_status.restype = ctypes.c_int
        L.nsa_debug_set_spin_limit.argtypes = [ctypes.c_int32]
        L.nsa_debug_set_spin_limit.restype = ctypes.c_int
        L.nsa_decode.restype = ctypes.c_int
        L.nsa_cmp_pool.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, P, P, P, P, P]
        L.nsa_cmp_pool.restype = ctypes.c_int
        L.nsa_timing_enable.argtypes = [ctypes.c_int]
        L.nsa_timing_enable.restype = ctypes.c_int
        L.nsa_timing_reset.restype = ctypes.c_int
        L.nsa_timing_read.argtypes = [ctypes.c_int, P, P, P]
        L.nsa_timing_read.restype = ctypes.c_int
        L.nsa_status_string.argtypes = [ctypes.c_int]
        L.nsa_status_string.restype = ctypes.c_char_p
        L.nsa_version.restype = ctypes.c_char_p
        L.nsa_probe_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P]
        L.nsa_probe_mfma_bf16.restype = ctypes.c_int
        L.nsa_probe_block_stream.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P]
        L.nsa_probe_block_stream.restype = ctypes.c_int
        _lib = L
    return _lib


def timing_enable(on: bool = True) -> None:
    lib().nsa_timing_enable(1 if on else 0)


def timing_reset() -> None:
    lib().nsa_timing_reset()


def timing_read() -> dict:
    """{kernel: (total_ms, launches)} over the launches timed since the last
    reset (waits for their events)."""
    n = lib().nsa_timing_read(0, None, None, None)
    names = (ctypes.c_char_p * max(n, 1))()
    ms = (ctypes.c_double * max(n, 1))()
    cnt = (ctypes.c_int * max(n, 1))()
    n = lib().nsa_timing_read(n, names, ms, cnt)
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(n)}


def workspace_status(workspace, stream=None) -> int:
    """Runs nsa_workspace_status on a prefill workspace: waits for the stream
    and returns the status word (0 = every wait completed and every fp16
    value was in range; bit 0: a bounded wait gave up; bit 1: an fp16
    overflow)."""
    flags = ctypes.c_int32(0)
    st = lib().nsa_workspace_status(_ptr(workspace), _stream(stream), ctypes.byref(flags))
    if st not in (NSA_OK, NSA_ERR_KERNEL):
        raise NsaError(st, "nsa_workspace_status")
    return int(flags.value)


def set_spin_limit(rounds: int) -> None:
    """Test aid (nsa_debug_set_spin_limit): bounded-wait rounds of the prefill
    kernels for later calls; <= 0 restores the default."""
    lib().nsa_debug_set_spin_limit(int(rounds))


def status_string(status: int) -> str:
    return lib().nsa_status_string(status).decode()


def version() -> str:
    return lib().nsa_version().decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data_as(ctypes.c_void_p)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_dev(name, t, dtype, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _mask_host(is_vision) -> np.ndarray:
    if isinstance(is_vision, torch.Tensor):
        is_vision = is_vision.detach().cpu().numpy()
    return np.ascontiguousarray(is_vision, dtype=np.uint8)


def prefill_desc(q, k, top_k, window, block=64, scale=0.0) -> PrefillDesc:
    n, hq, d = q.shape
    dt = {torch.bfloat16: NSA_DTYPE_BF16, torch.float32: NSA_DTYPE_FP32}[q.dtype]
    return PrefillDesc(n, hq, k.shape[1], d, block, top_k, window, float(scale), dt)


def prefill_workspace_size(desc: PrefillDesc, is_vision) -> int:
    mask = _mask_host(is_vision)
    n = ctypes.c_size_t(0)
    st = lib().nsa_prefill_workspace_size(ctypes.byref(desc), _ptr(mask), ctypes.byref(n))
    if st != NSA_OK:
        raise NsaError(st, "nsa_prefill_workspace_size")
    return n.value


def prefill(q, k, v, is_vision, w_cmp_k, w_cmp_v, gate_logits, top_k, window, block=64,
            scale=0.0, out=None, want_kcmp=False, want_sel=False, want_lse=False,
            workspace=None, stream=None) -> dict:
    """Runs nsa_prefill. q [N,Hq,d], k/v [N,Hkv,d], w_cmp_* [d,d] (bf16 or fp32,
    all the same dtype), gate_logits [N,Hq,3] fp32 on the device; is_vision [N]
    on the host (numpy or CPU tensor). Returns a dict with "out" (fp32) and
    the requested optional outputs."""
    desc = prefill_desc(q, k, top_k, window, block, scale)
    n, hq, d = q.shape
    hkv = k.shape[1]
    for name, t, shape in (("q", q, (n, hq, d)), ("k", k, (n, hkv, d)), ("v", v, (n, hkv, d)),
                           ("w_cmp_k", w_cmp_k, (d, d)), ("w_cmp_v", w_cmp_v, (d, d))):
        _check_dev(name, t, q.dtype, shape)
    _check_dev("gate_logits", gate_logits, torch.float32, (n, hq, 3))
    mask = _mask_host(is_vision)
    if mask.shape != (n,):
        raise ValueError("is_vision must have one entry per token")
    n_vis = int(mask.astype(bool).sum())
    dev = q.device
    res = {}
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.float32, device=dev)
    _check_dev("out", out, torch.float32, (n, hq, d))
    res["out"] = out
    kc = vc = sel = lse = None
    if want_kcmp:
        kc = res["k_cmp"] = torch.empty((n_vis // block, hkv, d), dtype=torch.float32, device=dev)
        vc = res["v_cmp"] = torch.empty((n_vis // block, hkv, d), dtype=torch.float32, device=dev)
    if want_sel:
        sel = res["sel_idx"] = torch.empty((n_vis, hkv, top_k), dtype=torch.int32, device=dev)
    if want_lse:
        lse = res["lse"] = torch.empty((n_vis, hq), dtype=torch.float32, device=dev)
    ws_bytes = prefill_workspace_size(desc, mask)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    st = lib().nsa_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(mask),
                           _ptr(w_cmp_k), _ptr(w_cmp_v), _ptr(gate_logits), _ptr(out), _ptr(kc),
                           _ptr(vc), _ptr(sel), _ptr(lse), _ptr(workspace), workspace.numel(),
                           _stream(stream))
    if st != NSA_OK:
        raise NsaError(st, "nsa_prefill")
    res["workspace"] = workspace
    return res


def prefill_varlen(q, k, v, cu_seqlens, is_vision, w_cmp_k, w_cmp_v, gate_logits, top_k, window,
                   block=64, scale=0.0, out=None, want_kcmp=False, want_sel=False, want_lse=False,
                   workspace=None, stream=None) -> dict:
    """Runs nsa_prefill_varlen: sequences i = rows cu_seqlens[i] .. cu_seqlens[i+1]-1
    (cu_seqlens on the host); tensors as for prefill over all rows. Optional
    outputs are concatenated over the sequences."""
    desc = prefill_desc(q, k, top_k, window, block, scale)
    n, hq, d = q.shape
    hkv = k.shape[1]
    for name, t, shape in (("q", q, (n, hq, d)), ("k", k, (n, hkv, d)), ("v", v, (n, hkv, d)),
                           ("w_cmp_k", w_cmp_k, (d, d)), ("w_cmp_v", w_cmp_v, (d, d))):
        _check_dev(name, t, q.dtype, shape)
    _check_dev("gate_logits", gate_logits, torch.float32, (n, hq, 3))
    mask = _mask_host(is_vision)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    if mask.shape != (n,) or cu.ndim != 1 or len(cu) < 2:
        raise ValueError("is_vision needs one entry per token and cu_seqlens at least two")
    ns = len(cu) - 1
    isv = mask.astype(bool)
    n_vis = int(isv.sum())
    n_blk = sum(int(isv[cu[i]:cu[i + 1]].sum()) // block for i in range(ns))
    dev = q.device
    res = {}
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.float32, device=dev)
    _check_dev("out", out, torch.float32, (n, hq, d))
    res["out"] = out
    kc = vc = sel = lse = None
    if want_kcmp:
        kc = res["k_cmp"] = torch.empty((n_blk, hkv, d), dtype=torch.float32, device=dev)
        vc = res["v_cmp"] = torch.empty((n_blk, hkv, d), dtype=torch.float32, device=dev)
    if want_sel:
        sel = res["sel_idx"] = torch.empty((n_vis, hkv, top_k), dtype=torch.int32, device=dev)
    if want_lse:
        lse = res["lse"] = torch.empty((n_vis, hq), dtype=torch.float32, device=dev)
    nb = ctypes.c_size_t(0)
    st = lib().nsa_prefill_varlen_workspace_size(ctypes.byref(desc), ns, _ptr(cu), _ptr(mask), ctypes.byref(nb))
    if st != NSA_OK:
        raise NsaError(st, "nsa_prefill_varlen_workspace_size")
    if workspace is None or workspace.numel() < nb.value:
        workspace = torch.empty(max(nb.value, 256), dtype=torch.uint8, device=dev)
    st = lib().nsa_prefill_varlen(ctypes.byref(desc), ns, _ptr(cu), _ptr(q), _ptr(k), _ptr(v), _ptr(mask),
                                  _ptr(w_cmp_k), _ptr(w_cmp_v), _ptr(gate_logits), _ptr(out), _ptr(kc),
                                  _ptr(vc), _ptr(sel), _ptr(lse), _ptr(workspace), workspace.numel(),
                                  _stream(stream))
    if st != NSA_OK:
        raise NsaError(st, "nsa_prefill_varlen")
    res["workspace"] = workspace
    return res


def prefill_dense_workspace_size(desc: PrefillDesc) -> int:
    n = ctypes.c_size_t(0)
    st = lib().nsa_prefill_dense_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != NSA_OK:
        raise NsaError(st, "nsa_prefill_dense_workspace_size")
    return n.value


def prefill_dense(q, k, v, scale=0.0, out=None, want_lse=False, workspace=None, stream=None) -> dict:
    """Runs nsa_prefill_dense (dense causal GQA over every token). q [N,Hq,d],
    k/v [N,Hkv,d] on the device (bf16 or fp32, one dtype). Returns a dict with
    "out" (fp32) and optionally "lse"."""
    desc = prefill_desc(q, k, 1, 1, 64, scale)
    n, hq, d = q.shape
    hkv = k.shape[1]
    for name, t, shape in (("q", q, (n, hq, d)), ("k", k, (n, hkv, d)), ("v", v, (n, hkv, d))):
        _check_dev(name, t, q.dtype, shape)
    dev = q.device
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.float32, device=dev)
    _check_dev("out", out, torch.float32, (n, hq, d))
    res = {"out": out}
    lse = None
    if want_lse:
        lse = res["lse"] = torch.empty((n, hq), dtype=torch.float32, device=dev)
    ws_bytes = prefill_dense_workspace_size(desc)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    st = lib().nsa_prefill_dense(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                 _ptr(workspace), workspace.numel(), _stream(stream))
    if st != NSA_OK:
        raise NsaError(st, "nsa_prefill_dense")
    res["workspace"] = workspace
    return res


def prefill_backward(q, k, v, is_vision, w_cmp_k, w_cmp_v, gate_logits, sel_idx, dout, top_k, window,
                     block=64, scale=0.0, stream=None, workspace=None) -> dict:
    """Runs nsa_prefill_backward: gradients (fp32, on the device) of the layer
    for the output gradient dout [N,Hq,d], reusing the forward's selection
    sel_idx [N_v,Hkv,top_k]. Returns dq, dk, dv, dw_cmp_k, dw_cmp_v, dgate.
    workspace: an optional uint8 device tensor of at least the required size
    (its status word can then be read with workspace_status)."""
    n, hq, d = q.shape
    hkv = k.shape[1]
    for name, t, shape in (("q", q, (n, hq, d)), ("k", k, (n, hkv, d)), ("v", v, (n, hkv, d)),
                           ("w_cmp_k", w_cmp_k, (d, d)), ("w_cmp_v", w_cmp_v, (d, d))):
        _check_dev(name, t, torch.bfloat16, shape)
    _check_dev("gate_logits", gate_logits, torch.float32, (n, hq, 3))
    _check_dev("dout", dout, torch.float32, (n, hq, d))
    mask = _mask_host(is_vision)
    nv = int(mask.sum())
    if nv > 0:
        _check_dev("sel_idx", sel_idx, torch.int32, (nv, hkv, top_k))
    desc = prefill_desc(q, k, top_k, window, block, scale)
    nb = ctypes.c_size_t(0)
    st = lib().nsa_prefill_backward_workspace_size(ctypes.byref(desc), _ptr(mask), ctypes.byref(nb))
    if st != NSA_OK:
        raise NsaError(st, "nsa_prefill_backward_workspace_size")
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    res = {"dq": torch.empty((n, hq, d), **f32), "dk": torch.empty((n, hkv, d), **f32),
           "dv": torch.empty((n, hkv, d), **f32), "dw_cmp_k": torch.empty((d, d), **f32),
           "dw_cmp_v": torch.empty((d, d), **f32), "dgate": torch.empty((n, hq, 3), **f32)}
    ws = workspace
    if ws is None or ws.numel() < nb.value:
        ws = torch.empty(max(nb.value, 256), dtype=torch.uint8, device=dev)
    st = lib().nsa_prefill_backward(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(w_cmp_k), _ptr(w_cmp_v),
        _ptr(gate_logits), _ptr(sel_idx if nv > 0 else None), _ptr(dout), _ptr(res["dq"]), _ptr(res["dk"]),
        _ptr(res["dv"]), _ptr(res["dw_cmp_k"]), _ptr(res["dw_cmp_v"]), _ptr(res["dgate"]), _ptr(ws),
        ws.numel(), _stream(stream))
    if st != NSA_OK:
        raise NsaError(st, "nsa_prefill_backward")
    return res


def gate_workspace_size(desc: GateDesc) -> int:
    n = ctypes.c_size_t(0)
    st = lib().nsa_gate_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != NSA_OK:
        raise NsaError(st, "nsa_gate_workspace_size")
    return n.value


def gate_logits(x, w1, b1, w2, b2, n_q_heads, activation="silu", out=None, workspace=None,
                stream=None) -> torch.Tensor:
    """Runs nsa_gate_logits: gate logits [N, Hq, 3] (fp32) of hidden states
    x [N, d_model] through W1 [d_hidden, d_model], act, W2 [3 Hq, d_hidden]
    (bf16 on the device; biases fp32 or None)."""
    n, dm = x.shape
    dh = w1.shape[0]
    _check_dev("x", x, torch.bfloat16, (n, dm))
    _check_dev("w1", w1, torch.bfloat16, (dh, dm))
    _check_dev("w2", w2, torch.bfloat16, (3 * n_q_heads, dh))
    if b1 is not None:
        _check_dev("b1", b1, torch.float32, (dh,))
    if b2 is not None:
        _check_dev("b2", b2, torch.float32, (3 * n_q_heads,))
    if activation not in NSA_ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(NSA_ACTIVATIONS)}")
    desc = GateDesc(n, dm, dh, n_q_heads, NSA_ACTIVATIONS[activation], NSA_DTYPE_BF16)
    if out is None:
        out = torch.empty((n, n_q_heads, 3), dtype=torch.float32, device=x.device)
    _check_dev("out", out, torch.float32, (n, n_q_heads, 3))
    ws_bytes = gate_workspace_size(desc)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=x.device)
    st = lib().nsa_gate_logits(ctypes.byref(desc), _ptr(x), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(out),
                               _ptr(workspace), workspace.numel(), _stream(stream))
    if st != NSA_OK:
        raise NsaError(st, "nsa_gate_logits")
    return out


def cache_append(k_new, v_new, k_cache, v_cache, w_cmp_k, w_cmp_v, k_cmp, v_cmp, cache_len,
                 block=64, stream=None) -> None:
    """Runs nsa_cache_append: the new token's k/v [Bt,Hkv,d] go to row
    cache_len - 1 of the caches [Bt,C,Hkv,d]; a block completed by it is pooled
    into the compressed caches [Bt,C//block,Hkv,d] (all bf16 on the device)."""
    bt, cap, hkv, d = k_cache.shape
    for name, t, shape in (("k_cache", k_cache, (bt, cap, hkv, d)), ("k_new", k_new, (bt, hkv, d)),
                           ("v_new", v_new, (bt, hkv, d)),
                           ("v_cache", v_cache, (bt, cap, hkv, d)), ("w_cmp_k", w_cmp_k, (d, d)),
                           ("w_cmp_v", w_cmp_v, (d, d)), ("k_cmp", k_cmp, (bt, cap // block, hkv, d)),
                           ("v_cmp", v_cmp, (bt, cap // block, hkv, d))):
        _check_dev(name, t, k_cache.dtype, shape)
    desc = DecodeDesc(bt, int(cache_len), hkv, hkv, d, block, 1, 1, 0.0,
                      {torch.bfloat16: NSA_DTYPE_BF16, torch.float32: NSA_DTYPE_FP32}[k_cache.dtype], cap)
    st = lib().nsa_cache_append(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                _ptr(w_cmp_k), _ptr(w_cmp_v), _ptr(k_cmp), _ptr(v_cmp), _stream(stream))
    if st != NSA_OK:
        raise NsaError(st, "nsa_cache_append")


def decode_desc(q, k_cache, top_k, window, block=64, scale=0.0, cache_len=None) -> DecodeDesc:
    """k_cache [Bt, C, Hkv, d]: C rows allocated per sequence, the first
    cache_len (default C) in use."""
    bt, hq, d = q.shape
    cap, hkv = k_cache.shape[1], k_cache.shape[2]
    dt = {torch.bfloat16: NSA_DTYPE_BF16, torch.float32: NSA_DTYPE_FP32}[q.dtype]
    L = cap if cache_len is None else int(cache_len)
    return DecodeDesc(bt, L, hq, hkv, d, block, top_k, window, float(scale), dt, cap)


def decode_workspace_size(desc: DecodeDesc) -> int:
    n = ctypes.c_size_t(0)
    st = lib().nsa_decode_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != NSA_OK:
        raise NsaError(st, "nsa_decode_workspace_size")
    return n.value


def decode(q, k_cache, v_cache, k_cmp, v_cmp, gate_logits, top_k, window, block=64, scale=0.0,
           out=None, want_sel=False, want_lse=False, workspace=None, stream=None, cache_len=None) -> dict:
    """Runs nsa_decode: q [Bt,Hq,d], caches [Bt,C,Hkv,d] with the first
    cache_len rows (default C) in use, compressed caches [Bt,C//B,Hkv,d]
    (bf16), gate_logits [Bt,Hq,3] fp32."""
    desc = decode_desc(q, k_cache, top_k, window, block, scale, cache_len)
    bt, hq, d = q.shape
    cap, hkv = k_cache.shape[1], k_cache.shape[2]
    for name, t, shape in (("q", q, (bt, hq, d)), ("k_cache", k_cache, (bt, cap, hkv, d)),
                           ("v_cache", v_cache, (bt, cap, hkv, d)),
                           ("k_cmp", k_cmp, (bt, cap // block, hkv, d)),
                           ("v_cmp", v_cmp, (bt, cap // block, hkv, d))):
        _check_dev(name, t, q.dtype, shape)
    _check_dev("gate_logits", gate_logits, torch.float32, (bt, hq, 3))
    dev = q.device
    if out is None:
        out = torch.empty((bt, hq, d), dtype=torch.float32, device=dev)
    _check_dev("out", out, torch.float32, (bt, hq, d))
    res = {"out": out}
    sel = lse = None
    if want_sel:
        sel = res["sel_idx"] = torch.empty((bt, hkv, top_k), dtype=torch.int32, device=dev)
    if want_lse:
        lse = res["lse"] = torch.empty((bt, hq), dtype=torch.float32, device=dev)
    ws_bytes = decode_workspace_size(desc)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    st = lib().nsa_decode(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_cmp),
                          _ptr(v_cmp), _ptr(gate_logits), _ptr(out), _ptr(sel), _ptr(lse),
                          _ptr(workspace), workspace.numel(), _stream(stream))
    if st != NSA_OK:
        raise NsaError(st, "nsa_decode")
    res["workspace"] = workspace
    return res


def decode_noalloc(q, k_cache, v_cache, k_cmp, v_cmp, gate_logits, top_k, window, block=64, scale=0.0,
                   out=None, sel_idx=None, lse=None, stream=None, cache_len=None) -> dict:
    """Runs nsa_decode_noalloc (decode with the library's fixed device
    scratch, no workspace): arguments as decode(); preallocated out / sel_idx
    / lse tensors may be passed so that the call itself allocates nothing."""
    desc = decode_desc(q, k_cache, top_k, window, block, scale, cache_len)
    bt, hq, d = q.shape
    cap, hkv = k_cache.shape[1], k_cache.shape[2]
    for name, t, shape in (("q", q, (bt, hq, d)), ("k_cache", k_cache, (bt, cap, hkv, d)),
                           ("v_cache", v_cache, (bt, cap, hkv, d)),
                           ("k_cmp", k_cmp, (bt, cap // block, hkv, d)),
                           ("v_cmp", v_cmp, (bt, cap // block, hkv, d))):
        _check_dev(name, t, q.dtype, shape)
    _check_dev("gate_logits", gate_logits, torch.float32, (bt, hq, 3))
    if out is None:
        out = torch.empty((bt, hq, d), dtype=torch.float32, device=q.device)
    _check_dev("out", out, torch.float32, (bt, hq, d))
    if sel_idx is not None:
        _check_dev("sel_idx", sel_idx, torch.int32, (bt, hkv, top_k))
    if lse is not None:
        _check_dev("lse", lse, torch.float32, (bt, hq))
    st = lib().nsa_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_cmp),
                                  _ptr(v_cmp), _ptr(gate_logits), _ptr(out), _ptr(sel_idx), _ptr(lse),
                                  _stream(stream))
    if st != NSA_OK:
        raise NsaError(st, "nsa_decode_noalloc")
    res = {"out": out}
    if sel_idx is not None:
        res["sel_idx"] = sel_idx
    if lse is not None:
        res["lse"] = lse
    return res


def cmp_pool(x, w, block=64, out_bf16=True, out_f32=False, stream=None) -> dict:
    """Runs nsa_cmp_pool over x [n_rows, H, d] with map w [d, d]."""
    n, h, d = x.shape
    _check_dev("x", x, x.dtype, (n, h, d))
    _check_dev("w", w, x.dtype, (d, d))
    dt = {torch.bfloat16: NSA_DTYPE_BF16, torch.float32: NSA_DTYPE_FP32}[x.dtype]
    res = {}
    ob = of = None
    if out_bf16:
        ob = res["bf16"] = torch.empty((n // block, h, d), dtype=torch.bfloat16, device=x.device)
    if out_f32:
        of = res["f32"] = torch.empty((n // block, h, d), dtype=torch.float32, device=x.device)
    st = lib().nsa_cmp_pool(n, h, d, block, dt, _ptr(x), _ptr(w), _ptr(ob), _ptr(of), _stream(stream))
    if st != NSA_OK:
        raise NsaError(st, "nsa_cmp_pool")
    return res


MFMA_PROBE_FLOPS_PER_WAVE_ROUND = 128 * 16384  # 128 products of 16x16x32 per round


def probe_block_stream(buf, n_wg: int, iters: int, out, stream=None) -> int:
    """Runs nsa_probe_block_stream over buf (a device tensor, a whole number
    of 32 KB blocks) into out (uint32 as int32 [n_wg * 512], device); returns
    the bytes it reads."""
    nbytes = buf.numel() * buf.element_size()
    if not buf.is_cuda or not buf.is_contiguous() or nbytes % 32768 != 0:
        raise ValueError("buf must be a contiguous device tensor of whole 32 KB blocks")
    _check_dev("out", out, torch.int32, (n_wg * 512,))
    st = lib().nsa_probe_block_stream(_ptr(buf), nbytes // 32768, n_wg, iters, _ptr(out), _stream(stream))
    if st != NSA_OK:
        raise NsaError(st, "nsa_probe_block_stream")
    return n_wg * iters * 32768


def probe_mfma_bf16(n_wg: int, iters: int, out, stream=None) -> int:
    """Runs nsa_probe_mfma_bf16 into out (float32 [n_wg * 256], device);
    returns the flops it issues."""
    _check_dev("out", out, torch.float32, (n_wg * 256,))
    st = lib().nsa_probe_mfma_bf16(n_wg, iters, _ptr(out), _stream(stream))
    if st != NSA_OK:
        raise NsaError(st, "nsa_probe_mfma_bf16")
    return n_wg * 4 * iters * MFMA_PROBE_FLOPS_PER_WAVE_ROUND
