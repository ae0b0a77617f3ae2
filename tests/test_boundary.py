"""C-ABI boundary checks that need no GPU: the library loads, exports every
entry point include/nsa.h declares, and rejects bad arguments with the
documented status before anything is launched (pointers here are fake,
16-byte-aligned integers that validation never dereferences)."""
import ctypes
import os
import re

import numpy as np
import pytest

from sparse_attention_long_nsa_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20  # aligned fake device address


def header_functions():
    with open(os.path.join(ROOT, "include", "nsa.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(nsa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    lib = binding.lib()
    names = header_functions()
    assert set(names) == set(binding.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    assert binding.status_string(0) == "ok"
    assert "workspace" in binding.status_string(3)
    assert re.match(r"^\d+\.\d+\.\d+$", binding.version())


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", "/nonexistent/libnsa.so")
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()


def desc(n=1024, hq=28, hkv=4, d=128, block=64, k=16, w=512, dtype=0):
    return binding.PrefillDesc(n, hq, hkv, d, block, k, w, 0.0, dtype)


def call_prefill(ds, mask, ptrs=None, ws=FAKE, ws_bytes=1 << 40):
    p = dict(q=FAKE, k=FAKE, v=FAKE, wk=FAKE, wv=FAKE, g=FAKE, out=FAKE)
    if ptrs:
        p.update(ptrs)
    L = binding.lib()
    return L.nsa_prefill(ctypes.byref(ds) if ds is not None else None, p["q"], p["k"], p["v"],
                         mask.ctypes.data_as(ctypes.c_void_p), p["wk"], p["wv"], p["g"], p["out"],
                         None, None, None, None, ws, ws_bytes, None)


def ws_size(ds, mask):
    n = ctypes.c_size_t(0)
    st = binding.lib().nsa_prefill_workspace_size(ctypes.byref(ds), mask.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n))
    return st, n.value


def vision_mask(n, a, b):
    m = np.zeros(n, np.uint8)
    m[a:b] = 1
    return m


@pytest.mark.parametrize("kw,status", [
    (dict(hq=28, hkv=5), binding.NSA_ERR_INVALID_ARG),
    (dict(k=0), binding.NSA_ERR_INVALID_ARG),
    (dict(w=0), binding.NSA_ERR_INVALID_ARG),
    (dict(n=0), binding.NSA_ERR_INVALID_ARG),
    (dict(dtype=7), binding.NSA_ERR_INVALID_ARG),
    (dict(block=32), binding.NSA_ERR_UNSUPPORTED),
    (dict(d=96), binding.NSA_ERR_UNSUPPORTED),
    (dict(hq=36, hkv=4), binding.NSA_ERR_UNSUPPORTED),   # 9 query heads per KV head
    (dict(hq=32, hkv=4, d=128), binding.NSA_ERR_UNSUPPORTED),
    (dict(k=65), binding.NSA_ERR_UNSUPPORTED),
    (dict(dtype=1), binding.NSA_ERR_UNSUPPORTED),        # fp32 with 7 x 128 query registers
])
def test_descriptor_validation(kw, status):
    ds = desc(**kw)
    n = max(ds.n_tokens, 1)
    mask = vision_mask(n, 0, n)
    assert ws_size(ds, mask)[0] == status
    assert call_prefill(ds, mask) == status


def test_null_descriptor_and_pointers():
    mask = vision_mask(1024, 0, 1024)
    assert call_prefill(None, mask) == binding.NSA_ERR_INVALID_ARG
    for name in ("q", "k", "v", "g", "out", "wk"):
        assert call_prefill(desc(), mask, {name: None}) == binding.NSA_ERR_INVALID_ARG, name


def test_misaligned_pointer_rejected():
    mask = vision_mask(1024, 0, 1024)
    assert call_prefill(desc(), mask, {"q": FAKE + 2}) == binding.NSA_ERR_INVALID_ARG


def test_element_wise_arrays_need_only_element_alignment():
    # gate logits are read one float at a time: a 4-byte-aligned pointer
    # passes the alignment checks (the missing workspace is reported next)
    mask = vision_mask(1024, 0, 1024)
    assert call_prefill(desc(), mask, {"g": FAKE + 4}, ws=None) == binding.NSA_ERR_WORKSPACE
    assert call_prefill(desc(), mask, {"g": FAKE + 2}, ws=None) == binding.NSA_ERR_INVALID_ARG


def test_varlen_slices_of_aligned_arrays_are_accepted():
    # Hkv 1, top_k 3 and a first sequence of 65 vision tokens put the second
    # sequence's selected-index slice 65 * 3 * 4 bytes into the array, which is
    # not a multiple of 16: still accepted (element-wise array)
    L = binding.lib()
    ds = desc(n=65 + 200, hq=8, hkv=1, d=64, k=3, w=64)
    cu = np.array([0, 65, 265], np.int64)
    mask = np.ones(265, np.uint8)
    P = ctypes.c_void_p
    args = [FAKE] * 7 + [None, None, FAKE, FAKE]  # q k v wk wv gates out, kcmp vcmp, sel, lse
    st = L.nsa_prefill_varlen(ctypes.byref(ds), 2, cu.ctypes.data_as(P), args[0], args[1], args[2],
                              mask.ctypes.data_as(P), args[3], args[4], args[5], args[6], args[7], args[8],
                              args[9], args[10], None, 0, None)
    assert st == binding.NSA_ERR_WORKSPACE


def test_several_vision_runs_accepted_with_row_maps_in_the_workspace():
    one = np.concatenate([np.zeros(10, np.uint8), np.ones(1014, np.uint8)])
    two = np.concatenate([np.ones(500, np.uint8), np.zeros(10, np.uint8), np.ones(514, np.uint8)])
    st1, n1 = ws_size(desc(), one)
    st2, n2 = ws_size(desc(), two)
    assert st1 == st2 == binding.NSA_OK
    up = lambda x: (x + 255) // 256 * 256
    # vision row -> position, text row -> position and vision tokens before it
    assert n2 - n1 == up(4 * 1014) + 2 * up(4 * 10)


def test_workspace_checks():
    ds = desc(n=4096 + 512)
    mask = vision_mask(4096 + 512, 0, 4096)
    st, need = ws_size(ds, mask)
    assert st == binding.NSA_OK and need > 0
    assert call_prefill(ds, mask, ws=None) == binding.NSA_ERR_WORKSPACE
    assert call_prefill(ds, mask, ws_bytes=need - 1) == binding.NSA_ERR_WORKSPACE
    assert call_prefill(ds, mask, ws=FAKE + 16, ws_bytes=need) == binding.NSA_ERR_WORKSPACE


def test_workspace_grows_with_context():
    sizes = []
    for nv in (4096, 8192, 16384):
        ds = desc(n=nv + 512)
        st, n = ws_size(ds, vision_mask(nv + 512, 0, nv))
        assert st == binding.NSA_OK
        sizes.append(n)
    assert sizes[0] < sizes[1] < sizes[2]
    # the frame-packed score buffer dominates: ~2.15 GB at 131,072 vision tokens
    st, n = ws_size(desc(n=131072 + 512, k=32, w=256), vision_mask(131072 + 512, 0, 131072))
    assert st == binding.NSA_OK and 2.1e9 < n < 3.0e9


def test_cmp_pool_validation():
    L = binding.lib()
    assert L.nsa_cmp_pool(640, 4, 128, 64, 0, None, FAKE, FAKE, None, None) == binding.NSA_ERR_INVALID_ARG
    assert L.nsa_cmp_pool(640, 4, 128, 64, 0, FAKE, FAKE, None, None, None) == binding.NSA_ERR_INVALID_ARG
    assert L.nsa_cmp_pool(640, 4, 96, 64, 0, FAKE, FAKE, FAKE, None, None) == binding.NSA_ERR_UNSUPPORTED


def test_mfma_probe_validation():
    L = binding.lib()
    assert L.nsa_probe_mfma_bf16(0, 10, FAKE, None) == binding.NSA_ERR_INVALID_ARG
    assert L.nsa_probe_mfma_bf16(8, 0, FAKE, None) == binding.NSA_ERR_INVALID_ARG
    assert L.nsa_probe_mfma_bf16(8, 10, None, None) == binding.NSA_ERR_INVALID_ARG


def ddesc(batch=16, L=131072, hq=28, hkv=4, d=128, block=64, k=16, w=512, dtype=0, cap=0):
    return binding.DecodeDesc(batch, L, hq, hkv, d, block, k, w, 0.0, dtype, cap)


def dws(ds):
    n = ctypes.c_size_t(0)
    return binding.lib().nsa_decode_workspace_size(ctypes.byref(ds), ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw,status", [
    (dict(cap=1000, L=1001), binding.NSA_ERR_INVALID_ARG),  # fewer rows allocated than in use
    (dict(dtype=1), binding.NSA_ERR_UNSUPPORTED),
    (dict(w=131073), binding.NSA_ERR_UNSUPPORTED),
    (dict(k=65), binding.NSA_ERR_UNSUPPORTED),
    (dict(hq=27), binding.NSA_ERR_INVALID_ARG),
    (dict(batch=0), binding.NSA_ERR_INVALID_ARG),
])
def test_decode_validation(kw, status):
    assert dws(ddesc(**kw))[0] == status


@pytest.mark.parametrize("L", [1, 63, 64, 65, 1000, 131071])
def test_decode_any_cache_length(L):
    # the own block may be partial; a larger allocation is allowed
    assert dws(ddesc(L=L, w=1))[0] == binding.NSA_OK
    assert dws(ddesc(L=L, w=1, cap=L + 100))[0] == binding.NSA_OK


def test_decode_workspace_and_pointer_checks():
    st, need = dws(ddesc())
    assert st == binding.NSA_OK and need > 0
    L = binding.lib()
    args = [FAKE] * 7
    assert L.nsa_decode(ctypes.byref(ddesc()), *args, None, None, FAKE, need - 1, None) == binding.NSA_ERR_WORKSPACE
    args[0] = None
    assert L.nsa_decode(ctypes.byref(ddesc()), *args, None, None, FAKE, need, None) == binding.NSA_ERR_INVALID_ARG


def dense_ws(ds):
    n = ctypes.c_size_t(0)
    return binding.lib().nsa_prefill_dense_workspace_size(ctypes.byref(ds), ctypes.byref(n)), n.value


def call_dense(ds, ptrs=None, ws=FAKE, ws_bytes=1 << 40):
    p = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None)
    if ptrs:
        p.update(ptrs)
    return binding.lib().nsa_prefill_dense(ctypes.byref(ds) if ds is not None else None, p["q"], p["k"],
                                           p["v"], p["out"], p["lse"], ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(hq=28, hkv=5), binding.NSA_ERR_INVALID_ARG),
    (dict(n=0), binding.NSA_ERR_INVALID_ARG),
    (dict(dtype=7), binding.NSA_ERR_INVALID_ARG),
    (dict(d=96), binding.NSA_ERR_UNSUPPORTED),
    (dict(hq=32, hkv=4), binding.NSA_ERR_UNSUPPORTED),  # 8 query heads per KV head at d = 128
    # block, top_k and window are not read by the dense mode
    (dict(block=32, k=0, w=0), binding.NSA_OK),
    (dict(dtype=1), binding.NSA_OK),
])
def test_dense_validation(kw, status):
    assert dense_ws(desc(**kw))[0] == status


def test_dense_workspace_and_pointer_checks():
    ds = desc(n=1000)
    st, need = dense_ws(ds)
    # packed key and value tiles of 16 blocks of 64 tokens, bf16
    assert st == binding.NSA_OK and need == 16 * 4 * 2 * 64 * 128 * 2
    st32, need32 = dense_ws(desc(n=1000, dtype=1))
    assert st32 == binding.NSA_OK and need32 > need  # plus fp16 copies of q, k, v
    assert call_dense(None) == binding.NSA_ERR_INVALID_ARG
    for name in ("q", "k", "v", "out"):
        assert call_dense(ds, {name: None}) == binding.NSA_ERR_INVALID_ARG, name
    assert call_dense(ds, {"lse": FAKE + 4}) == binding.NSA_ERR_INVALID_ARG
    assert call_dense(ds, ws=None) == binding.NSA_ERR_WORKSPACE
    assert call_dense(ds, ws_bytes=need - 1) == binding.NSA_ERR_WORKSPACE
    assert call_dense(ds, ws=FAKE + 16, ws_bytes=need) == binding.NSA_ERR_WORKSPACE


def call_append(ds, ptrs=None):
    p = dict(kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, wk=FAKE, wv=FAKE, kcmp=FAKE, vcmp=FAKE)
    if ptrs:
        p.update(ptrs)
    return binding.lib().nsa_cache_append(ctypes.byref(ds) if ds is not None else None, p["kn"], p["vn"],
                                          p["kc"], p["vc"], p["wk"], p["wv"], p["kcmp"], p["vcmp"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), binding.NSA_ERR_INVALID_ARG),
    (dict(L=0), binding.NSA_ERR_INVALID_ARG),
    (dict(cap=100, L=101), binding.NSA_ERR_INVALID_ARG),   # the new row does not fit
    (dict(dtype=1), binding.NSA_ERR_UNSUPPORTED),
    (dict(block=32), binding.NSA_ERR_UNSUPPORTED),
    (dict(d=96), binding.NSA_ERR_UNSUPPORTED),
])
def test_cache_append_validation(kw, status):
    assert call_append(ddesc(**kw)) == status


def test_cache_append_pointer_checks():
    assert call_append(None) == binding.NSA_ERR_INVALID_ARG
    for name in ("kn", "vn", "kc", "vc", "wk", "wv", "kcmp", "vcmp"):
        assert call_append(ddesc(), {name: None}) == binding.NSA_ERR_INVALID_ARG, name
    assert call_append(ddesc(), {"kc": FAKE + 8}) == binding.NSA_ERR_INVALID_ARG


def varlen_ws(ds, cu, mask):
    cu = np.asarray(cu, np.int64)
    n = ctypes.c_size_t(0)
    st = binding.lib().nsa_prefill_varlen_workspace_size(
        ctypes.byref(ds), len(cu) - 1, cu.ctypes.data_as(ctypes.c_void_p),
        mask.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n))
    return st, n.value


def test_varlen_workspace_is_the_largest_sequence():
    m1 = vision_mask(1024 + 64, 0, 1024)
    m2 = vision_mask(4096 + 32, 32, 4096 + 32)
    mask = np.concatenate([m1, m2])
    ds = desc(n=len(mask))
    st, n = varlen_ws(ds, [0, len(m1), len(mask)], mask)
    assert st == binding.NSA_OK
    assert n == max(ws_size(desc(n=len(m1)), m1)[1], ws_size(desc(n=len(m2)), m2)[1])


@pytest.mark.parametrize("cu", [[0, 500, 1000], [1, 1024], [0, 1025], [0, 600, 600, 1024], [0, 700, 500, 1024]])
def test_varlen_bad_offsets(cu):
    mask = vision_mask(1024, 0, 1024)
    ok = cu == [0, 500, 1000]
    st, _ = varlen_ws(desc(n=1000 if ok else 1024), cu, mask)
    assert st == (binding.NSA_OK if ok else binding.NSA_ERR_INVALID_ARG)


def test_varlen_validates_every_sequence_first():
    mask = vision_mask(2048, 0, 2048)
    cu = np.array([0, 1024, 2048], np.int64)
    L = binding.lib()

    def call(ptrs):
        p = dict(q=FAKE, k=FAKE, v=FAKE, wk=FAKE, wv=FAKE, g=FAKE, out=FAKE, ws=FAKE)
        p.update(ptrs)
        return L.nsa_prefill_varlen(ctypes.byref(desc(n=2048)), 2, cu.ctypes.data_as(ctypes.c_void_p),
                                    p["q"], p["k"], p["v"], mask.ctypes.data_as(ctypes.c_void_p), p["wk"],
                                    p["wv"], p["g"], p["out"], None, None, None, None, p["ws"], 1 << 40, None)
    assert call({"q": None}) == binding.NSA_ERR_INVALID_ARG
    assert call({"ws": None}) == binding.NSA_ERR_WORKSPACE
    assert call({"g": FAKE + 2}) == binding.NSA_ERR_INVALID_ARG


def gdesc(n=1000, dm=3584, dh=1024, hq=28, act=0, dtype=0):
    return binding.GateDesc(n, dm, dh, hq, act, dtype)


def gate_ws(ds):
    n = ctypes.c_size_t(0)
    st = binding.lib().nsa_gate_workspace_size(ctypes.byref(ds) if ds is not None else None, ctypes.byref(n))
    return st, n.value


def call_gate(ds, ptrs=None, ws=FAKE, ws_bytes=1 << 40):
    p = dict(x=FAKE, w1=FAKE, b1=None, w2=FAKE, b2=None, out=FAKE)
    if ptrs:
        p.update(ptrs)
    return binding.lib().nsa_gate_logits(ctypes.byref(ds) if ds is not None else None, p["x"], p["w1"], p["b1"],
                                         p["w2"], p["b2"], p["out"], ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=0), binding.NSA_ERR_INVALID_ARG),
    (dict(dh=0), binding.NSA_ERR_INVALID_ARG),
    (dict(act=3), binding.NSA_ERR_INVALID_ARG),
    (dict(dtype=7), binding.NSA_ERR_INVALID_ARG),
    (dict(dtype=1), binding.NSA_ERR_UNSUPPORTED),
    (dict(dm=3584 + 32), binding.NSA_ERR_UNSUPPORTED),
    (dict(dh=1024 + 64), binding.NSA_ERR_UNSUPPORTED),
    (dict(hq=33), binding.NSA_ERR_UNSUPPORTED),   # 99 outputs > 96
    (dict(hq=32, act=2), binding.NSA_OK),
])
def test_gate_validation(kw, status):
    assert gate_ws(gdesc(**kw))[0] == status


def test_gate_workspace_and_pointer_checks():
    st, need = gate_ws(gdesc())
    assert st == binding.NSA_OK and need == 1000 * 1024 * 2  # the fp16 hidden layer
    assert gate_ws(None)[0] == binding.NSA_ERR_INVALID_ARG
    assert call_gate(None) == binding.NSA_ERR_INVALID_ARG
    for name in ("x", "w1", "w2", "out"):
        assert call_gate(gdesc(), {name: None}) == binding.NSA_ERR_INVALID_ARG, name
    assert call_gate(gdesc(), {"b1": FAKE + 4}) == binding.NSA_ERR_INVALID_ARG
    assert call_gate(gdesc(), ws=None) == binding.NSA_ERR_WORKSPACE
    assert call_gate(gdesc(), ws_bytes=need - 1) == binding.NSA_ERR_WORKSPACE
    assert call_gate(gdesc(), ws=FAKE + 16, ws_bytes=need) == binding.NSA_ERR_WORKSPACE


def test_gate_size_limits():
    assert gate_ws(gdesc(n=(1 << 30) + 1, dh=256))[0] == binding.NSA_ERR_UNSUPPORTED
    assert gate_ws(gdesc(n=1 << 27, dh=2048))[0] == binding.NSA_ERR_UNSUPPORTED
    assert gate_ws(gdesc(n=1 << 26, dh=2048))[0] == binding.NSA_OK


def bwd_ws(ds, mask):
    n = ctypes.c_size_t(0)
    st = binding.lib().nsa_prefill_backward_workspace_size(ctypes.byref(ds), mask.ctypes.data_as(ctypes.c_void_p),
                                                          ctypes.byref(n))
    return st, n.value


def call_bwd(ds, mask, ptrs=None, ws=FAKE, ws_bytes=1 << 40):
    names = ("q", "k", "v", "wk", "wv", "g", "sel", "dout", "dq", "dk", "dv", "dwk", "dwv", "dg")
    p = {n: FAKE for n in names}
    if ptrs:
        p.update(ptrs)
    return binding.lib().nsa_prefill_backward(
        ctypes.byref(ds), p["q"], p["k"], p["v"], mask.ctypes.data_as(ctypes.c_void_p), p["wk"], p["wv"], p["g"],
        p["sel"], p["dout"], p["dq"], p["dk"], p["dv"], p["dwk"], p["dwv"], p["dg"], ws, ws_bytes, None)


def test_backward_validation_and_workspace():
    m = vision_mask(1024 + 64, 32, 1024 + 32)
    st, need = bwd_ws(desc(n=len(m)), m)
    # 1,024 vision tokens (16 blocks, one 2,048-token chunk), 64 text tokens,
    # 28 / 4 heads, d 128, k 16; every array rounded up to 256 bytes
    a = lambda x: (x + 255) // 256 * 256
    nb, tile = 16 * 4 * 128, 2 * 64 * 128 * 2 * 4  # a tile: K and V rows, fp16, four KV groups
    parts = [4]                                   # the status word
    parts += [4 * nb] * 6 + [2 * nb] * 2          # compressed k / v, means, their gradients; fp16 copies
    parts += [tile * 16, tile * 17, tile * 1]     # tiles: vision blocks, positions, compressed keys
    parts += [4 * 6 * 1024 * 28, 4 * 2 * 64 * 28]  # per-branch statistics: vision rows, text rows
    parts += [4 * 4 * 16 * 32, 4 * 4 * 16, 4 * (4 * 16 + 1), 4 * 1024 * 4 * 16]  # who chose which block
    parts += [4 * 1 * 1 * 4 * 2 * 64 * 128]       # partial compressed-key gradients
    parts += [4 * 8 * 64 * 28 * 130]              # text rows: eight key-tile splits
    assert st == binding.NSA_OK and need == sum(a(x) for x in parts) + 256
    assert bwd_ws(desc(n=len(m), dtype=1), m)[0] == binding.NSA_ERR_UNSUPPORTED
    two_runs = vision_mask(len(m), 0, 500) | vision_mask(len(m), 600, 1000)
    assert bwd_ws(desc(n=len(m)), two_runs)[0] == binding.NSA_ERR_UNSUPPORTED
    assert bwd_ws(desc(n=len(m), k=0), m)[0] == binding.NSA_ERR_INVALID_ARG
    ds = desc(n=len(m))
    for name in ("q", "k", "v", "wk", "wv", "g", "sel", "dout", "dq", "dk", "dv", "dwk", "dwv", "dg"):
        assert call_bwd(ds, m, {name: None}) == binding.NSA_ERR_INVALID_ARG, name
    assert call_bwd(ds, m, {"dq": FAKE + 4}) == binding.NSA_ERR_INVALID_ARG
    assert call_bwd(ds, m, ws=None) == binding.NSA_ERR_WORKSPACE
    assert call_bwd(ds, m, ws_bytes=need - 1) == binding.NSA_ERR_WORKSPACE
    text_only = np.zeros(64, np.uint8)  # no vision rows: no selection needed
    assert bwd_ws(desc(n=64), text_only)[0] == binding.NSA_OK


def test_workspace_status_and_spin_limit_arguments():
    L = binding.lib()
    flags = ctypes.c_int32(0)
    assert L.nsa_workspace_status(None, None, ctypes.byref(flags)) == binding.NSA_ERR_INVALID_ARG
    assert L.nsa_workspace_status(FAKE, None, None) == binding.NSA_ERR_INVALID_ARG
    assert L.nsa_workspace_status(FAKE + 16, None, ctypes.byref(flags)) == binding.NSA_ERR_INVALID_ARG
    assert L.nsa_debug_set_spin_limit(5) == binding.NSA_OK
    assert L.nsa_debug_set_spin_limit(0) == binding.NSA_OK  # default restored
    assert "bounded wait" in binding.status_string(binding.NSA_ERR_KERNEL)


def test_prefill_workspace_starts_with_the_status_word():
    # the status word takes the workspace's first 256-byte slot
    one = vision_mask(1024, 0, 1024)
    st, n = ws_size(desc(), one)
    assert st == binding.NSA_OK and n % 256 == 0 and n >= 256


def test_block_stream_probe_arguments():
    L = binding.lib()
    bad = binding.NSA_ERR_INVALID_ARG
    assert L.nsa_probe_block_stream(None, 4, 1, 2, FAKE, None) == bad
    assert L.nsa_probe_block_stream(FAKE, 4, 1, 2, None, None) == bad
    assert L.nsa_probe_block_stream(FAKE + 4, 4, 1, 2, FAKE, None) == bad  # 16-byte alignment
    assert L.nsa_probe_block_stream(FAKE, 0, 1, 2, FAKE, None) == bad
    assert L.nsa_probe_block_stream(FAKE, 4, 0, 2, FAKE, None) == bad
    assert L.nsa_probe_block_stream(FAKE, 4, 1, 3, FAKE, None) == bad  # blocks go two at a time
