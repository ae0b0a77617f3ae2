"""fp64 CPU oracle for the VideoNSA attention layer (forward).

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package. The GPU library never
links, loads or calls it, and it shares no code with the GPU library.

Two independent formulations live here:
  * ``nsa_oracle.c`` (wrapped below): the method's steps in the order the
    VideoNSA pages give them (paper summary page, "Method"), one query at a
    time, in double precision, OpenMP over queries;
  * ``brute.py``: the same layer written as dense attention under explicit
    boolean masks in numpy, for tiny inputs only.

Parity unpinned: the exact form of the learned compression map, the
importance score, the attention-budget accounting and the decode position are
not fixed by the pages; they follow the readings stated in ``nsa_oracle.c``
and are pinned only as far as those readings go.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "nsa_oracle.c")
_LIB_PATH = os.path.join(_DIR, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, strict IEEE arithmetic)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Desc(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("scale", ctypes.c_double),
    ]


class _DecDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("cache_len", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("scale", ctypes.c_double),
    ]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.ora_prefill.argtypes = [ctypes.POINTER(_Desc)] + [P] * 7 + [P, ctypes.c_int64] + [P] * 11
        lib.ora_prefill.restype = ctypes.c_int
        lib.ora_decode.argtypes = [ctypes.POINTER(_DecDesc)] + [P] * 15
        lib.ora_decode.restype = ctypes.c_int
        lib.ora_cmp_pool.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P]
        lib.ora_cmp_pool.restype = ctypes.c_int
        lib.ora_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().ora_num_threads())


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def cmp_pool(x: np.ndarray, w: np.ndarray, block: int) -> np.ndarray:
    """Compressed tokens of complete blocks: x [n,Hkv,d] -> [n//block,Hkv,d] fp64."""
    x = _f32(x)
    w = _f32(w)
    n, hkv, d = x.shape
    out = np.empty((n // block, hkv, d), dtype=np.float64)
    rc = _load().ora_cmp_pool(n, hkv, d, block, _ptr(x), _ptr(w), _ptr(out))
    if rc != 0:
        raise RuntimeError(f"ora_cmp_pool failed ({rc})")
    return out


def prefill(inp: dict, rows=None, inject_sel=None, top_k=None, window=None, scale=0.0,
            want=("out", "lse", "sel", "ocmp", "osel", "oswa", "counts", "kcmp"),
            outputs: bool = True) -> dict:
    """Evaluate the layer at global positions ``rows`` (default: all).

    ``inp`` holds q [N,Hq,d], k/v [N,Hkv,d], is_vision [N], w_k, w_v [d,d],
    gates [N,Hq,3] and ``shape`` (for block, top_k, window). Returns fp64
    arrays indexed by the requested rows. With ``outputs=False`` the layer
    output ("out") and the branch outputs are not computed: a selection-only
    evaluation (pooling, compression attention, scores and selection), a
    fraction of the cost, whose sel/lse/scores equal the full call's."""
    s = inp["shape"]
    q, k, v = _f32(inp["q"]), _f32(inp["k"]), _f32(inp["v"])
    gates = _f32(inp["gates"])
    wk, wv = _f32(inp["w_k"]), _f32(inp["w_v"])
    isv = np.ascontiguousarray(inp["is_vision"], dtype=np.uint8)
    N, hq, d = q.shape
    hkv = k.shape[1]
    kk = s.top_k if top_k is None else top_k
    ww = s.window if window is None else window
    rows = np.arange(N, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.shape[0]
    nv = int(isv.sum())
    n_blk = nv // s.block
    inj = None if inject_sel is None else np.ascontiguousarray(inject_sel, dtype=np.int32)
    res = {}

    def alloc(name, shape, dt=np.float64):
        if name in want:
            res[name] = np.empty(shape, dtype=dt)
            return res[name]
        return None

    if not outputs:
        want = tuple(w for w in want if w not in ("ocmp", "osel", "oswa"))
    out = np.empty((n, hq, d), dtype=np.float64) if outputs else None
    if outputs:
        res["out"] = out
    lse = alloc("lse", (n, hq))
    sel = alloc("sel", (n, hkv, kk), np.int32)
    ocmp = alloc("ocmp", (n, hq, d))
    osel = alloc("osel", (n, hq, d))
    oswa = alloc("oswa", (n, hq, d))
    counts = alloc("counts", (n, 3), np.int64)
    scores = alloc("scores", (n, hkv, n_blk))
    kc = alloc("kcmp", (n_blk, hkv, d))
    vc = None
    if kc is not None:
        vc = res["vcmp"] = np.empty((n_blk, hkv, d), dtype=np.float64)
    desc = _Desc(N, hq, hkv, d, s.block, kk, ww, float(scale))
    rc = _load().ora_prefill(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(isv), _ptr(wk), _ptr(wv), _ptr(gates),
        _ptr(rows), n, _ptr(inj), _ptr(out), _ptr(lse), _ptr(sel), _ptr(ocmp), _ptr(osel),
        _ptr(oswa), _ptr(counts), _ptr(scores), _ptr(kc), _ptr(vc))
    if rc != 0:
        raise RuntimeError(f"ora_prefill failed ({rc})")
    return res


def dense(inp: dict, rows=None) -> np.ndarray:
    """Dense-NSA mode (paper summary page, "Key claims" and "Results": the same
    weights under full attention): every token attends causally to all earlier
    tokens with GQA, which is the oracle's text-row path applied to every row,
    so this evaluates the layer with every token marked as text. Returns
    out [n_rows,Hq,d] fp64."""
    all_text = dict(inp)
    all_text["is_vision"] = np.zeros_like(np.asarray(inp["is_vision"]), dtype=np.uint8)
    return prefill(all_text, rows=rows, want=())["out"]


def decode(inp: dict, k_cmp: np.ndarray, v_cmp: np.ndarray, inject_sel=None,
           top_k=None, window=None, scale=0.0, want=("sel", "lse", "scores", "counts")) -> dict:
    """One query per sequence at the last cache slot; ``inp`` holds q [Bt,Hq,d],
    k_cache/v_cache [Bt,L,Hkv,d], gates [Bt,Hq,3]; compressed caches of the
    floor(L/B) complete blocks given. The own block is (L-1)//B (partial when
    B does not divide L)."""
    s = inp["shape"]
    q = _f32(inp["q"])
    kcache, vcache = _f32(inp["k_cache"]), _f32(inp["v_cache"])
    gates = _f32(inp["gates"])
    kc, vc = _f32(k_cmp), _f32(v_cmp)
    bt, L, hkv, d = kcache.shape
    hq = q.shape[1]
    kk = s.top_k if top_k is None else top_k
    ww = s.window if window is None else window
    n_blk = L // s.block
    inj = None if inject_sel is None else np.ascontiguousarray(inject_sel, dtype=np.int32)
    res = {"out": np.empty((bt, hq, d), dtype=np.float64)}
    for name, shape, dt in (("sel", (bt, hkv, kk), np.int32), ("lse", (bt, hq), np.float64),
                            ("ocmp", (bt, hq, d), np.float64), ("osel", (bt, hq, d), np.float64),
                            ("oswa", (bt, hq, d), np.float64), ("counts", (bt, 3), np.int64),
                            ("scores", (bt, hkv, n_blk), np.float64)):
        res[name] = np.empty(shape, dtype=dt) if name in want else None
    desc = _DecDesc(bt, L, hq, hkv, d, s.block, kk, ww, float(scale))
    rc = _load().ora_decode(
        ctypes.byref(desc), _ptr(q), _ptr(kcache), _ptr(vcache), _ptr(kc), _ptr(vc), _ptr(gates),
        _ptr(inj), _ptr(res["out"]), _ptr(res["sel"]), _ptr(res["lse"]), _ptr(res["ocmp"]),
        _ptr(res["osel"]), _ptr(res["oswa"]), _ptr(res["counts"]), _ptr(res["scores"]))
    if rc != 0:
        raise RuntimeError(f"ora_decode failed ({rc})")
    return {k2: v2 for k2, v2 in res.items() if v2 is not None}
