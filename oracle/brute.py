"""Brute-force numpy formulation of the VideoNSA attention layer, tiny inputs only.

TEST INFRASTRUCTURE (a second, independent oracle). Where ``nsa_oracle.c``
walks one query at a time through key lists, this file writes every branch as
dense attention under an explicit boolean mask over all (query, key) pairs,
in float64, and ranks blocks with ``numpy.lexsort``. The two agreeing on tiny
inputs pins both against slips of index, sign or operand order.

Steps follow the paper summary page, "Method" (partition by position, the
three NSA branches on vision tokens, sigmoid gates, dense GQA on text), with
the same readings as ``nsa_oracle.c`` (R1-R14 there).
"""
from __future__ import annotations

import math

import numpy as np


def _masked_attention(scores: np.ndarray, mask: np.ndarray, values: np.ndarray):
    """softmax over the last axis of scores restricted to mask; rows with an
    empty mask give zero output and lse = -inf. values: [..., keys, d]."""
    s = np.where(mask, scores, -np.inf)
    m = s.max(axis=-1, keepdims=True, initial=-np.inf)
    empty = ~mask.any(axis=-1, keepdims=True)
    m = np.where(empty, 0.0, m)
    e = np.where(mask, np.exp(s - m), 0.0)
    l = e.sum(axis=-1, keepdims=True)
    p = np.where(empty, 0.0, e / np.where(empty, 1.0, l))
    lse = np.where(empty[..., 0], -np.inf, (m + np.log(np.where(empty, 1.0, l)))[..., 0])
    return p @ values, p, lse


def layer(inp: dict, top_k=None, window=None, scale=None) -> dict:
    s = inp["shape"]
    q = np.asarray(inp["q"], dtype=np.float64)
    k = np.asarray(inp["k"], dtype=np.float64)
    v = np.asarray(inp["v"], dtype=np.float64)
    gates = np.asarray(inp["gates"], dtype=np.float64)
    wk = np.asarray(inp["w_k"], dtype=np.float64)
    wv = np.asarray(inp["w_v"], dtype=np.float64)
    isv = np.asarray(inp["is_vision"]).astype(bool)
    N, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    B = s.block
    kk = s.top_k if top_k is None else top_k
    w = s.window if window is None else window
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    grp = np.arange(hq) // G

    V = np.nonzero(isv)[0]
    T = np.nonzero(~isv)[0]
    nv = len(V)
    nb = nv // B
    qv, kv, vv = q[V], k[V], v[V]  # [nv, H, d]

    # pooling as a dense [nb, nv] averaging matrix, then y = W x
    pool = np.zeros((nb, nv))
    for b in range(nb):
        pool[b, b * B:(b + 1) * B] = 1.0 / B
    kc = np.einsum("bn,ngd->bgd", pool, kv) @ wk.T
    vc = np.einsum("bn,ngd->bgd", pool, vv) @ wv.T

    t_idx = np.arange(nv)
    # compression branch: block b visible once complete
    mask_c = (np.arange(nb)[None, :] + 1) * B <= t_idx[:, None] + 1  # [nv, nb]
    sc = scale * np.einsum("thd,bhd->htb", qv, kc[:, grp])  # [hq, nv, nb]
    o_cmp, p_cmp, lse = _masked_attention(sc, mask_c[None], vc[:, grp].transpose(1, 0, 2))

    # importance score per group, then ranked selection with lexsort
    gscore = p_cmp.reshape(hkv, G, nv, nb).sum(axis=1)  # [hkv, nv, nb]
    sel = -np.ones((nv, hkv, kk), dtype=np.int32)
    mask_s = np.zeros((hkv, nv, nv), dtype=bool)
    blk_of = t_idx // B
    for t in range(nv):
        cur = t // B
        cand = np.array([b for b in range(nb) if mask_c[t, b] and b != cur], dtype=np.int64)
        for g in range(hkv):
            if len(cand):
                order = np.lexsort((cand, -gscore[g, t, cand]))
                chosen = cand[order[: kk - 1]]
            else:
                chosen = cand
            S = np.sort(np.concatenate([[cur], chosen]))
            sel[t, g, : len(S)] = S
            mask_s[g, t] = np.isin(blk_of, S) & (t_idx <= t)
    ss = scale * np.einsum("thd,jhd->htj", qv, kv[:, grp])  # [hq, nv, nv]
    o_sel, _, _ = _masked_attention(ss, mask_s[grp], vv[:, grp].transpose(1, 0, 2))

    # sliding window of exactly w keys
    mask_w = (t_idx[None, :] <= t_idx[:, None]) & (t_idx[None, :] > t_idx[:, None] - w)
    o_swa, _, _ = _masked_attention(ss, mask_w[None], vv[:, grp].transpose(1, 0, 2))

    sig = 1.0 / (1.0 + np.exp(-gates[V]))  # [nv, hq, 3]
    out = np.zeros((N, hq, d))
    o_cmp_t = o_cmp.transpose(1, 0, 2)
    o_sel_t = o_sel.transpose(1, 0, 2)
    o_swa_t = o_swa.transpose(1, 0, 2)
    out[V] = sig[..., 0:1] * o_cmp_t + sig[..., 1:2] * o_sel_t + sig[..., 2:3] * o_swa_t

    # text rows: dense causal over every earlier position, all tokens
    if len(T):
        pos = np.arange(N)
        st = scale * np.einsum("thd,jhd->htj", q[T], k[:, grp])
        mask_t = pos[None, :] <= T[:, None]
        o_t, _, _ = _masked_attention(st, mask_t[None], v[:, grp].transpose(1, 0, 2))
        out[T] = o_t.transpose(1, 0, 2)

    return dict(out=out, kcmp=kc, vcmp=vc, lse=lse.T, sel=sel, ocmp=o_cmp_t, osel=o_sel_t,
                oswa=o_swa_t, scores=gscore.transpose(1, 0, 2), vis=V, text=T)
