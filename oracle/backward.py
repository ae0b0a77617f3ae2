"""fp64 oracle of the layer's backward pass: gradients by automatic
differentiation of a plain torch re-statement of the forward.

TEST INFRASTRUCTURE, like the rest of this package: only the tests,
``__graft_entry__.smoke()`` and the CPU baseline leg of ``bench.py`` may use
it; the GPU library shares no code with it.

The pages' main use of the layer is end-to-end training (model card,
"Training Details"; paper summary, "Method"). The block selection is a
discrete choice, so it has no gradient: the selected blocks are an input
here (the forward's choice), and gradients flow through q, k, v (all three
branches and the text rows), the gate logits and both compression maps.

The forward below restates the layer as dense attention under explicit
masks, in float64, with the readings of ``nsa_oracle.c``: vision tokens are
taken in position order; block b is the mean of vision keys 64 b .. 64 b + 63
mapped by W (y = W x); the compression branch of vision token t sees blocks
b with 64 (b + 1) <= t + 1; the selection branch sees the vision keys j <= t
whose block is selected for (t, KV group); the window sees vision keys
t - w < j <= t; an empty key set contributes zero; branch outputs are mixed by
sigmoid gates (cmp, sel, swa); text rows attend causally to every earlier
position. It is pinned against the C oracle's forward and, for its
gradients, against finite differences.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def _attend(s: torch.Tensor, mask: torch.Tensor, values: torch.Tensor) -> torch.Tensor:
    """softmax of scores s over the keys allowed by mask, applied to values;
    a row with no allowed key gives zeros. s [..., T, K], values [..., K, d]."""
    mask = mask.expand_as(s)
    empty = ~mask.any(dim=-1, keepdim=True)
    s = s.masked_fill(~mask, float("-inf"))
    s = torch.where(empty, torch.zeros_like(s), s)
    p = torch.softmax(s, dim=-1)
    p = torch.where(mask & ~empty, p, torch.zeros_like(p))
    return p @ values


def forward(q, k, v, w_k, w_v, gates, is_vision, sel, block: int, window: int, scale: float,
            branches: bool = False, rows=None):
    """Layer output [N, Hq, d] (torch float64) for tensors q [N, Hq, d],
    k/v [N, Hkv, d], w_k/w_v [d, d], gates [N, Hq, 3]; is_vision [N] (numpy,
    0/1), sel [N_v, Hkv, top_k] selected blocks of the vision tokens (-1 pads).
    With ``branches`` also returns the three branch outputs of the vision rows.

    ``rows`` (positions, ascending; default all) restricts the queries that
    are evaluated: the same formulas with the query index running over those
    positions only (every key stays available), so the result is
    [len(rows), Hq, d] and its cost grows with len(rows) instead of N. The
    branch outputs are then those of the vision rows among ``rows``."""
    isv = np.asarray(is_vision).astype(bool)
    N, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    grp = torch.arange(hq) // G
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    vloc = np.cumsum(isv) - 1  # vision-local index of each position
    V = torch.from_numpy(np.nonzero(isv)[0])
    Rv = rows[isv[rows]]  # evaluated vision positions
    Rt = rows[~isv[rows]]  # evaluated text positions
    nv = len(V)
    nb = nv // block
    kv, vv = k[V], v[V]  # [nv, H, d]

    kbar = kv[: nb * block].reshape(nb, block, hkv, d).mean(dim=1)
    vbar = vv[: nb * block].reshape(nb, block, hkv, d).mean(dim=1)
    kc, vc = kbar @ w_k.T, vbar @ w_v.T  # [nb, hkv, d]

    t_idx = torch.from_numpy(vloc[Rv])  # vision-local index of each evaluated vision query
    qv = q[torch.from_numpy(Rv)]  # [nr, Hq, d]
    # compression: [hq, nr, nb]
    mask_c = ((torch.arange(nb)[None, :] + 1) * block <= t_idx[:, None] + 1)[None]
    sc = scale * torch.einsum("thd,bhd->htb", qv, kc[:, grp])
    o_cmp = _attend(sc, mask_c, vc[:, grp].permute(1, 0, 2))

    # selection over vision keys j <= t of the selected blocks: [hq, nr, nv]
    sel = np.asarray(sel)[vloc[Rv]]
    blk_of = np.arange(nv) // block
    # columns: blocks 0 .. nb (nb: a trailing partial block, which its own
    # tokens select), then one column that collects the -1 pads
    nr = len(Rv)
    chosen = np.zeros((hkv, nr, nb + 2), dtype=bool)
    for g in range(hkv):
        s_g = sel[:, g, :]
        rr = np.repeat(np.arange(nr), s_g.shape[1])
        cols = np.where(s_g.reshape(-1) >= 0, s_g.reshape(-1), nb + 1)
        chosen[g, rr, cols] = True
    j_idx = torch.arange(nv)
    causal = j_idx[None, :] <= t_idx[:, None]
    mask_s = torch.from_numpy(chosen[:, :, blk_of]) & causal[None]  # [hkv, nr, nv]
    ss = scale * torch.einsum("thd,jhd->htj", qv, kv[:, grp])
    vals = vv[:, grp].permute(1, 0, 2)
    o_sel = _attend(ss, mask_s[grp], vals)

    # sliding window of w keys
    mask_w = (causal & (j_idx[None, :] > t_idx[:, None] - window))[None]
    o_swa = _attend(ss, mask_w, vals)

    sig = torch.sigmoid(gates[torch.from_numpy(Rv)])  # [nr, hq, 3]
    o_c, o_s, o_w = (o.permute(1, 0, 2) for o in (o_cmp, o_sel, o_swa))
    out_v = sig[..., 0:1] * o_c + sig[..., 1:2] * o_s + sig[..., 2:3] * o_w
    at = {int(r): i for i, r in enumerate(rows)}
    out = torch.zeros((len(rows), hq, d), dtype=q.dtype)
    out = out.index_put((torch.tensor([at[int(r)] for r in Rv], dtype=torch.long),), out_v)
    if len(Rt):
        pos = torch.arange(N)
        T = torch.from_numpy(Rt)
        st = scale * torch.einsum("thd,jhd->htj", q[T], k[:, grp])
        mask_t = (pos[None, :] <= T[:, None])[None]
        o_t = _attend(st, mask_t, v[:, grp].permute(1, 0, 2)).permute(1, 0, 2)
        out = out.index_put((torch.tensor([at[int(r)] for r in Rt], dtype=torch.long),), o_t)
    if branches:
        return out, (o_c, o_s, o_w)
    return out


def gradients(inp: dict, sel, dout, top_k=None, window=None, scale=None, rows=None) -> dict:
    """Gradients of sum(out * dout) (fp64 numpy) with respect to q, k, v,
    w_k, w_v and the gate logits, for the inputs of a prefill workload and
    the given selection sel [N_v, Hkv, top_k]. With ``rows`` (positions,
    ascending) only those rows of ``dout`` [N, Hq, d] enter the sum: the
    gradients of sum over r in rows of out[r] * dout[r], evaluated from those
    queries alone (equal to the full gradients when dout is zero elsewhere)."""
    s = inp["shape"]
    w = s.window if window is None else window
    d = inp["q"].shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    names = ("q", "k", "v", "w_k", "w_v", "gates")
    t = {n: torch.tensor(np.asarray(inp[n], dtype=np.float64), requires_grad=True) for n in names}
    out = forward(t["q"], t["k"], t["v"], t["w_k"], t["w_v"], t["gates"], inp["is_vision"], sel,
                  s.block, w, scale, rows=rows)
    dsel = np.asarray(dout, dtype=np.float64)
    if rows is not None:
        dsel = dsel[np.asarray(rows, dtype=np.int64)]
    grads = torch.autograd.grad(out, [t[n] for n in names], grad_outputs=torch.as_tensor(dsel))
    return {n: g.numpy() for n, g in zip(names, grads)}
