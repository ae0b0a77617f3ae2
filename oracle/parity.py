"""Comparison of GPU results with the fp64 oracle (test infrastructure).

Index parity (selected blocks): the query's own block must be present and
the -1 padding must match; where the two sets differ, the differing blocks
of each side are sorted by the oracle's importance score and paired, and the
row is exempt when every paired gap is at most ``tie_tol`` (score units: the
sum of the group's per-head probabilities). Any other difference counts.

Output parity: the oracle is re-evaluated with the GPU's selection on exempt
rows (index injection), then max |d| <= 1e-2 and mean |d| <= 1e-3 over every
compared element, fp32 GPU against fp64 oracle.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle

TIE_TOL = 1e-3
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


@dataclasses.dataclass
class IndexReport:
    rows: int
    exact: int
    exempt: int
    counted: int
    max_exempt_gap: float
    exempt_rows: np.ndarray  # indices into the compared rows

    def __str__(self):
        return (f"index parity: {self.rows} rows x groups, exact {self.exact}, exempt {self.exempt}"
                f" (max gap {self.max_exempt_gap:.3g}), counted {self.counted}")


def index_parity(gpu_sel: np.ndarray, ora_sel: np.ndarray, scores_fn, cur_blocks: np.ndarray,
                 tie_tol: float = TIE_TOL) -> IndexReport:
    """gpu_sel, ora_sel: [n, Hkv, k] int; cur_blocks: [n] own block of each row;
    scores_fn(row_indices) -> oracle scores [len, Hkv, n_blk] for those rows."""
    n, hkv, k = ora_sel.shape
    same = np.all(gpu_sel == ora_sel, axis=2)  # [n, hkv]
    bad_rows = np.nonzero(~np.all(same, axis=1))[0]
    exempt_rows, counted, exempt, max_gap = [], 0, 0, 0.0
    if len(bad_rows):
        sc = scores_fn(bad_rows)
        for j, r in enumerate(bad_rows):
            row_ok = True
            for g in range(hkv):
                if same[r, g]:
                    continue
                gs, os_ = gpu_sel[r, g], ora_sel[r, g]
                if (gs < 0).sum() != (os_ < 0).sum() or cur_blocks[r] not in set(gs.tolist()):
                    counted += 1
                    row_ok = False
                    continue
                a = sorted(set(os_[os_ >= 0].tolist()) - set(gs.tolist()), key=lambda b: -sc[j, g, b])
                b_ = sorted(set(gs[gs >= 0].tolist()) - set(os_.tolist()), key=lambda b: -sc[j, g, b])
                if len(a) != len(b_) or any(x < 0 or x > cur_blocks[r] for x in b_):
                    counted += 1
                    row_ok = False
                    continue
                gaps = [sc[j, g, x] - sc[j, g, y] for x, y in zip(a, b_)]
                if max(gaps) <= tie_tol:
                    exempt += 1
                    max_gap = max(max_gap, max(gaps))
                else:
                    counted += 1
                    row_ok = False
            if row_ok:
                exempt_rows.append(r)
    return IndexReport(n * hkv, int(same.sum()), exempt, counted, max_gap,
                       np.asarray(exempt_rows, dtype=np.int64))


@dataclasses.dataclass
class OutputReport:
    max_abs: float
    mean_abs: float
    n: int

    def ok(self, max_abs=MAX_ABS, mean_abs=MEAN_ABS) -> bool:
        return self.max_abs <= max_abs and self.mean_abs <= mean_abs

    def __str__(self):
        return f"output parity: max|d| {self.max_abs:.3g}, mean|d| {self.mean_abs:.3g} over {self.n}"


def compare(gpu: np.ndarray, ref: np.ndarray) -> OutputReport:
    d = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
    if not np.all(np.isfinite(d)):
        return OutputReport(float("inf"), float("inf"), d.size)
    return OutputReport(float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0, d.size)


def check_prefill(inp: dict, gpu: dict, rows: np.ndarray, top_k=None, window=None,
                  tie_tol: float = TIE_TOL):
    """Oracle at global positions ``rows`` against the GPU's full outputs.
    gpu: numpy dict with "out" [N,Hq,d] and "sel" [N_v,Hkv,k] (vision-local).
    Returns (IndexReport or None, OutputReport, oracle result)."""
    s = inp["shape"]
    isv = np.asarray(inp["is_vision"]).astype(bool)
    vloc = np.cumsum(isv) - 1
    rows = np.asarray(rows, dtype=np.int64)
    ref = oracle.prefill(inp, rows=rows, top_k=top_k, window=window,
                         want=("sel", "lse", "counts"))
    vis_mask = isv[rows]
    rep = None
    out_ref = ref["out"].copy()
    if vis_mask.any() and "sel" in gpu:
        vrows = rows[vis_mask]
        g_sel = gpu["sel"][vloc[vrows]]
        o_sel = ref["sel"][vis_mask]
        cur = vloc[vrows] // s.block

        def scores_fn(idx):
            return oracle.prefill(inp, rows=vrows[idx], top_k=top_k, window=window,
                                  want=("scores",))["scores"]

        rep = index_parity(g_sel, o_sel, scores_fn, cur, tie_tol)
        if len(rep.exempt_rows):
            inj_rows = vrows[rep.exempt_rows]
            inj = oracle.prefill(inp, rows=inj_rows, inject_sel=g_sel[rep.exempt_rows],
                                 top_k=top_k, window=window, want=())
            pos_in_rows = np.nonzero(vis_mask)[0][rep.exempt_rows]
            out_ref[pos_in_rows] = inj["out"]
    outrep = compare(gpu["out"][rows], out_ref)
    return rep, outrep, ref


def sample_rows(inp: dict, n_random: int = 256, seed: int = 0, n_text: int = 32) -> np.ndarray:
    """Stratified row sample: the first two blocks, block-boundary rows of
    random blocks, the last 256 vision rows, random vision rows and some text
    rows (first, last and random)."""
    s = inp["shape"]
    isv = np.asarray(inp["is_vision"]).astype(bool)
    V = np.nonzero(isv)[0]
    T = np.nonzero(~isv)[0]
    rng = np.random.default_rng(seed)
    picks = [V[: 2 * s.block]]
    nb = len(V) // s.block
    if nb > 2:
        blocks = rng.choice(np.arange(2, nb), size=min(16, nb - 2), replace=False)
        for b in blocks:
            picks.append(V[b * s.block + np.array([0, 1, s.block // 2, s.block - 2, s.block - 1])])
    picks.append(V[-256:])
    picks.append(rng.choice(V, size=min(n_random, len(V)), replace=False))
    if len(T):
        picks.append(T[[0, -1]])
        picks.append(rng.choice(T, size=min(n_text, len(T)), replace=False))
    return np.unique(np.concatenate(picks))


def stratified_rows(inp: dict, n_vision: int = 8192, n_boundary_blocks: int = 64, n_last: int = 1024,
                    seed: int = 0) -> np.ndarray:
    """Row sample for the largest workloads: the first two blocks, every row
    of the edges of ``n_boundary_blocks`` random blocks (their first two, middle
    and last two rows), the last ``n_last`` vision rows, random vision rows up
    to ``n_vision`` in all, and every text row."""
    s = inp["shape"]
    isv = np.asarray(inp["is_vision"]).astype(bool)
    V = np.nonzero(isv)[0]
    T = np.nonzero(~isv)[0]
    rng = np.random.default_rng(seed)
    picks = [V[: 2 * s.block], V[-n_last:]]
    nb = len(V) // s.block
    if nb > 2:
        blocks = rng.choice(np.arange(2, nb), size=min(n_boundary_blocks, nb - 2), replace=False)
        for b in blocks:
            picks.append(V[b * s.block + np.array([0, 1, s.block // 2, s.block - 2, s.block - 1])])
    vis = np.unique(np.concatenate(picks))
    rest = np.setdiff1d(V, vis)
    extra = max(0, min(n_vision - len(vis), len(rest)))
    vis = np.union1d(vis, rng.choice(rest, size=extra, replace=False))
    return np.union1d(vis, T)


def decode_inputs_cmp(inp: dict, round_fn) -> tuple:
    """Compressed caches for a decode workload, pooled by the oracle and
    rounded by round_fn (to the dtype both sides then consume)."""
    s = inp["shape"]
    kc = np.stack([cmp_pool_f32(inp["k_cache"][b], inp["w_k"], s.block) for b in range(s.batch)])
    vc = np.stack([cmp_pool_f32(inp["v_cache"][b], inp["w_v"], s.block) for b in range(s.batch)])
    return round_fn(kc), round_fn(vc)


def cmp_pool_f32(x, w, block):
    return oracle.cmp_pool(x, w, block).astype(np.float32)


def check_decode(inp: dict, kc: np.ndarray, vc: np.ndarray, gpu_out: np.ndarray,
                 gpu_sel: np.ndarray, tie_tol: float = TIE_TOL):
    """Oracle decode on the same compressed caches; index parity with the
    near-tie rule, then output parity with the GPU selection injected on
    exempt sequences."""
    s = inp["shape"]
    ref = oracle.decode(inp, kc, vc, want=("sel", "scores", "lse"))
    cur = np.full(s.batch, (s.cache_len - 1) // s.block)
    rep = index_parity(gpu_sel, ref["sel"], lambda idx: ref["scores"][idx], cur, tie_tol)
    out_ref = ref["out"].copy()
    if len(rep.exempt_rows):
        inj = oracle.decode(inp, kc, vc, inject_sel=gpu_sel, want=())
        out_ref[rep.exempt_rows] = inj["out"][rep.exempt_rows]
    return rep, compare(gpu_out, out_ref), ref
