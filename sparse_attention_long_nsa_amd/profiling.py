"""Profiling helpers around rocprofv3 (run on the GPU machine, summarised on
any machine):

* ``copy``: a plain device copy of known size, used to calibrate the memory
  counters (FETCH_SIZE / WRITE_SIZE, KiB per dispatch) before they are read
  for the layer's kernels;
* ``trace-summary``: per-kernel call counts and average durations from a
  ``rocprofv3 --kernel-trace --output-format csv`` run of bench.py, beside
  the event-timed averages bench.py printed in the same run;
* ``pmc-summary``: HBM-side bytes per launch of every kernel from two
  ``--pmc`` runs (FETCH_SIZE, then WRITE_SIZE) scaled by the copy probe's
  factors; writes a text table and one JSON record per kernel, which bench.py
  reads as the roofline's ``traffic`` while the kernel source is unchanged.

  python -m sparse_attention_long_nsa_amd.profiling copy --mib 1024 --reps 3
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:  # also runnable as a plain script
    sys.path.insert(0, ROOT)

# kernel symbol substring -> (short name, source file). Launches of one
# kernel told apart by their grid (pack_kv_kernel: vision blocks /
# compressed chunks / text rows; dec_item_kernel: compressed chunks and
# window slices / selected blocks) are named through grid_names, see
# short_name.
KERNELS = [
    ("sel_attn_kernel", "sel_attn", "sparse_attention_long_nsa_amd/csrc/nsa_sel_attn.hip"),
    ("cmp_lse_kernel", "cmp_lse", "sparse_attention_long_nsa_amd/csrc/nsa_cmp_attn.hip"),
    ("cmp_attn_dma_kernel", "cmp_attn", "sparse_attention_long_nsa_amd/csrc/nsa_cmp_attn.hip"),
    ("cmp_attn_kernel", "cmp_attn", "sparse_attention_long_nsa_amd/csrc/nsa_cmp_attn.hip"),
    ("swa_attn_kernel", "swa_attn", "sparse_attention_long_nsa_amd/csrc/nsa_fine_attn.hip"),
    ("text_attn_kernel", "text_attn", "sparse_attention_long_nsa_amd/csrc/nsa_fine_attn.hip"),
    ("text_merge_kernel", "text_merge", "sparse_attention_long_nsa_amd/csrc/nsa_fine_attn.hip"),
    ("dense_attn_kernel", "dense_attn", "sparse_attention_long_nsa_amd/csrc/nsa_fine_attn.hip"),
    ("row_map_kernel", "row_maps", "sparse_attention_long_nsa_amd/csrc/nsa_rowmap.hip"),
    ("topk_kernel", "blk_score_topk", "sparse_attention_long_nsa_amd/csrc/nsa_topk.hip"),
    ("cmp_pool_kernel", "@grid", "sparse_attention_long_nsa_amd/csrc/nsa_pool.hip"),
    ("pool_mean_kernel", "cmp_pool_mean", "sparse_attention_long_nsa_amd/csrc/nsa_pool.hip"),
    ("pool_map_kernel", "cmp_pool_map", "sparse_attention_long_nsa_amd/csrc/nsa_pool.hip"),
    ("pack_kv_kernel", "@grid", "sparse_attention_long_nsa_amd/csrc/nsa_sel_attn.hip"),
    ("dec_item_kernel", "@grid", "sparse_attention_long_nsa_amd/csrc/nsa_decode.hip"),
    ("dec_select_kernel", "dec_select", "sparse_attention_long_nsa_amd/csrc/nsa_decode.hip"),
    ("dec_combine_kernel", "dec_combine", "sparse_attention_long_nsa_amd/csrc/nsa_decode.hip"),
    ("mfma_loop_kernel", "mfma_probe", "sparse_attention_long_nsa_amd/csrc/nsa_probe.hip"),
    ("gate_hidden_kernel", "gate_hidden", "sparse_attention_long_nsa_amd/csrc/nsa_gate.hip"),
    ("gate_out_kernel", "gate_out", "sparse_attention_long_nsa_amd/csrc/nsa_gate.hip"),
    ("bwd_fill_kernel", "bwd_selclear", "sparse_attention_long_nsa_amd/csrc/nsa_backward.hip"),
    ("bwd_pool_kernel", "bwd_pool", "sparse_attention_long_nsa_amd/csrc/nsa_backward.hip"),
    ("bwd_pack_kernel", "bwd_pack", "sparse_attention_long_nsa_amd/csrc/nsa_backward.hip"),
    ("bwd_sel", "bwd_sellist", "sparse_attention_long_nsa_amd/csrc/nsa_backward.hip"),
    ("bwd_qt_kernel", "bwd_q_text", "sparse_attention_long_nsa_amd/csrc/nsa_backward.hip"),
    ("bwd_qtmerge_kernel", "bwd_q_text", "sparse_attention_long_nsa_amd/csrc/nsa_backward.hip"),
    ("bwd_qtsum_kernel", "bwd_q_text", "sparse_attention_long_nsa_amd/csrc/nsa_backward.hip"),
    ("bwd_q_kernel", "bwd_q_vis", "sparse_attention_long_nsa_amd/csrc/nsa_backward.hip"),
    ("bwd_kv_kernel", "bwd_kv", "sparse_attention_long_nsa_amd/csrc/nsa_backward.hip"),
    ("bwd_kvc_kernel", "bwd_kv_cmp", "sparse_attention_long_nsa_amd/csrc/nsa_backward.hip"),
    ("bwd_creduce_kernel", "bwd_cmp_sum", "sparse_attention_long_nsa_amd/csrc/nsa_backward.hip"),
    ("bwd_cmp_w_kernel", "bwd_cmp_w", "sparse_attention_long_nsa_amd/csrc/nsa_backward.hip"),
    ("bwd_cmp_tok_kernel", "bwd_cmp_tok", "sparse_attention_long_nsa_amd/csrc/nsa_backward.hip"),
]
DECODE_KERNELS = ("dec_item_cmp_win", "dec_item_sel", "dec_select", "dec_combine")
DENSE_KERNELS = ("pack_dense", "dense_attn")
GATE_KERNELS = ("gate_hidden", "gate_out")
BWD_KERNELS = ("bwd_selclear", "bwd_pool", "bwd_pack", "bwd_sellist", "bwd_q_vis", "bwd_q_text", "bwd_kv",
               "bwd_kv_cmp", "bwd_cmp_sum", "bwd_cmp_w", "bwd_cmp_tok")
PREFILL_KERNELS = ("sel_attn", "cmp_lse", "cmp_attn", "swa_attn", "text_attn", "text_merge", "blk_score_topk", "cmp_pool",
                   "cmp_pool_mean", "cmp_pool_map", "pack_kv", "pack_cmp", "pack_text")


def short_name(kernel_name: str, grid: int, grid_names: dict):
    for sub, short, src in KERNELS:
        if sub in kernel_name or sub.replace("_", "") in kernel_name:
            if short == "@grid":
                return grid_names.get((sub, grid), sub + "_other"), src
            return short, src
    return None, None


def pack_grid_names(n_frames: int, n_cch: int, n_tchunks: int, hkv: int, n_cmp: int,
                    n_all_tiles: int = 0) -> dict:
    """Grid sizes (threads) of the prefill's packing and pooling launches ->
    names (the layer pools keys and values in one launch of two grid rows;
    single-row pooling launches are other callers', e.g. cache building);
    n_all_tiles: 64-token tiles of the whole sequence (the dense mode packs
    them all)."""
    k = "pack_kv_kernel"
    names = {(k, n_frames * hkv * 256): "pack_kv", (k, n_cch * hkv * 256): "pack_cmp",
             (k, n_tchunks * hkv * 256): "pack_text", ("cmp_pool_kernel", 2 * min(n_cmp, 1024) * 256): "cmp_pool"}
    if n_all_tiles:
        names[(k, n_all_tiles * hkv * 256)] = "pack_dense"
    return names


def decode_grid_names(batch: int, hkv: int, n_blk: int, top_k: int, window: int) -> dict:
    """Grid sizes (threads) of the two decode item launches -> names."""
    pairs, k = batch * hkv, "dec_item_kernel"
    n_items0 = -(-n_blk // 64) + -(-window // 64)
    return {(k, pairs * n_items0 * 256): "dec_item_cmp_win", (k, pairs * top_k * 256): "dec_item_sel"}


def _grid(row: dict) -> int:
    if "Grid_Size" in row:
        return int(row["Grid_Size"])
    return int(row["Grid_Size_X"]) * int(row.get("Grid_Size_Y", 1)) * int(row.get("Grid_Size_Z", 1))


def _bench_line(log_path: str):
    with open(log_path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{") and '"metric"' in line:
                return json.loads(line)
    return None


def source_digest(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def trace_summary(trace_csv: str, bench_log: str, grid_names: dict, title: str, command: str,
                  out_md: str, group: str = "prefill") -> None:
    keep = {"decode": DECODE_KERNELS, "dense": DENSE_KERNELS, "gate": GATE_KERNELS,
            "backward": BWD_KERNELS}.get(group, PREFILL_KERNELS)
    dur = defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        name, _ = short_name(r["Kernel_Name"], _grid(r), grid_names)
        if name in keep:
            dur[name].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6)
    bench = _bench_line(bench_log)
    if group == "decode":
        dec = (bench or {}).get("decode") or {}
        kern = {k: {"avg_ms": round(v["avg_us"] * 1e-3, 4)} for k, v in dec.get("kernels", {}).items()}
    elif group == "dense":
        kern = ((bench or {}).get("dense_mode") or {}).get("kernels", {})
    elif group == "backward":
        kern = {k: {"avg_ms": v} for k, v in ((bench or {}).get("backward") or {}).get("kernels", {}).items()}
    elif group == "gate":
        kern = {k: {"avg_ms": v} for k, v in ((bench or {}).get("gate_prologue") or {}).get("kernels", {}).items()}
    else:
        kern = bench["kernels"] if bench else {}
    total = sum(sum(v) / len(v) for v in dur.values())
    rows = sorted(dur.items(), key=lambda kv: -sum(kv[1]) / len(kv[1]))
    lines = [f"# Kernel trace: {title}", "", "Command (from the repository root, on one MI355X):", "",
             "```", command, "```", ""]
    if bench and group == "decode" and bench.get("decode"):
        d = bench["decode"]
        lines += [f"bench.py in the same process reported {d['us_per_step']} us per decode step "
                  f"({d['roofline']['frac'] * 100:.1f}% of the HBM roofline); its event-timed per-kernel "
                  "averages are listed beside the profiler's. Under the profiler every launch of these "
                  "few-microsecond kernels gets a gap of its own, so that step time is inflated; the kernel "
                  "durations are not, and their sum is the unprofiled step.", ""]
    elif bench and group == "dense" and bench.get("dense_mode"):
        d = bench["dense_mode"]
        lines += [f"bench.py in the same process reported {d['ms_per_step']} ms per dense step "
                  f"({d['tflops']} TF/s of algorithmic flops, {d['mfma_peak_frac'] * 100:.1f}% of the bf16 "
                  "peak); its event-timed per-kernel averages are listed beside the profiler's.", ""]
    elif bench and group == "backward" and bench.get("backward"):
        d = bench["backward"]
        lines += [f"bench.py in the same process reported {d['ms_per_step']} ms per backward call over "
                  f"{d['n_vision']} vision + {d['n_text']} text tokens (k {d['top_k']}, w {d['window']}): "
                  f"{d['tflops']} TF/s of algorithmic flops ({d.get('mfma_peak_frac', 0) * 100:.1f}% of the "
                  "fp16 matrix peak); its event-timed per-kernel averages are listed beside the profiler's. "
                  "Rows that stand for several launches per call (bwd_sellist: mask, count, prefix sum, "
                  "decode; bwd_pack: three tile sets; bwd_q_text: two split passes, merge, sum) give the "
                  "profiler's average per launch and the events' time for the whole group.", ""]
    elif bench and group == "gate" and bench.get("gate_prologue"):
        d = bench["gate_prologue"]
        lines += [f"bench.py in the same process reported {d['ms_per_step']} ms per gate prologue over "
                  f"{d['n_tokens']} tokens (d_model {d['d_model']}, d_hidden {d['d_hidden']}); hidden layer "
                  f"{d.get('gate_hidden')}, output layer {d.get('gate_out')}; its event-timed per-kernel "
                  "averages are listed beside the profiler's.", ""]
    elif bench:
        lines += [f"bench.py in the same process reported {bench['ms_per_step']} ms/step "
                  f"({bench['value']:.0f} tokens/s); its event-timed per-kernel averages are listed "
                  "beside the profiler's."
                  + (" The compression attention is two kernels (cmp_lse: pass 1, the log-sum-exp; "
                     "cmp_attn: pass 2); the events time them together, under cmp_attn."
                     if "cmp_lse" in dur else "")
                  + (" The pooling's block means are taken inside pack_kv; cmp_pool is the maps alone "
                     "(they also write the packed compressed chunks)."
                     if "cmp_pool_map" in dur and "cmp_pool_mean" not in dur else ""), ""]
    lines += ["| kernel | calls | avg ms (rocprofv3) | avg ms (bench events) | share |", "|---|---|---|---|---|"]
    for name, v in rows:
        avg = sum(v) / len(v)
        ev = kern.get(name, {}).get("avg_ms", "")
        if name == "cmp_pool_map" and "cmp_pool_mean" not in dur:  # the maps alone are the event "cmp_pool"
            ev = kern.get("cmp_pool", {}).get("avg_ms", "")
        lines.append(f"| {name} | {len(v)} | {avg:.4f} | {ev} | {100 * avg / total:.1f}% |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counter_avgs(path: str, grid_names: dict) -> dict:
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        name, src = short_name(r["Kernel_Name"], _grid(r), grid_names)
        if name in PREFILL_KERNELS:
            vals[(name, src)].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def _copy_kib(path: str) -> float:
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path)) if "copyBuffer" in r["Kernel_Name"]]
    return sum(vals) / len(vals)


def pmc_summary(fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str,
                copy_mib: int, grid_names: dict, workload: str, commands: list, bench_log: str,
                out_md: str, out_dir: str) -> None:
    copy_kib = copy_mib * 1024.0
    f_fetch = copy_kib / _copy_kib(copy_fetch_csv)
    f_write = copy_kib / _copy_kib(copy_write_csv)
    fetch = _counter_avgs(fetch_csv, grid_names)
    write = _counter_avgs(write_csv, grid_names)
    bench = _bench_line(bench_log) if bench_log else None
    kern = bench["kernels"] if bench else {}
    lines = [f"# HBM-side traffic per launch: {workload}", "",
             "Counters: rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one run each), "
             "averaged over the dispatches of each kernel, scaled by a plain 1 GiB device copy "
             f"(`profiling.py copy`): FETCH x {f_fetch:.3f}, WRITE x {f_write:.3f} "
             "(the copy reads and writes exactly 1 GiB). FETCH_SIZE counts everything the L2 "
             "fetches from the memory fabric, Infinity Cache hits included, so these are upper "
             "bounds on HBM bytes.", "", "Commands (from the repository root, on one MI355X):", "", "```"]
    lines += commands + ["```", "",
                         "| kernel | read GB | write GB | total GB | kernel ms (events) | GB/s |",
                         "|---|---|---|---|---|---|"]
    recs = []
    for key in sorted(fetch, key=lambda k: -(fetch[k] * f_fetch + write.get(k, 0.0) * f_write)):
        name, src = key
        rd = fetch[key] * f_fetch * 1024
        wr = write.get(key, 0.0) * f_write * 1024
        ms = kern.get(name, {}).get("avg_ms")
        gbs = f"{(rd + wr) / (ms * 1e-3) / 1e9:.0f}" if ms else ""
        lines.append(f"| {name} | {rd / 1e9:.3f} | {wr / 1e9:.3f} | {(rd + wr) / 1e9:.3f} | {ms or ''} | {gbs} |")
        recs.append({"kernel": name, "workload": workload, "source": src,
                     "source_sha256_16": source_digest(os.path.join(ROOT, src)),
                     "fetch_kib_per_dispatch": round(fetch[key], 3),
                     "write_kib_per_dispatch": round(write.get(key, 0.0), 3),
                     "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4),
                     "hbm_bytes_per_launch": round(rd + wr), "commands": commands})
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    for rec in recs:
        with open(os.path.join(out_dir, f"{rec['kernel']}_{workload}_pmc.json"), "w") as f:
            json.dump(rec, f, indent=1)


def counter_summary(csv_a: str, csv_b: str, grid_names: dict, workload: str, commands: list,
                    bench_log: str, out_md: str) -> None:
    """Instruction mix and pipe utilisation per kernel from two SQ counter runs.

    Cycle counters of the SQ (SQ_WAVE_CYCLES, SQ_WAIT_ANY, SQ_ACTIVE_INST_*)
    count in units of four clocks, summed over waves; SQ_VALU_MFMA_BUSY_CYCLES
    counts clocks summed over SIMDs. Utilisation is taken against 256 CUs x 4
    SIMDs at 2.4 GHz over the dispatch's duration."""
    simds, clk = 256 * 4, 2.4e9
    vals = defaultdict(lambda: defaultdict(list))
    dur = defaultdict(list)
    for path in (csv_a, csv_b):
        for r in csv.DictReader(open(path)):
            name, _ = short_name(r["Kernel_Name"], _grid(r), grid_names)
            if name not in PREFILL_KERNELS:
                continue
            vals[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
            dur[name].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    bench = _bench_line(bench_log) if bench_log else None
    kern = bench["kernels"] if bench else {}
    lines = [f"# Instruction mix and pipe utilisation: {workload}", "",
             "Counters: two rocprofv3 --pmc runs of SQ counters (one dispatch per kernel each). "
             "SQ cycle counters count units of four clocks summed over waves; the matrix-core busy "
             "counter counts clocks summed over SIMDs. Utilisation is against 256 CUs x 4 SIMDs at "
             "2.4 GHz over the dispatch; `issued TF` counts every 16x16x32 matrix instruction "
             "(16,384 flops), `useful` is the kernel's algorithmic flops from bench.py over the issued ones.",
             "", "Commands (from the repository root, on one MI355X):", "", "```"] + commands + ["```", ""]
    lines += ["| kernel | ms | waves | VALU / wave | MFMA / wave | LDS / wave | SALU / wave | exp share of VALU | "
              "VALU busy | MFMA busy | waiting | LDS bank-conflict cycles | issued TF | useful |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for name in sorted(vals, key=lambda n: -sum(dur[n]) / len(dur[n])):
        v = {c: sum(x) / len(x) for c, x in vals[name].items()}
        secs = sum(dur[name]) / len(dur[name])
        cyc = secs * clk
        waves = v.get("SQ_WAVES", 0.0) or 1.0

        def per_wave(c):
            return f"{v[c] / waves:.0f}" if c in v else ""

        valu_busy = v.get("SQ_ACTIVE_INST_VALU", 0.0) * 4 / (simds * cyc)
        mfma_busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (simds * cyc)
        wait = v.get("SQ_WAIT_ANY", 0.0) / v["SQ_WAVE_CYCLES"] if v.get("SQ_WAVE_CYCLES") else 0.0
        exp_share = 4 * v.get("SQ_INSTS_VALU_TRANS_F32", 0.0) / (
            v.get("SQ_INSTS_VALU", 1.0) + 3 * v.get("SQ_INSTS_VALU_TRANS_F32", 0.0))
        conflict = v.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(v.get("SQ_ACTIVE_INST_LDS", 0.0), 1.0)
        issued = v.get("SQ_INSTS_MFMA", 0.0) * 16384 / 1e12
        tf = kern.get(name, {}).get("tflops")
        ms = kern.get(name, {}).get("avg_ms")
        both = issued
        if name == "cmp_attn" and "cmp_lse" in vals:  # the events time both passes as cmp_attn
            lse = vals["cmp_lse"].get("SQ_INSTS_MFMA", [])
            both += (sum(lse) / len(lse) if lse else 0.0) * 16384 / 1e12
        useful = f"{tf * ms * 1e-3 / both:.0%}" if (tf and ms and both) else ""
        lines.append(f"| {name} | {secs * 1e3:.3f} | {waves:.0f} | {per_wave('SQ_INSTS_VALU')} | "
                     f"{per_wave('SQ_INSTS_MFMA')} | {per_wave('SQ_INSTS_LDS')} | {per_wave('SQ_INSTS_SALU')} | "
                     f"{exp_share:.0%} | {valu_busy:.0%} | {mfma_busy:.0%} | {wait:.0%} | {conflict:.2%} | "
                     f"{issued:.2f} | {useful} |")
    lines += ["", "`exp share` weights the transcendental instructions (exp2) four times, their issue cost "
              "relative to plain fp32 vector instructions."]
    if "cmp_lse" in vals:
        lines += ["", "The compression attention is two kernels, cmp_lse (pass 1) and cmp_attn (pass 2); "
                  "cmp_attn's `useful` divides the algorithmic flops of both passes by the matrix "
                  "instructions both issue."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def copy_probe(mib: int, reps: int) -> None:
    import torch
    n = mib * 1024 * 1024 // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x {reps}: each dispatch reads {mib * 1024} KiB and writes {mib * 1024} KiB",
          flush=True)


def mfma_peak(n_wg: int = 256 * 8, iters: int = 400, reps: int = 8) -> dict:
    """Dense bf16 matrix-core rate measured by the MFMA-loop probe: the best
    of `reps` timed launches (events on the launch stream)."""
    import torch
    from sparse_attention_long_nsa_amd import binding
    out = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda:0")
    st = torch.cuda.current_stream()
    binding.probe_mfma_bf16(n_wg, 4, out, st)  # warm-up
    best = float("inf")
    flops = 0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        flops = binding.probe_mfma_bf16(n_wg, iters, out, st)
        e1.record(st)
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("MFMA probe produced non-finite values")
    return {"tflops": round(flops / (best * 1e-3) / 1e12, 1), "ms": round(best, 4), "flops": flops,
            "workgroups": n_wg, "rounds": iters, "instr": "v_mfma_f32_16x16x32_bf16"}


def block_stream(sizes_mib=(4, 64, 268, 1024), n_wg: int = 4096, iters: int = 96, reps: int = 3) -> dict:
    """Rate of pseudo-random whole 32 KB block reads (the selection kernel's
    copy pattern) for several buffer sizes: the best of `reps` timed launches
    of the block-stream probe per size, in TB/s. 268 MiB is the packed
    key/value size of the 128K workload; 4 MiB fits one XCD's L2."""
    import torch
    from sparse_attention_long_nsa_amd import binding
    out = torch.empty(n_wg * 512, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    res = {}
    for mib in sizes_mib:
        buf = torch.ones(mib * 1024 * 1024 // 4, dtype=torch.int32, device="cuda:0")
        binding.probe_block_stream(buf, n_wg, 2, out, st)  # warm-up
        best = float("inf")
        nbytes = 0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            nbytes = binding.probe_block_stream(buf, n_wg, iters, out, st)
            e1.record(st)
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1))
        res[f"{mib}_mib"] = round(nbytes / (best * 1e-3) / 1e12, 2)
        del buf
    return {"tb_per_s": res, "block_bytes": 32768, "workgroups": n_wg, "blocks_per_workgroup": iters}


def _layer_grids(workload: str) -> dict:
    from sparse_attention_long_nsa_amd.inputs import DECODE_PRESETS, PREFILL_PRESETS
    if workload in DECODE_PRESETS:
        s = DECODE_PRESETS[workload]
        return decode_grid_names(s.batch, s.n_kv_heads, s.cache_len // s.block, s.top_k, s.window)
    s = PREFILL_PRESETS[workload]
    n_frames = -(-s.n_vis // s.block)
    n_cch = -(-(s.n_vis // s.block) // s.block)
    return pack_grid_names(n_frames, n_cch, -(-s.n_text // s.block), s.n_kv_heads, s.n_vis // s.block,
                           -(-s.n_tokens // s.block))


def main(argv=None) -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=3)
    sub.add_parser("mfma-peak")
    sub.add_parser("block-stream")
    t = sub.add_parser("trace-summary")
    t.add_argument("--trace-csv", required=True)
    t.add_argument("--bench-log", required=True)
    t.add_argument("--workload", default="qwen_128k_k32_w256")
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--group", choices=("prefill", "decode", "dense", "gate", "backward"), default="prefill")
    m = sub.add_parser("pmc-summary")
    for k in ("fetch", "write", "copy-fetch", "copy-write"):
        m.add_argument(f"--{k}-csv", required=True)
    m.add_argument("--copy-mib", type=int, default=1024)
    m.add_argument("--workload", default="qwen_128k_k32_w256")
    m.add_argument("--bench-log", default=None)
    m.add_argument("--command", action="append", default=[])
    m.add_argument("--out-md", required=True)
    m.add_argument("--out-dir", required=True)
    x = sub.add_parser("counter-summary")
    x.add_argument("--csv-a", required=True)
    x.add_argument("--csv-b", required=True)
    x.add_argument("--workload", default="qwen_128k_k32_w256")
    x.add_argument("--bench-log", default=None)
    x.add_argument("--command", action="append", default=[])
    x.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "copy":
        copy_probe(a.mib, a.reps)
    elif a.cmd == "mfma-peak":
        print(json.dumps(mfma_peak()), flush=True)
    elif a.cmd == "block-stream":
        print(json.dumps(block_stream()), flush=True)
    elif a.cmd == "trace-summary":
        trace_summary(a.trace_csv, a.bench_log, _layer_grids(a.workload), a.title, a.command, a.out, a.group)
    elif a.cmd == "counter-summary":
        counter_summary(a.csv_a, a.csv_b, _layer_grids(a.workload), a.workload, a.command, a.bench_log, a.out)
    else:
        pmc_summary(a.fetch_csv, a.write_csv, a.copy_fetch_csv, a.copy_write_csv, a.copy_mib,
                    _layer_grids(a.workload), a.workload, a.command, a.bench_log, a.out_md, a.out_dir)


if __name__ == "__main__":
    main(sys.argv[1:])
