"""Host-side logic of the profiling summaries (no GPU): kernel naming by
symbol and grid, and the trace table for the prefill and decode groups."""
import csv
import json

from sparse_attention_long_nsa_amd import profiling as prof


def _trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, grid, ns in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Start_Timestamp": 1000,
                        "End_Timestamp": 1000 + ns})


def test_grid_names_tell_launches_apart():
    g = prof._layer_grids("decode_16x128k")
    # 16 sequences x 4 KV groups; 2048 compressed blocks -> 32 chunks, window 512 -> 8 slices
    assert g[("dec_item_kernel", 64 * 40 * 256)] == "dec_item_cmp_win"
    assert g[("dec_item_kernel", 64 * 16 * 256)] == "dec_item_sel"
    name, src = prof.short_name("void nsa::(anonymous namespace)::dec_item_kernel<128, 7>(nsa::DecodeParams, int)",
                                64 * 16 * 256, g)
    assert name == "dec_item_sel" and src.endswith("nsa_decode.hip")
    p = prof._layer_grids("qwen_128k_k32_w256")
    assert p[("pack_kv_kernel", 2048 * 4 * 256)] == "pack_kv"
    assert p[("cmp_pool_kernel", 2 * 1024 * 256)] == "cmp_pool"
    assert prof.short_name("pack_kv_kernel<128, true>", 12345, p)[0] == "pack_kv_kernel_other"
    assert prof.short_name("some_other_kernel", 1, p) == (None, None)


def test_trace_summary_groups(tmp_path):
    trace = tmp_path / "trace.csv"
    _trace(trace, [("sel_attn_kernel<128, 7, true>", 655360, 11_000_000),
                   ("sel_attn_kernel<128, 7, true>", 655360, 13_000_000),
                   ("dec_select_kernel<128, 7, 32>", 16384, 9_000),
                   ("mfma_loop_kernel", 524288, 2_000_000)])
    log = tmp_path / "bench.log"
    line = {"metric": "m", "value": 1.0, "ms_per_step": 20.0,
            "kernels": {"sel_attn": {"avg_ms": 11.9}},
            "decode": {"us_per_step": 44.0, "roofline": {"frac": 0.33},
                       "kernels": {"dec_select": {"avg_us": 9.5}}}}
    log.write_text("noise\n" + json.dumps(line) + "\n")
    out = tmp_path / "p.md"
    prof.trace_summary(str(trace), str(log), prof._layer_grids("qwen_128k_k32_w256"), "t", "cmd", str(out))
    text = out.read_text()
    assert "| sel_attn | 2 | 12.0000 | 11.9 | 100.0% |" in text
    assert "dec_select" not in text and "mfma" not in text
    out_d = tmp_path / "d.md"
    prof.trace_summary(str(trace), str(log), prof._layer_grids("decode_16x128k"), "t", "cmd", str(out_d),
                       group="decode")
    text = out_d.read_text()
    assert "| dec_select | 1 | 0.0090 | 0.0095 | 100.0% |" in text
    assert "44.0 us per decode step" in text


def test_trace_summary_gate_group(tmp_path):
    trace = tmp_path / "trace.csv"
    _trace(trace, [("nsa::(anonymous namespace)::gate_hidden_kernel(nsa::GateParams, int)", 1064960, 1_450_000),
                   ("nsa::(anonymous namespace)::gate_out_kernel(nsa::GateParams)", 131584, 220_000),
                   ("sel_attn_kernel<128, 7, true>", 655360, 11_000_000)])
    log = tmp_path / "bench.log"
    line = {"metric": "m", "value": 1.0, "ms_per_step": 20.0, "kernels": {},
            "gate_prologue": {"ms_per_step": 1.7, "n_tokens": 131584, "d_model": 3584, "d_hidden": 1024,
                              "kernels": {"gate_hidden": 1.45, "gate_out": 0.22},
                              "gate_hidden": {"tflops": 665.0}, "gate_out": {"gbs": 1400.0}}}
    log.write_text(json.dumps(line) + "\n")
    out = tmp_path / "g.md"
    prof.trace_summary(str(trace), str(log), prof._layer_grids("qwen_128k_k32_w256"), "t", "cmd", str(out),
                       group="gate")
    text = out.read_text()
    assert "| gate_hidden | 1 | 1.4500 | 1.45 |" in text
    assert "| gate_out | 1 | 0.2200 | 0.22 |" in text
    assert "sel_attn" not in text and "1.7 ms per gate prologue" in text


def test_counter_summary_utilisation(tmp_path):
    # one sel_attn dispatch of 1 ms: 1,024 SIMDs x 2.4e6 clocks; counters
    # chosen so that vector busy = 50%, matrix busy = 25%, waiting = 40%
    cyc = 2.4e6 * 1024
    a = {"SQ_WAVES": 100.0, "SQ_INSTS_VALU": 1000.0, "SQ_INSTS_MFMA": 1e9, "SQ_INSTS_LDS": 300.0,
         "SQ_INSTS_SALU": 50.0, "SQ_WAVE_CYCLES": 1e9, "SQ_BUSY_CYCLES": 1.0, "SQ_WAIT_INST_ANY": 1.0}
    b = {"SQ_ACTIVE_INST_VALU": 0.5 * cyc / 4, "SQ_VALU_MFMA_BUSY_CYCLES": 0.25 * cyc, "SQ_WAIT_ANY": 0.4e9,
         "SQ_ACTIVE_INST_LDS": 100.0, "SQ_LDS_BANK_CONFLICT": 1.0, "SQ_INSTS_VALU_TRANS_F32": 0.0,
         "SQ_ACTIVE_INST_ANY": 1.0, "SQ_ACTIVE_INST_MISC": 1.0}
    paths = []
    for tag, counters in (("a", a), ("b", b)):
        path = tmp_path / f"{tag}.csv"
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value",
                                              "Start_Timestamp", "End_Timestamp"])
            w.writeheader()
            for c, v in counters.items():
                w.writerow({"Kernel_Name": "sel_attn_kernel<128, 7, false>", "Grid_Size": 1, "Counter_Name": c,
                            "Counter_Value": v, "Start_Timestamp": 0, "End_Timestamp": 1_000_000})
        paths.append(str(path))
    out = tmp_path / "mix.md"
    prof.counter_summary(paths[0], paths[1], prof._layer_grids("qwen_128k_k32_w256"), "w", ["cmd"], None,
                         str(out))
    row = [l for l in out.read_text().splitlines() if l.startswith("| sel_attn")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1] == "1.000" and cells[3] == "10"          # ms, VALU per wave
    assert cells[8:11] == ["50%", "25%", "40%"]               # vector busy, matrix busy, waiting
    assert cells[12] == "16.38"                               # 1e9 matrix instructions x 16,384 flops


def test_committed_counter_profiles_match_their_current_sources():
    """A *_pmc.json records the hash of the source its kernel was built from;
    a profile of a kernel that has changed since is stale and must be retaken
    or removed (the benchmark also reports no traffic figure for it)."""
    import glob
    import hashlib
    import json
    import os

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for path in sorted(glob.glob(os.path.join(root, "profiles", "*_pmc.json"))):
        with open(path) as f:
            rec = json.load(f)
        src = os.path.join(root, rec["source"])
        assert os.path.exists(src), (path, rec["source"])
        with open(src, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()[:16]
        assert digest == rec["source_sha256_16"], f"{os.path.basename(path)} is stale: retake or remove it"
