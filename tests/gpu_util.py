"""Helpers shared by the GPU tests: upload seeded inputs, run the C-ABI path."""
import numpy as np
import torch

from sparse_attention_long_nsa_amd import binding


def dev_dtype(shape):
    return torch.bfloat16 if shape.dtype == "bf16" else torch.float32


def upload(inp: dict, device="cuda:0") -> dict:
    dt = dev_dtype(inp["shape"])
    d = {}
    for key in ("q", "k", "v", "w_k", "w_v"):
        # bf16 inputs hold bf16-exact float32 values, so the cast is exact
        d[key] = torch.from_numpy(np.ascontiguousarray(inp[key])).to(device).to(dt).contiguous()
    d["gates"] = torch.from_numpy(np.ascontiguousarray(inp["gates"])).to(device)
    return d


def run_prefill(inp: dict, top_k=None, window=None, dev=None, kcmp=False, lse=False) -> dict:
    s = inp["shape"]
    if dev is None:
        dev = upload(inp)
    r = binding.prefill(dev["q"], dev["k"], dev["v"], inp["is_vision"], dev["w_k"], dev["w_v"],
                        dev["gates"], s.top_k if top_k is None else top_k,
                        s.window if window is None else window, block=s.block,
                        want_kcmp=kcmp, want_sel=True, want_lse=lse)
    torch.cuda.synchronize()
    out = {"out": r["out"].cpu().numpy(), "sel": r["sel_idx"].cpu().numpy()}
    if kcmp:
        out["kcmp"] = r["k_cmp"].cpu().numpy()
        out["vcmp"] = r["v_cmp"].cpu().numpy()
    if lse:
        out["lse"] = r["lse"].cpu().numpy()
    return out
