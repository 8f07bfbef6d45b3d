"""Moves synthetic inputs to the GPU and GPU outputs back (tests only)."""
from __future__ import annotations

import numpy as np


def to_device(inp, device="cuda:0") -> dict:
    import torch

    def bf16(a):
        if a is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    def f32(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)

    hidden = f32(inp.hidden) if inp.hidden_f32 else bf16(inp.hidden)
    return {
        "hidden": hidden,
        "lm_head": bf16(inp.lm_head),
        "lm_head_bias": f32(inp.lm_head_bias),
        "markov_w1": bf16(inp.markov_w1),
        "markov_w2": bf16(inp.markov_w2),
        "conf_w": bf16(inp.conf_w),
        "anchors": torch.from_numpy(np.ascontiguousarray(inp.anchors)).to(device),
    }


def run_propose(inp, dev=None, out=None):
    import dspark_block_drafter_amd as dsp
    import torch
    d = dev if dev is not None else to_device(inp)
    c = inp.cfg
    res = dsp.propose(d["hidden"], d["lm_head"], d["markov_w1"], d["markov_w2"], d["anchors"],
                      layout=c.layout, top_k=c.top_k, p_min=c.p_min,
                      lm_head_bias=d["lm_head_bias"], conf_w=d["conf_w"], out=out)
    torch.cuda.synchronize()
    return res


def to_host(res) -> dict:
    out = {}
    for k, v in res.as_dict().items():
        out[k] = None if v is None else v.cpu().numpy()
    return out
