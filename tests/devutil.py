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
        "lm_head": bf16(getattr(inp, "lm_head", None)),
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


def to_device_reduced(red, device="cuda:0") -> dict:
    """Device tensors of a reduced-vocabulary input (synthetic.ReducedInputs)."""
    import torch
    def bf16(a):
        if a is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    hidden = (torch.from_numpy(np.ascontiguousarray(red.hidden)).to(device) if red.hidden_f32
              else bf16(red.hidden))
    return {
        "hidden": hidden,
        "lm_head": bf16(red.lm_head),
        "d2t": torch.from_numpy(np.ascontiguousarray(red.d2t)).to(device),
        "markov_w1": bf16(red.markov_w1),
        "markov_w2": bf16(red.markov_w2),
        "conf_w": bf16(red.conf_w),
        "anchors": torch.from_numpy(np.ascontiguousarray(red.anchors)).to(device),
    }


def run_propose_d2t(red, dev=None, out=None):
    import dspark_block_drafter_amd as dsp
    import torch
    d = dev if dev is not None else to_device_reduced(red)
    c = red.cfg
    res = dsp.propose_d2t(d["hidden"], d["lm_head"], d["d2t"], d["markov_w1"], d["markov_w2"],
                          d["anchors"], vocab=c.V, layout=c.layout, top_k=c.top_k, p_min=c.p_min,
                          conf_w=d["conf_w"], out=out)
    torch.cuda.synchronize()
    return res


def scatter_logits(logits_d: np.ndarray, d2t: np.ndarray, V: int) -> np.ndarray:
    """Draft-column projections placed at their target columns; every other
    column holds -1e9, the value the expanded form's bias gives it."""
    full = np.full((logits_d.shape[0], V), np.float32(-1e9), dtype=np.float32)
    full[:, d2t] = logits_d
    return full


def to_device_q4(qinp, device="cuda:0") -> dict:
    """Device tensors of a 4-bit-head input (synthetic.Q4Inputs); the head is
    uploaded as its GGUF blocks and packed on the device."""
    import torch
    import dspark_block_drafter_amd as dsp
    d = to_device(qinp, device)
    c = qinp.cfg
    blocks = torch.from_numpy(np.ascontiguousarray(qinp.lm_head_q4)).to(device)
    d["lm_head_blocks"] = blocks
    d["lm_head_q4"] = dsp.q4_pack(blocks, c.V, c.H)
    return d


def run_propose_q4(qinp, dev=None, out=None):
    import dspark_block_drafter_amd as dsp
    import torch
    d = dev if dev is not None else to_device_q4(qinp)
    c = qinp.cfg
    res = dsp.propose_q4(d["hidden"], d["lm_head_q4"], d["markov_w1"], d["markov_w2"], d["anchors"],
                         V=c.V, layout=c.layout, top_k=c.top_k, p_min=c.p_min,
                         lm_head_bias=d["lm_head_bias"], conf_w=d["conf_w"], out=out)
    torch.cuda.synchronize()
    return res
