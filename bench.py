#!/usr/bin/env python3
"""Throughput of the DSpark proposal step on one MI355X.

One step = one dspark_propose call over one batch of seeded synthetic input:
lm_head projection, Markov chain over every slot, top-k candidates,
confidence truncation. The default workload is the throughput case at the
Qwen3.8-27B shape (B=64 blocks of L=16 anchor-first slots, H=5120,
V=248320, r=128, top_k=4, p_min=0.3); inputs are resident in HBM before the
timed region starts. Prints one JSON line.

Per-kernel figures come from the timed steps themselves: each step is a
dspark_propose_marked call, which records HIP events on the launch stream
between its launches (after the set-up kernel, after the lm_head projection,
after the last chain step), and the bench records one event before and one
after every call. An unmarked loop of dspark_propose calls is timed beside it
as a cross-check that the events cost nothing.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "drafted tokens/s (B×L Markov-chain proposals) at Qwen3.8-27B shape; % roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# HBM traffic of one lm_head GEMM launch at the throughput workload, from two
# rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script, each scaled by
# what the counter reads for a plain copy of known size (--calibrate-copy).
# The figures and commands are in profiles/lmhead_gemm_qwen38_27b_throughput_traffic.txt.
# They describe the kernel source whose SHA-256 is recorded here and are not
# reported for any other source or workload.
GEMM_TRAFFIC = {
    "workload": "qwen38_27b_throughput",
    "source_sha256": "6aaf425b8a82f80e734bb6da1d0d745c2844622dc6c9f2588090d0a7e190595b",
    "bytes": 5759954386,
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemm_source_sha256() -> str:
    import hashlib
    path = os.path.join(ROOT, "dspark_block_drafter_amd", "csrc", "lmhead_gemm.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: str):
    t = GEMM_TRAFFIC
    if t["bytes"] is None or workload != t["workload"] or gemm_source_sha256() != t["source_sha256"]:
        return None
    return t["bytes"]


def calibrate_copy(mib: int, reps: int) -> int:
    """A plain device-to-device copy of a known size, for scaling the HBM byte
    counters (read `mib` MiB, write `mib` MiB per launch)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4, "launches": reps}), flush=True)
    return 0


def reference(d: dict, cfg, reps: int) -> dict:
    """Ceilings from outside the library on the same shapes, for context, next
    to the library's own projection (dspark_logits) in the same process: the
    projection as one vendor GEMM (torch's F.linear over the prediction rows,
    hipBLASLt; bf16 in and out, so it writes half the bytes of the library's
    fp32 logits), and a plain device copy of 1 GiB (read and write), the rate
    a streaming kernel can expect from HBM."""
    import torch
    import torch.nn.functional as F
    i0 = 1 if cfg.layout == "bonus_anchor" else 0
    x = d["hidden"][:, i0:, :].reshape(-1, cfg.H).contiguous()
    w = d["lm_head"]
    stream = torch.cuda.current_stream()

    def timed(fn) -> float:
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3   # us per call

    import dspark_block_drafter_amd as dsp
    logits = torch.empty((x.shape[0], cfg.V), dtype=torch.float32, device="cuda:0")
    def ours():
        dsp.logits(d["hidden"], w, layout=cfg.layout, lm_head_bias=d["lm_head_bias"], out=logits,
                   stream=stream)

    # alternated, twice each, so that clock drift touches both alike
    o1, g1, o2, g2 = timed(ours), timed(lambda: F.linear(x, w)), timed(ours), timed(lambda: F.linear(x, w))
    ours_us, gemm_us = (o1 + o2) / 2, (g1 + g2) / 2
    flop = 2.0 * x.shape[0] * cfg.H * cfg.V
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    copy_us = timed(lambda: dst.copy_(src))
    return {"reference": {"workload": cfg.name, "reps": reps,
                          "dspark_logits_fp32": {"us": ours_us, "TFLOP/s": flop / ours_us / 1e6,
                                                 "runs_us": [o1, o2]},
                          "hipblaslt_linear_bf16": {"us": gemm_us, "TFLOP/s": flop / gemm_us / 1e6,
                                                    "runs_us": [g1, g2],
                                                    "M": x.shape[0], "K": cfg.H, "N": cfg.V},
                          "device_copy_1GiB": {"us": copy_us, "GB/s": 2.0 * src.numel() * 4 / copy_us / 1e3}}}


def graph_timing(d: dict, cfg, steps: int) -> dict:
    """dspark_propose_noalloc eagerly, and the same call captured once in a
    HIP graph and replayed (the launches of a step issued as one graph),
    alternated twice each in one process: the cost of the step's launches."""
    import torch
    import dspark_block_drafter_amd as dsp
    out = dsp.Outputs(cfg.B, cfg.L, cfg.V, cfg.top_k, cfg.layout, "cuda:0")

    def call():
        dsp.propose_noalloc(d["hidden"], d["lm_head"], d["markov_w1"], d["markov_w2"], d["anchors"],
                            layout=cfg.layout, top_k=cfg.top_k, p_min=cfg.p_min,
                            lm_head_bias=d["lm_head_bias"], conf_w=d["conf_w"], out=out)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(fn) -> float:
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3   # us per step

    e1_, g1, e2_, g2 = timed(call), timed(g.replay), timed(call), timed(g.replay)
    return {"graph": {"workload": cfg.name, "steps": steps,
                      "eager_noalloc_us": (e1_ + e2_) / 2, "graph_replay_us": (g1 + g2) / 2,
                      "runs_us": {"eager": [e1_, e2_], "replay": [g1, g2]}}}


def host_cpu() -> str:
    """The host's CPU model (lscpu), for the record of the CPU baseline."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
    except (OSError, subprocess.SubprocessError):
        return "unknown"
    for line in out.splitlines():
        if line.startswith("Model name:"):
            return line.split(":", 1)[1].strip()
    return "unknown"


def cpu_baseline(inp, blocks: int, single_blocks: int) -> dict:
    """The oracle as it stands (OpenMP over the vocabulary), on the host
    cores: `blocks` blocks on every OpenMP thread, then `single_blocks` on one."""
    import ctypes
    from oracle import Oracle
    orc = Oracle()
    gomp = ctypes.CDLL("libgomp.so.1")   # the OpenMP runtime the oracle is linked with
    cores = int(gomp.omp_get_max_threads())

    def run(nb: int):
        t0 = time.perf_counter()
        orc.propose(inp, blocks=list(range(nb)), keep_logits=False)
        return time.perf_counter() - t0

    dt = run(blocks)
    toks = blocks * inp.cfg.n_pred
    gomp.omp_set_num_threads(1)
    dt1 = run(single_blocks)
    gomp.omp_set_num_threads(cores)
    toks1 = single_blocks * inp.cfg.n_pred
    return {"value": toks / dt, "unit": "drafted tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{blocks} of {inp.cfg.B} blocks ({toks} drafted tokens) of the same "
                      f"workload, {dt:.1f} s wall on {cores} OpenMP threads",
            "single_thread": {"value": toks1 / dt1, "cores": 1,
                              "sample": f"{single_blocks} block ({toks1} drafted tokens), "
                                        f"{dt1:.1f} s wall on 1 thread"},
            "host": {"cpu": host_cpu(), "nproc": os.cpu_count()}}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen38_27b_throughput")
    ap.add_argument("--cpu-blocks", type=int, default=2)
    ap.add_argument("--cpu-single-blocks", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--adaptive", action="store_true",
                    help="run dspark_propose_adaptive (confidence gate before the chain, "
                         "the workload's p_min for every block); value counts submitted slots")
    ap.add_argument("--d2t", action="store_true",
                    help="run the workload's reduced-vocabulary form (dspark_propose_d2t)")
    ap.add_argument("--q4", action="store_true",
                    help="run the workload with its lm_head requantized to 4-bit GGUF blocks "
                         "(dspark_q4_pack once, then dspark_propose_q4 per step)")
    ap.add_argument("--reference", action="store_true",
                    help="time a vendor GEMM on the projection's shape and a plain device copy "
                         "(one JSON line; no proposal step)")
    ap.add_argument("--graph", action="store_true",
                    help="time dspark_propose_noalloc eagerly and as a replayed HIP graph "
                         "(one JSON line; no proposal record)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the proposal step is built and measured on a "
              "single MI355X; run it with --gpus 1", file=sys.stderr)
        return 2

    if args.calibrate_copy > 0:
        return calibrate_copy(args.calibrate_copy, max(args.steps, 1))

    import torch

    import dspark_block_drafter_amd as dsp
    from devutil import to_device
    from synthetic import CONFIGS, make_inputs

    cfg = CONFIGS[args.workload]
    t0 = time.perf_counter()
    inp = make_inputs(cfg)
    log(f"inputs for {cfg.name} generated in {time.perf_counter() - t0:.1f} s")
    stream = torch.cuda.current_stream()
    if sum([args.d2t, args.adaptive, args.q4]) > 1:
        print("--d2t, --adaptive and --q4 are separate forms; pick one", file=sys.stderr)
        return 2
    if args.q4:
        from devutil import to_device_q4
        from synthetic import quantize_q4
        if cfg.H % 32 != 0:
            print(f"--q4 needs H to be a multiple of 32; {cfg.name} has H={cfg.H}", file=sys.stderr)
            return 2
        t0 = time.perf_counter()
        inp = quantize_q4(inp, "round")
        log(f"lm_head requantized to 4-bit blocks in {time.perf_counter() - t0:.1f} s")
        d = to_device_q4(inp)
        del d["lm_head_blocks"]
        N = cfg.V
        out = dsp.OutputsQ4(cfg.B, cfg.L, cfg.H, cfg.V, cfg.top_k, cfg.layout, "cuda:0")
        q4_ws = torch.empty((dsp.q4_workspace_bytes(cfg.B, cfg.L, cfg.H, cfg.V, 1, cfg.layout),),
                            dtype=torch.uint8, device="cuda:0")

        def step():
            dsp.propose_q4(d["hidden"], d["lm_head_q4"], d["markov_w1"], d["markov_w2"],
                           d["anchors"], V=cfg.V, layout=cfg.layout, top_k=cfg.top_k,
                           p_min=cfg.p_min, lm_head_bias=d["lm_head_bias"], conf_w=d["conf_w"],
                           out=out, stream=stream)
    elif args.d2t:
        from devutil import to_device_reduced
        from synthetic import reduce_vocab
        if inp.reachable is None:
            print(f"--d2t needs a workload with a reduced vocabulary; {cfg.name} has none",
                  file=sys.stderr)
            return 2
        red = reduce_vocab(inp)
        d = to_device_reduced(red)
        N = red.D
        out = dsp.Outputs(cfg.B, cfg.L, N, cfg.top_k, cfg.layout, "cuda:0")

        def step():
            dsp.propose_d2t(d["hidden"], d["lm_head"], d["d2t"], d["markov_w1"], d["markov_w2"],
                            d["anchors"], vocab=cfg.V, layout=cfg.layout, top_k=cfg.top_k,
                            p_min=cfg.p_min, conf_w=d["conf_w"], out=out, stream=stream)
    elif args.adaptive:
        if inp.conf_w is None:
            print(f"--adaptive needs a confidence head; {cfg.name} has none", file=sys.stderr)
            return 2
        d = to_device(inp)
        N = cfg.V
        out = dsp.Outputs(cfg.B, cfg.L, cfg.V, cfg.top_k, cfg.layout, "cuda:0")
        p_min_b = torch.full((cfg.B,), float(cfg.p_min), dtype=torch.float32, device="cuda:0")

        def step():
            dsp.propose_adaptive(d["hidden"], d["lm_head"], d["markov_w1"], d["markov_w2"],
                                 d["anchors"], d["conf_w"], p_min_b, layout=cfg.layout,
                                 top_k=cfg.top_k, lm_head_bias=d["lm_head_bias"], out=out,
                                 stream=stream)
    else:
        d = to_device(inp)
        if args.reference:
            print(json.dumps(reference(d, cfg, max(args.steps, 1))), flush=True)
            return 0
        if args.graph:
            print(json.dumps(graph_timing(d, cfg, max(args.steps, 1))), flush=True)
            return 0
        N = cfg.V
        out = dsp.Outputs(cfg.B, cfg.L, cfg.V, cfg.top_k, cfg.layout, "cuda:0")

        def step():
            dsp.propose(d["hidden"], d["lm_head"], d["markov_w1"], d["markov_w2"], d["anchors"],
                        layout=cfg.layout, top_k=cfg.top_k, p_min=cfg.p_min,
                        lm_head_bias=d["lm_head_bias"], conf_w=d["conf_w"], out=out, stream=stream)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    def event():
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream)   # creates the HIP event before the timed region
        return ev

    plain = not (args.d2t or args.adaptive or args.q4)
    # Unmarked steps: the cross-check (and the timed region of the d2t,
    # adaptive and 4-bit forms, which have no marked entry point).
    ev0, ev1 = event(), event()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_unmarked = ev0.elapsed_time(ev1) / args.steps
    log(f"{args.steps} unmarked steps: {ms_unmarked:.3f} ms/step (events), "
        f"{1e3 * wall / args.steps:.3f} ms/step (wall)")

    phases = None
    if plain:
        # The timed region: marked steps. Events per step: before the call,
        # after the set-up kernel, after the projection, after the last chain
        # step, after the call.
        evs = [[event() for _ in range(5)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for e in evs:
            e[0].record(stream)
            dsp.propose(d["hidden"], d["lm_head"], d["markov_w1"], d["markov_w2"], d["anchors"],
                        layout=cfg.layout, top_k=cfg.top_k, p_min=cfg.p_min,
                        lm_head_bias=d["lm_head_bias"], conf_w=d["conf_w"], out=out,
                        stream=stream, marks=(e[1], e[2], e[3]))
            e[4].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms = evs[0][0].elapsed_time(evs[-1][4]) / args.steps
        avg = lambda a, b: sum(e[a].elapsed_time(e[b]) for e in evs) / args.steps
        phases = {"init": avg(0, 1), "gemm": avg(1, 2), "chain": avg(2, 3), "finalize": avg(3, 4)}
        gemm_ms, chain_ms = phases["gemm"], phases["chain"] + phases["finalize"]
        log(f"timed {args.steps} marked steps: {ms:.3f} ms/step (events), "
            f"{1e3 * wall / args.steps:.3f} ms/step (wall); set-up {phases['init'] * 1e3:.1f} us, "
            f"lm_head GEMM {gemm_ms * 1e3:.1f} us, chain steps {phases['chain'] * 1e3:.1f} us, "
            f"finalize {phases['finalize'] * 1e3:.1f} us")
    else:
        ms = ms_unmarked
        # the projection alone through dspark_logits / dspark_logits_q4 (the
        # chain's time is the step minus it)
        evs = [[event() for _ in range(2)] for _ in range(args.steps)]
        for e in evs:
            e[0].record(stream)
            if args.q4:
                dsp.logits_q4(d["hidden"], d["lm_head_q4"], V=cfg.V, layout=cfg.layout,
                              lm_head_bias=d["lm_head_bias"], out=out.logits, workspace=q4_ws,
                              stream=stream)
            else:
                dsp.logits(d["hidden"], d["lm_head"], layout=cfg.layout,
                           lm_head_bias=None if args.d2t else d["lm_head_bias"], out=out.logits,
                           stream=stream)
            e[1].record(stream)
        torch.cuda.synchronize()
        gemm_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
        chain_ms = ms - gemm_ms
        log(f"lm_head GEMM alone {gemm_ms * 1e3:.1f} us, rest of the step {chain_ms * 1e3:.1f} us")
    assert dsp.read_flags(out) == 0
    submitted = int(out.lengths.sum().item())
    if args.adaptive:
        log(f"adaptive gate: {submitted} of {cfg.drafted_tokens} slots submitted per step")

    # Greedy lattice verification of the step's proposal (dspark_verify), with
    # the target taken equal to the drafted chain: every submitted slot is
    # walked, the longest walk the data allows.
    acc_buf = torch.empty((cfg.B,), dtype=torch.int32, device="cuda:0")
    tot_buf = torch.empty((2,), dtype=torch.int32, device="cuda:0")
    target = out.tokens.clone()
    v0, v1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    v0.record(stream)
    for _ in range(args.steps):
        dsp.verify(out.candidates, out.lengths, target, lattice=True, accepted=acc_buf,
                   totals=tot_buf, stream=stream)
    v1.record(stream)
    torch.cuda.synchronize()
    verify_us = v0.elapsed_time(v1) / args.steps * 1e3
    walked = tot_buf.cpu().tolist()
    log(f"lattice verify {verify_us:.1f} us per call ({walked[0]} of {walked[1]} submitted slots walked)")

    M, H, V, r, B, n = cfg.B * cfg.n_pred, cfg.H, N, cfg.r, cfg.B, cfg.n_pred
    flops = 2.0 * M * H * V
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    # algorithmic bytes: the head (bf16, or the packed 4-bit head: 4.5 bits per
    # weight), the hidden rows once, the fp32 logits once
    head_bytes = dsp.q4_packed_bytes(V, H) if args.q4 else V * H * 2
    gemm_bytes = head_bytes + M * H * 2 + M * V * 4
    # the projection is matrix-bound above the ridge point (peak FLOP/s over
    # peak bytes/s, 312 FLOP/B), HBM-bound below it
    if flops / gemm_bytes > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        gemm_roof = {"bound": "mfma", "achieved": gemm_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": gemm_tflops / PEAK_BF16_TFLOPS}
    else:
        gemm_gbs = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        gemm_roof = {"bound": "hbm", "achieved": gemm_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gemm_gbs / PEAK_HBM_GBS}
    # chain: per slot the B logits rows and markov_w2 are streamed, plus B rank-r gathers;
    # the adaptive gate runs the chain only up to the longest surviving block, and a
    # slot streams the logits rows (and gathers) of the blocks still drafting there
    if args.adaptive:
        lens = out.lengths.cpu().tolist()
        slots_run = max(lens)
        live = [sum(1 for x in lens if x > jj) for jj in range(slots_run)]
        chain_bytes = sum(lv * V * 4 + V * r * 2 + lv * r * 2 for lv in live)
    else:
        slots_run = n
        chain_bytes = slots_run * (B * V * 4 + V * r * 2 + B * r * 2)
    chain_gbs = chain_bytes / (chain_ms * 1e-3) / 1e9

    res = {
        "metric": METRIC,
        "value": (submitted if args.adaptive else cfg.drafted_tokens) / (ms * 1e-3),
        "unit": "drafted tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "L": cfg.L, "H": H, "V": cfg.V, "r": r,
                   "top_k": cfg.top_k, "p_min": cfg.p_min, "layout": cfg.layout,
                   "drafted_tokens_per_step": cfg.drafted_tokens,
                   **({"d2t_draft_vocab": N} if args.d2t else {}),
                   **({"lm_head": "4-bit GGUF blocks (binary16 scale per 32), packed",
                       "head_bytes": head_bytes} if args.q4 else {}),
                   **({"adaptive": True, "counted": "submitted slots (sum of lengths)",
                       "submitted_per_step": submitted} if args.adaptive else {})},
        "roofline": {**gemm_roof,
                     "traffic": None if (args.d2t or args.q4) else measured_traffic(cfg.name),
                     "kernel": "q4_prep + lmhead_q4" if args.q4 else "lmhead_gemm",
                     "us": gemm_ms * 1e3,
                     "timed": "events around the projection inside the timed steps" if plain
                              else ("dspark_logits_q4 alone" if args.q4 else "dspark_logits alone")},
        "roofline_chain": {"bound": "hbm", "achieved": chain_gbs, "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": chain_gbs / PEAK_HBM_GBS,
                           "bytes": chain_bytes, "kernels": "chain_step x n_pred + finalize",
                           "us": chain_ms * 1e3,
                           **({"us_steps": phases["chain"] * 1e3,
                               "us_finalize": phases["finalize"] * 1e3,
                               "frac_steps": chain_bytes / (phases["chain"] * 1e-3) / 1e9 / PEAK_HBM_GBS}
                              if plain else {})},
        **({"phases_us": {k: v * 1e3 for k, v in phases.items()}} if plain else {}),
        "unmarked_ms_per_step": ms_unmarked,
        "wall_ms_per_step": 1e3 * wall / args.steps,
        # call time of dspark_verify through the binding, host enqueue included
        # (its two kernels take a few microseconds: see the kernel statistics)
        "verify": {"kernels": "verify_walk + verify_totals", "call_us": verify_us, "lattice": True,
                   "submitted_slots": walked[1]},
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_blocks} blocks")
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_blocks, args.cpu_single_blocks)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
