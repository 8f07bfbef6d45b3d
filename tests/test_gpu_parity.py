"""GPU parity: the HIP path (called through the C ABI) against the CPU oracle.

Small cases run the oracle on every block; they span several GEMM and chain
tiles, ragged M / N / K tails, both block layouts, fp32 and bf16 hidden
states, ranks from 0 to 256, top_k from 1 to 16 and more than 64 blocks. The
full-size workloads are checked against the oracle on every block: all its
logits, every slot's token and candidates, its confidences and its cut.
"""
from __future__ import annotations

import sys
from dataclasses import replace

import numpy as np
import pytest

from oracle.check import check
from synthetic import CONFIGS, make_inputs, make_small, reduce_vocab
from synthetic.inputs import BONUS_ANCHOR

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dspark_block_drafter_amd as dsp
    dsp.load_library()
    return torch.device("cuda:0")


def _gpu(inp):
    from devutil import run_propose, to_host
    return to_host(run_propose(inp))


SMALL = {
    "tiny": lambda: make_inputs(CONFIGS["tiny"]),
    "ragged_conf": lambda: make_small(3, 5, 264, 1000, 24, top_k=3, conf=True, p_min=0.45, seed=1),
    "bonus_f32_v777": lambda: make_small(5, 7, 136, 777, 16, top_k=4, layout=BONUS_ANCHOR,
                                         hidden_f32=True, conf=True, p_min=0.5, conf_trend=True,
                                         seed=2),
    "B70_two_groups": lambda: make_small(70, 3, 64, 2100, 8, top_k=2, seed=3, w_std=0.3),
    "B40_k16_r128": lambda: make_small(40, 4, 520, 5000, 128, top_k=16, conf=True, p_min=0.3,
                                       seed=4),
    "r0_plain_argmax": lambda: make_small(4, 6, 96, 3000, 0, top_k=5, seed=5),
    "topk_equals_V": lambda: make_small(2, 3, 16, 8, 8, top_k=8, seed=6),
    "single_slot": lambda: make_small(1, 1, 32, 33, 8, top_k=1, seed=7),
    "mid_gemm_M33": lambda: make_small(11, 3, 1032, 4097, 32, top_k=2, seed=8),
    "rank256": lambda: make_small(6, 4, 128, 1536, 256, top_k=3, seed=9, w_std=0.2),
    # ranks above 128: the three-stage ring over two block groups (top-4 and
    # top-1), the same ring at top-1 with the rank padded from 200, and the
    # direct kernel (V % 4 != 0) with one and two block groups
    "B40_r256_top4": lambda: make_small(40, 3, 128, 4096, 256, top_k=4, w_std=0.2, seed=111),
    "B40_r256_top1": lambda: make_small(40, 3, 128, 4096, 256, top_k=1, w_std=0.2, seed=112),
    "r200_top1": lambda: make_small(6, 3, 128, 3000, 200, top_k=1, w_std=0.2, seed=113),
    "r256_V_odd": lambda: make_small(5, 3, 128, 3001, 256, top_k=2, w_std=0.2, seed=114),
    "B40_r192_V_odd": lambda: make_small(40, 3, 64, 2003, 192, top_k=3, w_std=0.2, seed=115),
    "dma_mid_M63": lambda: make_small(9, 7, 160, 3001, 16, top_k=2, conf=True, p_min=0.4, seed=18),
    # 32 < M <= 128 with H % 64 == 0 and too few 256-row tiles for the CUs:
    # the 128-row tiles with 64-value stage rows, ragged M and N
    "dma_mid_small_vocab": lambda: make_small(10, 6, 128, 5000, 16, top_k=2, seed=32),
    "dma_big_K32": lambda: make_small(20, 13, 32, 700, 8, top_k=3, seed=19),
    "dma_big_K96_bonus": lambda: make_small(23, 12, 96, 1000, 24, top_k=1, layout=BONUS_ANCHOR,
                                             conf=True, p_min=0.5, seed=20),
    # four-wave GEMM path (M > 128, K % 64 == 0): ragged M and N tiles,
    # several K steps; two K steps (loads past the end are clamped)
    "w4_ragged_K320": lambda: make_small(37, 8, 320, 3000, 16, top_k=2, conf=True, p_min=0.4, seed=21),
    "w4_two_ksteps": lambda: make_small(33, 9, 128, 1000, 8, top_k=1, layout=BONUS_ANCHOR, seed=22),
    # a tile count that is not a multiple of 8 (plain tile order, no XCD
    # grouping) and an odd number of K steps
    "w4_six_tiles_K192": lambda: make_small(40, 9, 192, 700, 8, top_k=2, seed=38),
    # several tiles per workgroup (V > 256 tiles): the two-stage ring of
    # top-k over two block groups (2-3 tiles each of 512 workgroups), the
    # four-stage ring with fewer tiles than stages (2-3 of 256) and with more
    # (4-5 of 256, two block groups, top-1)
    "two_stage_multi_tile": lambda: make_small(40, 4, 64, 70000, 64, top_k=4, seed=23),
    "four_stage_short": lambda: make_small(4, 5, 64, 70000, 64, top_k=1, conf=True, p_min=0.45,
                                           seed=24),
    "four_stage_two_groups": lambda: make_small(34, 3, 64, 70000, 32, top_k=1, seed=25),
    # long top-4 lists (six or more steps per wave or tile range): two block
    # groups (the second partly filled) at ranks 128 and 64, and one group on
    # the per-wave rings (seven 32-column steps per wave)
    "long_lists_two_groups": lambda: make_small(40, 3, 64, 98404, 128, top_k=4, seed=26),
    "long_lists_one_group": lambda: make_small(8, 3, 64, 229412, 128, top_k=4, conf=True,
                                               p_min=0.3, seed=27),
    "long_lists_r64": lambda: make_small(40, 3, 64, 110000, 64, top_k=4, seed=28),
    # per-wave rings staging 16 logits rows: two workgroups per CU (rank 64,
    # top-4, several steps per wave) and one per CU (rank 128, top-1)
    "rows16_two_per_cu": lambda: make_small(12, 3, 64, 229412, 64, top_k=4, conf=True, p_min=0.3,
                                            seed=29),
    "rows16_rank128_top1": lambda: make_small(16, 3, 64, 160000, 128, top_k=1, seed=30),
    "rows16_rank128_top4": lambda: make_small(12, 3, 64, 160000, 128, top_k=4, seed=33),
    # 8 staged rows, two workgroups per CU: rank 0 (eight-stage rings) and
    # rank 24 (six stages), several steps per wave
    "rows8_rank0_top4": lambda: make_small(4, 4, 64, 300000, 0, top_k=4, seed=34),
    "rows8_rank24_top3": lambda: make_small(3, 4, 64, 300000, 24, top_k=3, conf=True, p_min=0.4,
                                            seed=35),
    # more than 64 blocks over a long vocabulary: two block groups of 64 in the
    # grid, each with the full workgroup count (per-wave form at top-1, the
    # two-stage ring at top-4)
    "B96_two_groups_wave_top1": lambda: make_small(96, 3, 64, 100000, 64, top_k=1, seed=36),
    "B80_two_groups_pipe_top4": lambda: make_small(80, 3, 64, 100000, 128, top_k=4, conf=True,
                                                   p_min=0.3, seed=37),
    # fp32 hidden states with more than 32 rows: the register-staged GEMM with
    # 128-row tiles, K a multiple of 64 (whole K steps) and not (H = 200:
    # the last K step is partly past H)
    "f32_M45_K192": lambda: make_small(9, 5, 192, 3001, 16, top_k=2, hidden_f32=True, conf=True,
                                       p_min=0.4, seed=39),
    "f32_M45_K200": lambda: make_small(9, 5, 200, 2900, 16, top_k=3, hidden_f32=True, seed=40),
    "f32_M300_K200_bonus": lambda: make_small(50, 7, 200, 1500, 8, top_k=1, layout=BONUS_ANCHOR,
                                              hidden_f32=True, seed=47),
    "reduced_vocab": lambda: make_small(4, 7, 176, 4096, 64, top_k=4, layout=BONUS_ANCHOR,
                                        reachable=300, conf=True, p_min=0.5, conf_trend=True,
                                        seed=10),
    # 512 (block, slot) pairs or more: the one-wave-per-pair finalize
    "final_wave_k4_conf": lambda: make_small(64, 9, 64, 3000, 16, top_k=4, conf=True, p_min=0.4,
                                             seed=48),
    "final_wave_k1": lambda: make_small(130, 4, 64, 2000, 8, top_k=1, conf=True, p_min=0.3, seed=49),
    "final_wave_k16_bonus": lambda: make_small(70, 9, 64, 1500, 8, top_k=16, layout=BONUS_ANCHOR,
                                               seed=50),
    # an odd number of (block, slot) pairs: the last workgroup holds one pair
    "final_wave_odd_pairs": lambda: make_small(103, 5, 64, 2500, 16, top_k=4, conf=True, p_min=0.4,
                                               seed=101),
    # ten block groups (grid y of five pairs of groups, or ten groups), and a
    # block of 48 prediction slots
    "B300_ten_groups_top4": lambda: make_small(300, 3, 64, 20000, 64, top_k=4, conf=True, p_min=0.35,
                                               seed=61),
    "B300_ten_groups_top1": lambda: make_small(300, 3, 64, 20000, 32, top_k=1, seed=62),
    "L48_long_block": lambda: make_small(2, 48, 64, 9000, 16, top_k=2, conf=True, p_min=0.2, seed=63),
    # a vocabulary of a million odd columns (the direct form, ~7800 workgroups
    # and their partial lists), a thousand blocks, and a 1+1 bonus-anchor block
    # (one predicting slot)
    "V1M_direct_odd": lambda: make_small(2, 3, 64, 1000003, 16, top_k=2, seed=64),
    "B1000_short": lambda: make_small(1000, 2, 64, 5000, 16, top_k=3, conf=True, p_min=0.3, seed=65),
    "bonus_L2": lambda: make_small(3, 2, 64, 3000, 16, top_k=2, layout=BONUS_ANCHOR, seed=66),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_parity(dev, orc, name):
    inp = SMALL[name]()
    _say(f"[parity] {name}: {inp.cfg}")
    g = _gpu(inp)
    reps = check(orc, inp, g)
    ties = sum(r["near_tie"] for r in reps)
    err = max(r["max_logit_err"] for r in reps)
    _say(f"[parity] {name}: ok, max logit err {err:.3g}, near ties {ties}")
    if inp.reachable is not None:
        allowed = set(int(x) for x in inp.reachable)
        assert set(g["tokens"].ravel().tolist()) <= allowed
        assert set(g["candidates"].ravel().tolist()) <= allowed


@pytest.mark.parametrize("B", [36, 8])
def test_exact_ties_across_workgroups(dev, orc, B):
    """Columns repeat with period 8 (identical lm_head and markov_w2 rows), so
    every score is shared by V/8 columns spread over every workgroup. The
    answer is unique (larger score, then lower id) and both sides compute tied
    columns identically, so tokens and candidates must equal the oracle's
    exactly wherever the best two classes are apart by more than rounding.
    Two block groups run on the shared two-stage ring, one on per-wave rings."""
    inp = make_small(B, 3, 64, 98404, 128, top_k=4, seed=31)
    idx = np.arange(inp.cfg.V) % 8
    inp.lm_head[:] = inp.lm_head[idx]
    inp.markov_w2[:] = inp.markov_w2[idx]
    g = _gpu(inp)
    ref = orc.propose(inp, keep_logits=False)
    c = inp.cfg
    checked = 0
    for b in range(c.B):
        z = orc.block_logits(inp, b)
        prev = int(inp.anchors[b])
        for j in range(c.n_pred):
            cls = np.sort(np.unique(orc.step_scores(inp, z[j], prev)[:8]))[::-1]
            if cls[0] - cls[1] <= 1e-3:
                break   # a near tie: later slots may be conditioned on another token
            assert g["tokens"][b, j] == ref["tokens"][b, j], (b, j)
            assert np.array_equal(g["candidates"][b, j], ref["candidates"][b, j]), (b, j)
            checked += 1
            prev = int(ref["tokens"][b, j])
    _say(f"[ties] {checked} of {c.B * c.n_pred} slots compared exactly")
    assert checked >= c.B * c.n_pred // 2


def test_chain_alone_on_oracle_logits(dev, orc):
    """The chain kernel fed the oracle's own projections (rounded to fp32 on the
    host), so chain errors cannot hide behind GEMM errors."""
    import torch

    import dspark_block_drafter_amd as dsp
    from devutil import to_device
    inp = make_small(9, 6, 64, 3333, 64, top_k=4, conf=True, p_min=0.4, seed=11, w_std=0.3)
    z = np.concatenate([orc.block_logits(inp, b) for b in range(inp.cfg.B)]).astype(np.float32)
    d = to_device(inp)
    zt = torch.from_numpy(z).to(dev)
    res = dsp.chain(zt, d["markov_w1"], d["markov_w2"], d["anchors"], B=inp.cfg.B, L=inp.cfg.L,
                    layout=inp.cfg.layout, top_k=4, p_min=inp.cfg.p_min, hidden=d["hidden"],
                    conf_w=d["conf_w"])
    torch.cuda.synchronize()
    g = {k: (None if v is None else v.cpu().numpy()) for k, v in res.as_dict().items()}
    g["logits"] = None
    check(orc, inp, g)
    assert dsp.read_flags(res) == 0


BOUND_CASES = {
    "throughput_like_B64_k4": lambda: make_small(64, 4, 128, 40000, 128, top_k=4, conf=True,
                                                 p_min=0.3, w_std=0.05, seed=51),
    "tree_like_B8_k4": lambda: make_small(8, 5, 128, 60000, 128, top_k=4, w_std=0.05, seed=52),
    "k16_r64": lambda: make_small(12, 3, 64, 30000, 64, top_k=16, w_std=0.2, seed=53),
    "k3_strong_markov": lambda: make_small(40, 4, 64, 20000, 32, top_k=3, w_std=0.5, seed=54),
    "k2_rank256": lambda: make_small(6, 3, 128, 9000, 256, top_k=2, w_std=0.2, seed=55),
    "k4_bias_ragged": lambda: make_small(37, 5, 320, 5003, 16, top_k=4, reachable=900, seed=56),
    # top-1 (a running argmax: no list for the bound to filter), one block group
    "k1_B1_r64": lambda: make_small(1, 9, 256, 50000, 64, top_k=1, conf=True, w_std=0.05, seed=57),
    "k1_B4_bonus_reachable": lambda: make_small(4, 7, 128, 40000, 64, top_k=1, layout=BONUS_ANCHOR,
                                                reachable=5000, conf=True, p_min=0.5, seed=58),
    "k1_B32_rank0": lambda: make_small(32, 3, 64, 20000, 0, top_k=1, seed=60),
    "k1_B20_V_odd": lambda: make_small(20, 4, 64, 30011, 128, top_k=1, w_std=0.5, seed=59),
}



@pytest.mark.parametrize("name", sorted(BOUND_CASES))
def test_bound_changes_nothing(dev, orc, name):
    """dspark_propose filters its top-k inserts with a bound taken from the
    projection's row maxima; dspark_chain on the same projections runs
    without it. The bound only drops columns that cannot be among the top
    k, so every output must be identical, bit for bit, and the proposal
    must pass the oracle check."""
    import torch

    import dspark_block_drafter_amd as dsp
    from devutil import run_propose, to_device, to_host
    inp = BOUND_CASES[name]()
    c = inp.cfg
    d = to_device(inp)
    res = to_host(run_propose(inp, dev=d))
    logits = torch.from_numpy(res["logits"]).to(dev)
    plain = dsp.chain(logits, d["markov_w1"], d["markov_w2"], d["anchors"], B=c.B, L=c.L,
                      layout=c.layout, top_k=c.top_k, p_min=c.p_min, hidden=d["hidden"],
                      conf_w=d["conf_w"])
    torch.cuda.synchronize()
    assert dsp.read_flags(plain) == 0
    plain = to_host(plain)
    for k in ("tokens", "candidates", "cand_logits", "conf", "lengths"):
        assert np.array_equal(res[k], plain[k]), k
    check(orc, inp, res)


def test_logits_alone(dev, orc):
    import torch

    import dspark_block_drafter_amd as dsp
    from devutil import to_device
    inp = make_small(7, 5, 328, 2500, 8, seed=12, layout=BONUS_ANCHOR)
    inp = replace(inp, lm_head_bias=np.linspace(-2, 2, 2500).astype(np.float32))
    d = to_device(inp)
    out = dsp.logits(d["hidden"], d["lm_head"], layout=BONUS_ANCHOR, lm_head_bias=d["lm_head_bias"])
    torch.cuda.synchronize()
    g = out.cpu().numpy().astype(np.float64)
    for b in range(inp.cfg.B):
        z = orc.block_logits(inp, b)
        np.testing.assert_allclose(g[b * 4:(b + 1) * 4], z, atol=2e-2, rtol=0)


def test_bonus_slot_never_read(dev):
    inp = make_small(3, 7, 64, 1024, 16, top_k=3, layout=BONUS_ANCHOR, conf=True, p_min=0.5, seed=13)
    h = inp.hidden.copy()
    h[:, 0, :] = 0x7FC0  # NaN in every bonus slot
    a, b = _gpu(inp), _gpu(replace(inp, hidden=h))
    for k in ("logits", "tokens", "candidates", "cand_logits", "conf", "lengths"):
        assert np.array_equal(a[k], b[k]), k


def test_deterministic(dev):
    inp = make_small(33, 5, 256, 7000, 64, top_k=4, conf=True, p_min=0.3, seed=14)
    a, b = _gpu(inp), _gpu(inp)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_bad_anchor_raises_flag_without_fault(dev):
    import dspark_block_drafter_amd as dsp
    from devutil import run_propose
    inp = make_small(2, 3, 32, 200, 8, top_k=2, seed=15)
    bad = replace(inp, anchors=np.array([5, 200 + 17], np.int32))
    res = run_propose(bad)
    assert dsp.read_flags(res) & dsp.FLAG_BAD_ANCHOR
    res = run_propose(inp)
    assert dsp.read_flags(res) == 0


def test_workspace_reuse_across_shapes(dev, orc):
    """One Outputs/workspace reused by a second, smaller call of the same shape
    family: stale contents from the first call must not leak."""
    import dspark_block_drafter_amd as dsp
    from devutil import run_propose, to_host
    big = make_small(8, 4, 64, 2048, 16, top_k=4, seed=16)
    run_propose(big)
    small = make_small(8, 4, 64, 2048, 16, top_k=4, seed=17)
    out = dsp.Outputs(8, 4, 2048, 4, "anchor_first", "cuda:0")
    run_propose(big, out=out)
    g = to_host(run_propose(small, out=out))
    check(orc, small, g)


# ---- reduced draft vocabulary (d2t table) ------------------------------------

D2T_SMALL = {
    "d2t_k4_conf": lambda: make_small(5, 7, 136, 3000, 16, top_k=4, layout=BONUS_ANCHOR,
                                      reachable=300, conf=True, p_min=0.5, conf_trend=True, seed=41),
    "d2t_top1_r64": lambda: make_small(3, 9, 64, 5000, 64, top_k=1, reachable=1031, seed=42),
    "d2t_ragged_D": lambda: make_small(37, 6, 128, 2000, 8, top_k=2, reachable=333, seed=43),
    "d2t_topk_equals_D": lambda: make_small(2, 4, 32, 700, 8, top_k=5, reachable=5, seed=44),
    # fp32 hidden states (the register-staged projection over D rows), and
    # top-1 over two block groups
    "d2t_f32_hidden": lambda: make_small(9, 5, 96, 3000, 16, top_k=3, hidden_f32=True, reachable=512,
                                         conf=True, p_min=0.4, seed=116),
    "d2t_B40_top1": lambda: make_small(40, 4, 64, 3000, 16, top_k=1, reachable=700, seed=117),
}


def _same_outputs(a: dict, b: dict):
    for k in ("tokens", "candidates", "cand_logits", "conf", "lengths"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("name", sorted(D2T_SMALL))
def test_d2t_equals_expanded_form(dev, orc, name):
    """The d2t path (projection and chain over the D draft ids) against the
    expanded form through dspark_propose: bit for bit on every output, the
    draft projections equal to the expanded ones at the d2t columns; and the
    re-conditioning checker against the oracle."""
    from devutil import run_propose_d2t, scatter_logits, to_host
    inp = D2T_SMALL[name]()
    red = reduce_vocab(inp)
    _say(f"[d2t] {name}: {inp.cfg} D={red.D}")
    e = _gpu(inp)
    g = to_host(run_propose_d2t(red))
    _same_outputs(e, g)
    assert np.array_equal(e["logits"][:, red.d2t], g["logits"])
    g["logits"] = scatter_logits(g["logits"], red.d2t, inp.cfg.V)
    check(orc, inp, g)


def test_d2t_bad_entry_raises_flag_without_fault(dev):
    import dspark_block_drafter_amd as dsp
    from devutil import run_propose_d2t
    red = reduce_vocab(make_small(2, 4, 32, 500, 8, top_k=2, reachable=50, seed=45))
    bad = replace(red, d2t=np.full(red.D, 10_000_000, dtype=np.int64))
    res = run_propose_d2t(bad)
    assert dsp.read_flags(res) & dsp.FLAG_BAD_D2T
    res = run_propose_d2t(red)
    assert dsp.read_flags(res) == 0


def test_d2t_full_size_gemma(dev, orc):
    """The Gemma-4-26B-A4B workload in its reduced form (D = 32768 of
    V = 262144): every block equal to the expanded form, sampled blocks against
    the oracle."""
    from devutil import run_propose_d2t, scatter_logits, to_host
    inp = make_inputs(CONFIGS["gemma4_26b_a4b"])
    red = reduce_vocab(inp)
    e = _gpu(inp)
    g = to_host(run_propose_d2t(red))
    _say(f"[d2t] gemma: GPU done, D={red.D}")
    _same_outputs(e, g)
    assert np.array_equal(e["logits"][:, red.d2t], g["logits"])
    g["logits"] = scatter_logits(g["logits"], red.d2t, inp.cfg.V)
    check(orc, inp, g, blocks=[0, 3])


# ---- adaptive gate: per-block thresholds and candidate counts -------------------

ADAPTIVE = {
    # trend 0.9 -> 0.3 over the slots; thresholds spread over the blocks
    "adaptive_k4": lambda: make_small(6, 8, 96, 3000, 16, top_k=4, conf=True, conf_trend=True,
                                      seed=61),
    "adaptive_bonus_direct": lambda: make_small(5, 7, 64, 1001, 8, top_k=3, conf=True,
                                                conf_trend=True, layout=BONUS_ANCHOR, seed=62),
    "adaptive_B70": lambda: make_small(70, 5, 64, 2048, 16, top_k=2, conf=True, conf_trend=True,
                                       seed=63),
    "adaptive_B72_final_wave": lambda: make_small(72, 8, 64, 2048, 16, top_k=4, conf=True,
                                                  conf_trend=True, seed=64),
    "adaptive_odd_pairs_final_wave": lambda: make_small(75, 7, 64, 2048, 16, top_k=4, conf=True,
                                                        conf_trend=True, seed=102),
    # top-1 (the per-wave form) with one and two block groups, and a rank
    # above 128 (the three-stage ring) over two block groups
    "adaptive_top1": lambda: make_small(6, 8, 96, 3000, 16, top_k=1, conf=True, conf_trend=True,
                                        seed=118),
    "adaptive_B40_top1": lambda: make_small(40, 6, 64, 3000, 16, top_k=1, conf=True,
                                            conf_trend=True, seed=119),
    "adaptive_B36_r256": lambda: make_small(36, 5, 64, 2048, 256, top_k=3, conf=True,
                                            conf_trend=True, w_std=0.2, seed=120),
}


def _run_adaptive(inp, p_min_b, top_k_b):
    import torch

    import dspark_block_drafter_amd as dsp
    from devutil import to_device, to_host
    d = to_device(inp)
    c = inp.cfg
    res = dsp.propose_adaptive(d["hidden"], d["lm_head"], d["markov_w1"], d["markov_w2"],
                               d["anchors"], d["conf_w"], torch.from_numpy(p_min_b).to("cuda:0"),
                               layout=c.layout, top_k=c.top_k, lm_head_bias=d["lm_head_bias"],
                               block_top_k=None if top_k_b is None else
                               torch.from_numpy(top_k_b).to("cuda:0"))
    torch.cuda.synchronize()
    assert dsp.read_flags(res) == 0
    return to_host(res)


@pytest.mark.parametrize("name", sorted(ADAPTIVE))
@pytest.mark.parametrize("thresholds", ["spread", "cut_mid", "all_cut_early", "none_cut"])
def test_adaptive_against_full_step_and_oracle(dev, orc, name, thresholds):
    """On every slot a block keeps, the gated step equals the plain step bit
    for bit (tokens, candidates up to the block's count, values, conf); past
    the cut it reports -1 / -inf; the cuts equal the oracle's under each
    block's threshold (a confidence within 1e-3 of its threshold may go
    either way). The plain step itself is checked against the oracle."""
    inp = ADAPTIVE[name]()
    c = inp.cfg
    rng = np.random.default_rng(len(name))
    p_min_b = {"spread": rng.uniform(0.2, 0.95, c.B),
               "cut_mid": np.full(c.B, 0.6),
               "all_cut_early": np.full(c.B, 0.97),
               "none_cut": np.zeros(c.B)}[thresholds].astype(np.float32)
    top_k_b = rng.integers(1, c.top_k + 1, c.B).astype(np.int32)
    _say(f"[adaptive] {name} {thresholds}: {c}")
    g = _run_adaptive(inp, p_min_b, top_k_b)
    full = _gpu(inp)            # p_min 0: every slot drafted
    check(orc, inp, full)
    assert np.array_equal(g["conf"], full["conf"])
    assert np.array_equal(g["logits"], full["logits"])
    for b in range(c.B):
        n, kb = int(g["lengths"][b]), int(top_k_b[b])
        o = orc.propose_block_gated(inp, b, float(p_min_b[b]), kb, keep_logits=False)
        if n != o["length"]:
            lo = min(n, o["length"])
            assert abs(float(o["conf"][lo]) - float(p_min_b[b])) < 1e-3, (b, n, o["length"])
        assert np.array_equal(g["tokens"][b, :n], full["tokens"][b, :n])
        assert np.all(g["tokens"][b, n:] == -1)
        assert np.array_equal(g["candidates"][b, :n, :kb], full["candidates"][b, :n, :kb])
        assert np.array_equal(g["cand_logits"][b, :n, :kb], full["cand_logits"][b, :n, :kb])
        assert np.all(g["candidates"][b, n:] == -1) and np.all(g["candidates"][b, :, kb:] == -1)
        assert np.all(np.isneginf(g["cand_logits"][b, n:]))
    if thresholds in ("cut_mid", "all_cut_early"):
        assert g["lengths"].max() < c.n_pred     # the chain stopped early
    if thresholds == "none_cut":
        assert np.all(g["lengths"] == c.n_pred)


# ---- greedy verification of the lattice -----------------------------------------

def _verify_tables(B, n, k, vocab, seed, p_hit=0.8):
    """Seeded candidate tables and targets: a target equals the chain token
    with probability p_hit, else the runner-up or a random id."""
    rng = np.random.default_rng(seed)
    cand = rng.integers(0, vocab, size=(B, n, k)).astype(np.int32)
    lengths = rng.integers(-1, n + 2, size=B).astype(np.int32)
    u = rng.random((B, n))
    target = np.where(u < p_hit, cand[:, :, 0],
                      np.where(u < (1 + p_hit) / 2, cand[:, :, min(1, k - 1)],
                               rng.integers(0, vocab, size=(B, n)))).astype(np.int32)
    return cand, lengths, target


@pytest.mark.parametrize("shape", [(3, 5, 1), (64, 16, 4), (257, 7, 16), (100_003, 6, 2)],
                         ids=lambda s: "x".join(map(str, s)))
def test_verify_against_oracle(dev, orc, shape):
    import torch

    import dspark_block_drafter_amd as dsp
    B, n, k = shape
    cand, lengths, target = _verify_tables(B, n, k, vocab=50, seed=B + n + k)
    t = lambda a: torch.from_numpy(a).to(dev)
    for lattice in (False, True):
        acc, tot = dsp.verify(t(cand), t(lengths), t(target), lattice=lattice)
        torch.cuda.synchronize()
        want_acc, want_tot = orc.verify(cand, lengths, target, lattice=lattice)
        assert np.array_equal(acc.cpu().numpy(), want_acc)
        assert tuple(tot.cpu().numpy().tolist()) == want_tot


def test_verify_own_chain_accepts_whole_blocks(dev):
    """Verified against its own greedy chain, a proposal keeps every submitted
    slot."""
    import torch

    import dspark_block_drafter_amd as dsp
    inp = make_small(9, 6, 64, 3000, 16, top_k=3, conf=True, p_min=0.45, seed=46)
    res = _gpu(inp)
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    acc, tot = dsp.verify(dv(res["candidates"]), dv(res["lengths"]), dv(res["tokens"]))
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), res["lengths"])
    assert tot.cpu().numpy().tolist() == [int(res["lengths"].sum())] * 2


# ---- full-size workloads, every block ------------------------------------------

FULL = ["qwen3_8b", "gemma4_26b_a4b", "qwen38_27b_tree", "qwen38_27b_throughput"]


@pytest.mark.parametrize("name", FULL)
def test_full_size(dev, orc, name):
    import time
    inp = make_inputs(CONFIGS[name])
    _say(f"[full] {name}: generated inputs")
    g = _gpu(inp)
    _say(f"[full] {name}: GPU done, checking all {inp.cfg.B} blocks against the oracle")
    reps = []
    t0 = time.perf_counter()
    for b in range(inp.cfg.B):
        reps += check(orc, inp, g, blocks=[b])
        _say(f"[full] {name}: block {b} ok ({time.perf_counter() - t0:.0f} s)")
    _say(f"[full] {name}: max logit err {max(r['max_logit_err'] for r in reps):.3g}, "
         f"near ties {sum(r['near_tie'] for r in reps)}")
    c = inp.cfg
    # properties that hold for every block, checked on all of them
    assert g["tokens"].shape == (c.B, c.n_pred)
    assert np.all((g["tokens"] >= 0) & (g["tokens"] < c.V))
    assert np.array_equal(g["candidates"][:, :, 0], g["tokens"])
    assert np.all(np.diff(g["cand_logits"], axis=-1) <= 0)
    if inp.reachable is not None:
        assert np.all(np.isin(g["tokens"], inp.reachable))
        assert np.all(np.isin(g["candidates"], inp.reachable))
    if inp.conf_w is not None:
        first = np.array([next((j for j in range(c.n_pred) if g["conf"][b, j] < np.float32(c.p_min)),
                               c.n_pred) for b in range(c.B)])
        assert np.array_equal(first, g["lengths"])
