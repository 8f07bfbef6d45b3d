"""GPU parity of the 4-bit lm_head path (dspark_q4_pack, dspark_logits_q4,
dspark_propose_q4, called through the C ABI) against the CPU oracle's q4
projection and proposal.

The packed layout is compared byte for byte with a numpy statement of it. The
logits are compared with the oracle's exact-weight projection: the kernel
sums x * (128 + q) in the MFMA (every product exact), removes 136 * sum(x)
per block with an fp32 product, and scales each block by d in fp32, so its
error is at most about gamma_33 * sum_g |d_g| * (272 * sum|x_g| + ...) plus
the fp32 accumulation over blocks; at H = 5120 with the synthetic
distributions that is below 1e-2, and typical errors are ~1e-5 (tolerance
2e-2, the same as the bf16 path's). Proposals go through the re-conditioning
checker on every block.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle.check import TOL_LOGITS, check
from synthetic import CONFIGS, make_inputs, make_small, quantize_q4
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


def _np_pack(q4: np.ndarray, V: int, H: int) -> np.ndarray:
    """The packed layout, stated with numpy: tiles of 16 rows, quads of 4
    blocks; code record (t, u) = [kq][c][gg][4 code bytes 4kq..4kq+3 of block
    4u+gg of row 16t+c]; all code records, then scale records (t, u) =
    [c][gg][binary16]; padding rows / blocks hold code bytes 0x88, scale 0."""
    G, GQ, T16 = H // 32, (H // 32 + 3) // 4, (V + 15) // 16
    blk = q4.reshape(V, G, 18)
    codes = np.full((T16 * 16, GQ * 4, 16), 0x88, np.uint8)
    codes[:V, :G] = blk[:, :, 2:]
    scales = np.zeros((T16 * 16, GQ * 4, 2), np.uint8)
    scales[:V, :G] = blk[:, :, :2]
    rec = codes.reshape(T16, 16, GQ, 4, 4, 4).transpose(0, 2, 4, 1, 3, 5)   # t, u, kq, c, gg, byte
    srec = scales.reshape(T16, 16, GQ, 4, 2).transpose(0, 2, 1, 3, 4)       # t, u, c, gg, byte
    return np.concatenate([rec.ravel(), srec.ravel()])


@pytest.mark.parametrize("V,H", [(37, 96), (16, 128), (300, 64), (1000, 2816), (5003, 4096)])
def test_pack_layout(dev, V, H):
    import torch
    import dspark_block_drafter_amd as dsp
    q = quantize_q4(make_small(1, 2, H, V, 0, seed=71), "random")
    packed = dsp.q4_pack(torch.from_numpy(q.lm_head_q4).to(dev), V, H)
    torch.cuda.synchronize()
    got = packed.cpu().numpy()
    assert got.size == dsp.q4_packed_bytes(V, H)
    assert np.array_equal(got, _np_pack(q.lm_head_q4, V, H))


# (inputs, quantization mode); M = B * n_pred spans the 16-, 32- and 64-row
# projections, with ragged V (not a multiple of 16) and H (not of 128)
LOGITS = {
    "M8_rand_f32": (lambda: make_small(2, 4, 96, 1003, 8, hidden_f32=True, seed=72), "random"),
    "M16_round": (lambda: make_small(1, 16, 256, 2048, 8, seed=73), "round"),
    "M24_bonus_bias": (lambda: make_small(4, 7, 160, 3001, 8, layout=BONUS_ANCHOR, reachable=700,
                                          seed=74), "round"),
    "M32_rand": (lambda: make_small(2, 16, 384, 1500, 8, seed=75), "random"),
    "M45_f32_rand": (lambda: make_small(9, 5, 224, 999, 8, hidden_f32=True, seed=76), "random"),
    "M130_round": (lambda: make_small(10, 13, 512, 2500, 8, seed=77), "round"),
    "M300_bonus_rand": (lambda: make_small(50, 7, 128, 777, 8, layout=BONUS_ANCHOR, seed=78),
                        "random"),
}


@pytest.mark.parametrize("name", sorted(LOGITS))
def test_logits_q4(dev, orc, name):
    import torch
    import dspark_block_drafter_amd as dsp
    from devutil import to_device_q4
    make, mode = LOGITS[name]
    q = quantize_q4(make(), mode)
    c = q.cfg
    d = to_device_q4(q)
    z = dsp.logits_q4(d["hidden"], d["lm_head_q4"], V=c.V, layout=c.layout,
                      lm_head_bias=d["lm_head_bias"])
    torch.cuda.synchronize()
    g = z.cpu().numpy().reshape(c.B, c.n_pred, c.V).astype(np.float64)
    worst = 0.0
    for b in range(c.B):
        err = np.abs(g[b] - orc.block_logits_q4(q, b))
        worst = max(worst, float(err.max()))
    _say(f"[q4 logits] {name}: max err {worst:.3g}")
    assert worst <= TOL_LOGITS


PROPOSE = {
    "tiny_q4": (lambda: make_inputs(CONFIGS["tiny"]), "round"),
    "B3_k3_conf": (lambda: make_small(3, 5, 264 - 8, 1000, 24, top_k=3, conf=True, p_min=0.45,
                                      seed=79), "round"),
    "B8_k4_rand": (lambda: make_small(8, 8, 192, 4000, 16, top_k=4, seed=80), "random"),
    "B4_bonus_reach": (lambda: make_small(4, 7, 288, 3000, 8, top_k=2, layout=BONUS_ANCHOR,
                                          reachable=500, conf=True, p_min=0.5, conf_trend=True,
                                          seed=81), "round"),
    "B40_k16_f32": (lambda: make_small(40, 3, 128, 1111, 32, top_k=16, hidden_f32=True, seed=82),
                    "random"),
    # top-1 over two block groups; a rank above 128 (the three-stage ring)
    "B40_top1_conf": (lambda: make_small(40, 4, 128, 3000, 16, top_k=1, conf=True, p_min=0.4,
                                         seed=121), "random"),
    "B6_r256": (lambda: make_small(6, 3, 128, 2048, 256, top_k=3, w_std=0.2, seed=122), "round"),
}


def _check_q4(orc, q, g, blocks=None):
    blocks = range(q.cfg.B) if blocks is None else blocks
    reps = []
    for b in blocks:
        reps += check(orc, q, g, blocks=[b])
    return reps


@pytest.mark.parametrize("name", sorted(PROPOSE))
def test_propose_q4(dev, orc, name):
    from devutil import run_propose_q4, to_host
    make, mode = PROPOSE[name]
    q = quantize_q4(make(), mode)
    g = to_host(run_propose_q4(q))
    reps = _check_q4(orc, q, g)
    _say(f"[q4 propose] {name}: max logit err {max(r['max_logit_err'] for r in reps):.3g}, "
         f"near ties {sum(r['near_tie'] for r in reps)}")


BOUNDED = {
    # The 4-bit call takes the bound where the chain prunes slabs with it (one
    # block group, V % 4 == 0, rank up to 128): pruned_*, lists16_*. Elsewhere
    # it runs unbounded: direct (V % 4 != 0) and the two-per-CU ring (two
    # groups). Every case must equal the unbounded chain bit for bit.
    "direct_V2222": lambda: make_small(6, 9, 320, 2222, 16, top_k=4, conf=True, p_min=0.4, seed=83),
    "pruned_B8": lambda: make_small(8, 6, 256, 40000, 64, top_k=4, seed=85),
    "pruned_conf_B16": lambda: make_small(16, 5, 160, 24000, 48, top_k=8, conf=True, p_min=0.35,
                                          seed=88),
    "two_groups_B40": lambda: make_small(40, 4, 128, 30000, 128, top_k=4, conf=True, p_min=0.3,
                                         seed=86),
    "lists16_B12": lambda: make_small(12, 5, 96, 20000, 32, top_k=16, seed=87),
}


@pytest.mark.parametrize("name", sorted(BOUNDED))
def test_propose_q4_equals_chain_on_q4_logits(dev, orc, name):
    """The proposal (with the top-k bound from the 4-bit projection's slab
    maxima where the chain prunes) is the unbounded chain of the library run
    on the q4 projections, bit for bit; and it passes the oracle's checker."""
    import torch
    import dspark_block_drafter_amd as dsp
    from devutil import run_propose_q4, to_device_q4, to_host
    q = quantize_q4(BOUNDED[name](), "round")
    c = q.cfg
    d = to_device_q4(q)
    a = to_host(run_propose_q4(q, dev=d))
    z = dsp.logits_q4(d["hidden"], d["lm_head_q4"], V=c.V, layout=c.layout)
    b = dsp.chain(z, d["markov_w1"], d["markov_w2"], d["anchors"], B=c.B, L=c.L, layout=c.layout,
                  top_k=c.top_k, p_min=c.p_min, hidden=d["hidden"], conf_w=d["conf_w"])
    torch.cuda.synchronize()
    b = to_host(b)
    assert np.array_equal(a["logits"], z.cpu().numpy())
    for k in ("tokens", "candidates", "cand_logits", "conf", "lengths"):
        assert np.array_equal(a[k], b[k]), k
    _check_q4(orc, q, a)


FULL = ["qwen3_8b", "gemma4_26b_a4b", "qwen38_27b_tree", "qwen38_27b_throughput"]


@pytest.mark.parametrize("name", FULL)
def test_propose_q4_full_size(dev, orc, name):
    import time
    from devutil import run_propose_q4, to_host
    inp = make_inputs(CONFIGS[name])
    q = quantize_q4(inp, "round")
    _say(f"[q4 full] {name}: quantized")
    g = to_host(run_propose_q4(q))
    c = q.cfg
    # every block of the three small workloads; every 8th of the 64-block one
    blocks = list(range(c.B)) if c.B <= 8 else list(range(0, c.B, 8))
    t0 = time.perf_counter()
    reps = []
    for b in blocks:
        reps += _check_q4(orc, q, g, [b])
        _say(f"[q4 full] {name}: block {b} ok ({time.perf_counter() - t0:.0f} s)")
    _say(f"[q4 full] {name}: max logit err {max(r['max_logit_err'] for r in reps):.3g}, "
         f"near ties {sum(r['near_tie'] for r in reps)}")
    assert np.all((g["tokens"] >= 0) & (g["tokens"] < c.V))
    assert np.array_equal(g["candidates"][:, :, 0], g["tokens"])
    if q.reachable is not None:
        assert np.all(np.isin(g["candidates"], q.reachable))


def test_q4_flags_in_the_workspace(dev):
    """The chain's flags word sits at offset 0 of the 4-bit call's workspace:
    clear after a valid call, DSPARK_FLAG_BAD_ANCHOR after an anchor outside
    [0, V) (which the kernels replace by 0)."""
    import dspark_block_drafter_amd as dsp
    from devutil import run_propose_q4, to_device_q4
    q = quantize_q4(make_small(3, 4, 64, 700, 8, top_k=2, seed=84), "random")
    d = to_device_q4(q)
    out = run_propose_q4(q, dev=d)
    assert dsp.read_flags(out) == 0
    d["anchors"][1] = 100000
    out = run_propose_q4(q, dev=d, out=out)
    assert dsp.read_flags(out) & dsp.FLAG_BAD_ANCHOR
