"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with a closed form, a library routine (numpy argmax,
lexsort, fp64 matmul), a brute force over every previous token at tiny
vocabulary, an invariant of the method, or the hand-worked example in
``golden/hand_chain_v4.txt``. ``test_oracle_pins.py`` runs them against the
oracle; ``test_oracle_mutants.py`` runs them against copies of the oracle
with planted mistakes and requires each mistake to be caught.
"""
from __future__ import annotations

import math
import os
from dataclasses import replace

import numpy as np

from synthetic import (Q4Inputs, ReducedInputs, bf16_bits_to_f32, f32_to_bf16_bits, make_small,
                       q4_blocks, quantize_q4, reduce_vocab)
from synthetic.inputs import BONUS_ANCHOR, Config, Inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bf(x) -> np.ndarray:
    """Exact bf16 bits of values that are representable in bf16."""
    a = np.asarray(x, dtype=np.float32)
    b = f32_to_bf16_bits(a)
    assert np.array_equal(bf16_bits_to_f32(b), a), "value not exact in bf16"
    return b


def _np_logits(inp: Inputs) -> np.ndarray:
    """[B, n_pred, V] projections in fp64 via numpy matmul (independent of the oracle)."""
    c = inp.cfg
    if inp.hidden_f32:
        x = bf16_bits_to_f32(f32_to_bf16_bits(inp.hidden)).astype(np.float64)
    else:
        x = bf16_bits_to_f32(inp.hidden).astype(np.float64)
    x = x[:, c.i_first_pred:, :]
    w = bf16_bits_to_f32(inp.lm_head).astype(np.float64)
    z = x @ w.T
    if inp.lm_head_bias is not None:
        z = z + inp.lm_head_bias.astype(np.float64)
    return z


def _np_markov_table(inp: Inputs) -> np.ndarray:
    """T[p, v] = markov_w1[p] . markov_w2[v] for every previous token p."""
    c = inp.cfg
    if c.r == 0:
        return np.zeros((c.V, c.V))
    w1 = bf16_bits_to_f32(inp.markov_w1).astype(np.float64)
    w2 = bf16_bits_to_f32(inp.markov_w2).astype(np.float64)
    return w1 @ w2.T


def _np_topk(zp: np.ndarray, k: int):
    order = np.lexsort((np.arange(zp.size), -zp.astype(np.float64)))
    return order[:k], zp[order[:k]]


def _custom(B, L, H, V, r, hidden, lm_head, w1, w2, anchors, top_k=1, conf_w=None, p_min=0.0,
            bias=None, layout="anchor_first") -> Inputs:
    cfg = Config("custom", B=B, L=L, H=H, V=V, r=r, top_k=top_k, layout=layout,
                 conf=conf_w is not None, p_min=p_min)
    return Inputs(cfg=cfg, hidden=np.ascontiguousarray(hidden), lm_head=np.ascontiguousarray(lm_head),
                  lm_head_bias=bias, markov_w1=w1, markov_w2=w2, conf_w=conf_w,
                  anchors=np.asarray(anchors, dtype=np.int32))


# --------------------------------------------------------------------------
# number format
# --------------------------------------------------------------------------

def pin_bf16_round_known_values(orc):
    one = 1.0
    cases = [
        (one, 0x3F80),
        (one + 2.0 ** -8, 0x3F80),             # halfway, even neighbour is 0x3F80
        (one + 3 * 2.0 ** -8, 0x3F82),         # halfway, even neighbour is 0x3F82
        (one + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # just above halfway
        (one + 2.0 ** -8 - 2.0 ** -20, 0x3F80),  # just below halfway
        (-2.5, 0xC020),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (3.4028234663852886e38, 0x7F80),       # FLT_MAX is past the last bf16 halfway point
        (3.3895313892515355e38, 0x7F7F),       # largest finite bf16
        (2.0 ** -149, 0x0000),                 # smallest float subnormal rounds to zero
        (float("inf"), 0x7F80),
        (float("-inf"), 0xFF80),
    ]
    for x, want in cases:
        got = orc.bf16_round(x)
        assert got == want, f"bf16_round({x!r}) = {got:#06x}, want {want:#06x}"
    # agrees with the bit-trick rounding of the input generator on random data
    rng = np.random.default_rng(123)
    xs = np.concatenate([rng.standard_normal(2000).astype(np.float32),
                         (rng.standard_normal(2000) * 1e-38).astype(np.float32),
                         (1 + rng.integers(0, 512, 2000) * 2.0 ** -9).astype(np.float32)])
    want = f32_to_bf16_bits(xs)
    got = np.array([orc.bf16_round(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, want)


def pin_bf16_value(orc):
    for bits, want in {0x3F80: 1.0, 0xC020: -2.5, 0x0001: 2.0 ** -133, 0x7F7F: 3.3895313892515355e38,
                       0x4049: 3.140625}.items():
        assert orc.bf16_value(bits) == want


# --------------------------------------------------------------------------
# projection through lm_head
# --------------------------------------------------------------------------

def pin_logits_one_hot_closed_form(orc):
    """lm_head[v] = s_v * e_{(3v+1) mod H}: z_j[v] = s_v * x_j[(3v+1) mod H] + bias[v] exactly."""
    B, L, H, V = 2, 3, 16, 40
    rng = np.random.default_rng(7)
    hidden = f32_to_bf16_bits(rng.standard_normal((B, L, H)).astype(np.float32))
    s = np.array([1.0, -2.0, 0.5, 4.0])[np.arange(V) % 4]
    lm = np.zeros((V, H), dtype=np.float32)
    col = (3 * np.arange(V) + 1) % H
    lm[np.arange(V), col] = s
    bias = (rng.integers(-8, 8, V) * 0.25).astype(np.float32)
    inp = _custom(B, L, H, V, 0, hidden, _bf(lm), None, None, [0, 0], bias=bias)
    x = bf16_bits_to_f32(hidden).astype(np.float64)
    for b in range(B):
        z = orc.block_logits(inp, b)
        want = x[b][:, col] * s[None, :] + bias[None, :]
        assert np.array_equal(z, want), f"block {b}"


def pin_logits_vs_numpy_fp64(orc):
    for kw in (dict(), dict(layout=BONUS_ANCHOR), dict(hidden_f32=True)):
        inp = make_small(3, 5, 72, 97, 8, seed=3, **kw)
        want = _np_logits(inp)
        for b in range(inp.cfg.B):
            z = orc.block_logits(inp, b)
            np.testing.assert_allclose(z, want[b], rtol=0, atol=1e-12)


def pin_logits_bias_added(orc):
    inp = make_small(2, 3, 32, 50, 4, seed=5)
    bias = np.linspace(-3, 3, 50).astype(np.float32)
    inp2 = replace(inp, lm_head_bias=bias)
    for b in range(2):
        np.testing.assert_allclose(orc.block_logits(inp2, b) - orc.block_logits(inp, b),
                                   np.broadcast_to(bias.astype(np.float64), (3, 50)), atol=1e-12)


# --------------------------------------------------------------------------
# Markov bias and chain
# --------------------------------------------------------------------------

def pin_markov_bias_closed_form(orc):
    """w2[v] = a_v e_{v mod r}, w1[p] = c_p e_{p mod r}: m_p[v] = a_v c_p [v = p mod r]."""
    V, r = 24, 4
    a = np.array([1.0, -0.5, 2.0])[np.arange(V) % 3]
    cc = np.array([3.0, -1.0])[np.arange(V) % 2]
    w2 = np.zeros((V, r), np.float32)
    w1 = np.zeros((V, r), np.float32)
    w2[np.arange(V), np.arange(V) % r] = a
    w1[np.arange(V), (np.arange(V) + 1) % r] = cc
    inp = _custom(1, 1, 8, V, r, np.zeros((1, 1, 8), np.uint16), np.zeros((V, 8), np.uint16),
                  _bf(w1), _bf(w2), [0])
    for p in range(V):
        m = orc.markov_bias(inp, p)
        want = np.where(np.arange(V) % r == (p + 1) % r, a * cc[p], 0.0)
        assert np.array_equal(m, want), f"prev {p}"


def pin_markov_bias_vs_numpy(orc):
    inp = make_small(1, 2, 16, 300, 24, seed=9, w_std=0.3)
    T = _np_markov_table(inp)
    for p in (0, 1, 150, 299):
        np.testing.assert_allclose(orc.markov_bias(inp, p), T[p], atol=1e-12)


def pin_argmax_first_occurrence(orc):
    assert orc.argmax(np.array([1, 3, 3, 2], np.float32)) == 1
    assert orc.argmax(np.zeros(7, np.float32)) == 0
    assert orc.argmax(np.array([-0.0, 0.0], np.float32)) == 0
    assert orc.argmax(np.array([0.0, -0.0], np.float32)) == 0
    assert orc.argmax(np.array([-1e9, -1e9, -5.0, -5.0], np.float32)) == 2
    rng = np.random.default_rng(11)
    for _ in range(50):
        z = (rng.integers(-4, 5, 200) * 0.5).astype(np.float32)
        assert orc.argmax(z) == int(np.argmax(z))


def pin_topk_order(orc):
    rng = np.random.default_rng(12)
    for k in (1, 2, 4, 8, 16):
        for _ in range(20):
            z = (rng.integers(-6, 7, 90) * 0.25).astype(np.float32)
            idx, val = orc.topk(z, k)
            widx, wval = _np_topk(z, k)
            assert np.array_equal(idx, widx) and np.array_equal(val, wval), (k, idx, widx)


def pin_zero_markov_is_plain_argmax(orc):
    """Zero Markov weights (or r = 0): tokens are numpy.argmax of the fp32 projections,
    whatever the anchors."""
    inp = make_small(3, 6, 40, 211, 8, top_k=3, seed=21)
    zw = np.zeros_like(inp.markov_w1)
    want = np.argmax(_np_logits(inp).astype(np.float32), axis=-1)
    for variant in (replace(inp, markov_w1=zw, markov_w2=zw),
                    replace(inp, markov_w1=None, markov_w2=None, cfg=replace(inp.cfg, r=0))):
        for anchors in ([0, 5, 7], [210, 1, 100]):
            v2 = replace(variant, anchors=np.array(anchors, np.int32))
            out = orc.propose(v2)
            assert np.array_equal(out["tokens"], want)
            assert np.array_equal(out["candidates"][:, :, 0], want)


def _walk_tables(inp: Inputs, z: np.ndarray, k: int):
    """Brute force: for every slot j and every possible previous token p, the
    fp32 scores z_j + T[p] and their top-k; then walk the chain from the anchor."""
    T = _np_markov_table(inp)
    out = []
    for b in range(inp.cfg.B):
        scores = (z[b][:, None, :] + T[None, :, :]).astype(np.float32)   # [n, p, v]
        nxt = np.argmax(scores, axis=-1)                                   # [n, p]
        prev = int(inp.anchors[b])
        toks, cands, vals = [], [], []
        for j in range(z.shape[1]):
            t = int(nxt[j, prev])
            ci, cv = _np_topk(scores[j, prev], k)
            toks.append(t)
            cands.append(ci)
            vals.append(cv)
            prev = t
        out.append((np.array(toks), np.array(cands), np.array(vals)))
    return out


def pin_bruteforce_tiny_vocab(orc):
    """The tiny oracle workload (B=1, L=4, H=64, V=512, r=8, fp32 hidden) and a
    top-4 / bonus-anchor variant, against per-prev lookup tables."""
    from synthetic import CONFIGS, make_inputs
    cases = [make_inputs(CONFIGS["tiny"]),
             make_small(2, 5, 64, 512, 8, top_k=4, layout=BONUS_ANCHOR, seed=1, w_std=0.5)]
    for inp in cases:
        z = _np_logits(inp)
        want = _walk_tables(inp, z, inp.cfg.top_k)
        got = orc.propose(inp)
        for b, (t, c, v) in enumerate(want):
            assert np.array_equal(got["tokens"][b], t), (inp.cfg.name, b, got["tokens"][b], t)
            assert np.array_equal(got["candidates"][b], c)
            assert np.array_equal(got["cand_logits"][b], v)


def _golden():
    vals = {}
    with open(os.path.join(GOLDEN, "hand_chain_v4.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, *rest = line.split()
                vals[key] = rest
    return vals


def _golden_inputs(p_min=0.5, layout="anchor_first"):
    g = _golden()
    f = lambda k: np.array([float(x) for x in g[k]], np.float32)  # noqa: E731
    hidden = f("hidden").reshape(1, 3, 2)
    if layout == BONUS_ANCHOR:
        hidden = np.concatenate([np.full((1, 1, 2), np.nan, np.float32), hidden], axis=1)
    L = hidden.shape[1]
    return g, _custom(1, L, 2, 4, 2, f32_to_bf16_bits(hidden), _bf(f("lm_head").reshape(4, 2)),
                      _bf(f("markov_w1").reshape(4, 2)), _bf(f("markov_w2").reshape(4, 2)),
                      [int(g["anchor"][0])], top_k=2, conf_w=_bf(f("conf_w")), p_min=p_min,
                      layout=layout)


def pin_golden_hand_example(orc):
    for layout in ("anchor_first", BONUS_ANCHOR):
        g, inp = _golden_inputs(layout=layout)
        f = lambda k: np.array([float(x) for x in g[k]])  # noqa: E731
        out = orc.propose(inp)
        assert np.array_equal(out["logits"][0].ravel(), f("logits")), out["logits"]
        assert np.array_equal(out["tokens"][0], f("tokens").astype(int)), out["tokens"]
        assert np.array_equal(out["candidates"][0].ravel(), f("candidates").astype(int))
        assert np.array_equal(out["cand_logits"][0].ravel().astype(np.float64), f("cand_logits"))
        assert np.array_equal(out["conf"][0], f("conf").astype(np.float32))
        z = out["logits"][0]
        prev = int(g["anchor"][0])
        sc = f("scores").reshape(3, 4)
        for j in range(3):
            zp = orc.step_scores(inp, z[j], prev)
            assert np.array_equal(zp.astype(np.float64), sc[j])
            prev = int(out["tokens"][0][j])
        for item in g["lengths"]:
            p, want = item.split(":")
            _, inp_p = _golden_inputs(p_min=float(p), layout=layout)
            assert orc.propose(inp_p)["lengths"][0] == int(want), (layout, p)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def pin_masked_rows_never_emitted(orc):
    """Rows with a -1e9 bias (reduced draft vocabulary) never appear."""
    inp = make_small(3, 5, 48, 400, 8, top_k=4, layout=BONUS_ANCHOR, reachable=37, seed=4,
                     w_std=1.0)
    out = orc.propose(inp)
    allowed = set(int(x) for x in inp.reachable)
    assert set(out["tokens"].ravel().tolist()) <= allowed
    assert set(out["candidates"].ravel().tolist()) <= allowed
    assert np.all(out["cand_logits"] > -1e8)


def pin_layout_equivalence(orc):
    """1+N bonus-anchor block == anchor-first block without its slot 0, and the
    bonus slot is never read (NaN there changes nothing)."""
    for hf in (False, True):
        inp = make_small(3, 6, 40, 150, 8, top_k=3, layout=BONUS_ANCHOR, hidden_f32=hf, seed=8,
                         conf=True, p_min=0.45)
        af = replace(inp, hidden=np.ascontiguousarray(inp.hidden[:, 1:, :]),
                     cfg=replace(inp.cfg, layout="anchor_first", L=5))
        h = inp.hidden.copy()
        h[:, 0, :] = np.float32(np.nan) if hf else np.uint16(0x7FC0)
        poisoned = replace(inp, hidden=h)
        a, b, c = orc.propose(inp), orc.propose(af), orc.propose(poisoned)
        for key in ("logits", "tokens", "candidates", "cand_logits", "conf", "lengths"):
            assert np.array_equal(a[key], b[key]), key
            assert np.array_equal(a[key], c[key]), key


def pin_block_permutation_equivariance(orc):
    inp = make_small(5, 4, 32, 120, 8, top_k=2, seed=13, conf=True, p_min=0.4)
    perm = np.array([3, 0, 4, 2, 1])
    pin = replace(inp, hidden=np.ascontiguousarray(inp.hidden[perm]),
                  anchors=np.ascontiguousarray(inp.anchors[perm]))
    a, b = orc.propose(inp), orc.propose(pin)
    for key in ("logits", "tokens", "candidates", "cand_logits", "conf", "lengths"):
        assert np.array_equal(a[key][perm], b[key]), key


def pin_candidates_head_is_token(orc):
    for k in (1, 4):
        inp = make_small(4, 5, 32, 256, 8, top_k=k, seed=17, w_std=0.4)
        out = orc.propose(inp)
        assert np.array_equal(out["candidates"][:, :, 0], out["tokens"])
        for b in range(4):
            for j in range(5):
                assert len(set(out["candidates"][b, j].tolist())) == k
                assert np.all(np.diff(out["cand_logits"][b, j]) <= 0)


def pin_chain_conditions_on_previous_argmax(orc):
    """Each slot's scores equal the projection plus the Markov row of the previous
    slot's token (the anchor for slot 0), checked through the numpy table."""
    inp = make_small(2, 6, 32, 97, 8, top_k=1, seed=19, w_std=0.6)
    T = _np_markov_table(inp)
    z = _np_logits(inp)
    out = orc.propose(inp)
    for b in range(2):
        prev = int(inp.anchors[b])
        for j in range(6):
            want = np.argmax((z[b, j] + T[prev]).astype(np.float32))
            assert out["tokens"][b, j] == want
            prev = int(want)


# --------------------------------------------------------------------------
# confidence and truncation
# --------------------------------------------------------------------------

def pin_sigmoid_closed_form(orc):
    """conf_w = e_0: conf_j = sigma(x_j[0]); sigma(0) = 1/2 exactly, sigma(+-2) known."""
    H = 8
    x = np.zeros((1, 4, H), np.float32)
    x[0, :, 0] = [0.0, 2.0, -2.0, 0.5]
    x[0, :, 3] = 7.0          # not read by conf_w = e_0
    cw = np.zeros(H, np.float32)
    cw[0] = 1.0
    inp = _custom(1, 4, H, 5, 0, _bf(x), np.zeros((5, H), np.uint16), None, None, [0],
                  conf_w=_bf(cw))
    got = orc.conf(inp, 0)
    want = np.array([0.5, 1 / (1 + math.exp(-2)), 1 / (1 + math.exp(2)), 1 / (1 + math.exp(-0.5))],
                    np.float32)
    assert np.array_equal(got, want), (got, want)


def pin_truncation_patterns(orc):
    c = np.array([0.9, 0.8, 0.2, 0.9], np.float32)      # non-monotone: dips at slot 2
    assert orc.truncate(c, 0.5) == 2
    assert orc.truncate(c, 0.0) == 4                     # 0 disables
    assert orc.truncate(c, 1.5) == 0                     # p_min > 1 cuts everything
    assert orc.truncate(c, 0.2) == 4                     # equal is not below
    assert orc.truncate(c, 0.85) == 1
    assert orc.truncate(np.array([0.1], np.float32), 0.5) == 0
    # end to end through hidden states: conf logits 2, 1, -1, 3 -> cut at slot 2
    H = 8
    x = np.zeros((2, 4, H), np.float32)
    x[0, :, 1] = [2.0, 1.0, -1.0, 3.0]
    x[1, :, 1] = [3.0, 3.0, 3.0, 3.0]
    cw = np.zeros(H, np.float32)
    cw[1] = 1.0
    for p_min, want in ((0.5, [2, 4]), (0.0, [4, 4]), (1.01, [0, 0]), (0.75, [1, 4])):
        inp = _custom(2, 4, H, 6, 0, _bf(x), np.zeros((6, H), np.uint16), None, None, [0, 1],
                      conf_w=_bf(cw), p_min=p_min)
        assert orc.propose(inp)["lengths"].tolist() == want, p_min


def pin_no_conf_head_keeps_full_block(orc):
    inp = make_small(2, 5, 32, 64, 4, seed=23)
    out = orc.propose(replace(inp, cfg=replace(inp.cfg, p_min=0.9)))
    assert out["lengths"].tolist() == [5, 5]
    assert np.all(out["conf"] == 1.0)


def _d2t_cases():
    from synthetic.inputs import BONUS_ANCHOR
    return [
        make_small(3, 5, 64, 700, 16, top_k=3, reachable=90, conf=True, p_min=0.45, seed=31),
        make_small(2, 6, 32, 300, 0, top_k=2, reachable=40, seed=32),
        make_small(2, 5, 48, 257, 8, top_k=4, reachable=4, layout=BONUS_ANCHOR, conf=True,
                   p_min=0.5, conf_trend=True, seed=33),
    ]


def pin_d2t_equals_expanded_form(orc):
    """The run-time d2t scatter (llama.cpp PR #26275, rework commit message)
    and the expanded form it replaces (first commit message: lm_head and
    markov_w2 rows placed at their target ids, zero rows and a -1e9 bias
    elsewhere) give the same tokens, candidates, scores, confidences and
    cuts; the draft projections are the expanded ones at the d2t columns."""
    for inp in _d2t_cases():
        red = reduce_vocab(inp)
        assert not np.array_equal(red.d2t, np.arange(red.D))   # a real remap
        for b in range(inp.cfg.B):
            e = orc.propose_block(inp, b)
            d = orc.propose_block_d2t(red, b)
            for key in ("tokens", "candidates", "cand_logits", "conf"):
                assert np.array_equal(e[key], d[key]), key
            assert e["length"] == d["length"]
            assert np.array_equal(e["logits"][:, red.d2t], d["logits"])
            assert set(d["candidates"].ravel().tolist()) <= set(red.d2t.tolist())


def pin_d2t_identity_is_plain(orc):
    """With D = V and d2t the identity, the reduced form is the plain step."""
    inp = make_small(2, 4, 32, 200, 8, top_k=3, conf=True, p_min=0.4, seed=34)
    red = ReducedInputs(cfg=inp.cfg, hidden=inp.hidden, lm_head=inp.lm_head,
                        d2t=np.arange(inp.cfg.V, dtype=np.int64), markov_w1=inp.markov_w1,
                        markov_w2=inp.markov_w2, conf_w=inp.conf_w, anchors=inp.anchors)
    for b in range(inp.cfg.B):
        e = orc.propose_block(inp, b)
        d = orc.propose_block_d2t(red, b)
        for key in ("logits", "tokens", "candidates", "cand_logits", "conf"):
            assert np.array_equal(e[key], d[key]), key


def pin_verify_hand_example(orc):
    """Greedy verification worked by hand. Candidates [B=3, n=4, k=2]:
    block 0 drafts 5 6 7 8 (runners-up 1 2 3 4), length 4, target 5 6 3 8:
    the chain stops at slot 2 (3 is not the draft 7), the lattice takes the
    runner-up 3 and then 8: 2 and 4. Block 1, length 2 (truncated), target
    equal to the draft everywhere: 2 for both (the cut ends the walk).
    Block 2, target 9 at slot 0: 0 for both."""
    cand = np.array([[[5, 1], [6, 2], [7, 3], [8, 4]],
                     [[1, 2], [3, 4], [5, 6], [7, 8]],
                     [[4, 5], [6, 7], [8, 9], [1, 2]]], dtype=np.int32)
    lengths = np.array([4, 2, 4], dtype=np.int32)
    target = np.array([[5, 6, 3, 8], [1, 3, 5, 7], [9, 6, 8, 1]], dtype=np.int32)
    acc, tot = orc.verify(cand, lengths, target, lattice=False)
    assert acc.tolist() == [2, 2, 0] and tot == (4, 10)
    acc, tot = orc.verify(cand, lengths, target, lattice=True)
    assert acc.tolist() == [4, 2, 0] and tot == (6, 10)


def pin_verify_bruteforce(orc):
    """Random small lattices against the definition written as a maximum: the
    largest m <= clamped length such that every slot below m holds the target
    among its first w candidates. Also: target equal to the chain accepts the
    whole submitted block, and the lattice never accepts less than the chain."""
    rng = np.random.default_rng(7)
    for _ in range(40):
        B, n, k = int(rng.integers(1, 6)), int(rng.integers(1, 7)), int(rng.integers(1, 5))
        cand = rng.integers(0, 5, size=(B, n, k)).astype(np.int32)
        lengths = rng.integers(-1, n + 2, size=B).astype(np.int32)
        target = rng.integers(0, 5, size=(B, n)).astype(np.int32)
        for lattice in (False, True):
            w = k if lattice else 1
            acc, tot = orc.verify(cand, lengths, target, lattice=lattice)
            want = []
            for b in range(B):
                cap = min(max(int(lengths[b]), 0), n)
                ok = [m for m in range(cap + 1)
                      if all(target[b, j] in cand[b, j, :w].tolist() for j in range(m))]
                want.append(max(ok))
            assert acc.tolist() == want
            assert tot == (sum(want), sum(min(max(int(l), 0), n) for l in lengths))
        chain_acc, _ = orc.verify(cand, lengths, target, lattice=False)
        lat_acc, _ = orc.verify(cand, lengths, target, lattice=True)
        assert np.all(lat_acc >= chain_acc)
        acc, _ = orc.verify(cand, lengths, cand[:, :, 0], lattice=False)
        assert acc.tolist() == [min(max(int(l), 0), n) for l in lengths]


def pin_gated_equals_masked_full_step(orc):
    """Under the adaptive gate a block drafts only the slots that survive its
    own threshold, with its own number of candidates: on those slots the
    outputs are the plain step's (same prefix of the chain, top-k a prefix of
    the larger top-k), everything past the cut is -1 / -inf, and the cut is
    the plain step's cut under that threshold."""
    from synthetic.inputs import BONUS_ANCHOR
    cases = [make_small(4, 6, 64, 900, 16, top_k=4, conf=True, conf_trend=True, seed=51),
             make_small(3, 7, 48, 500, 8, top_k=3, conf=True, conf_trend=True,
                        layout=BONUS_ANCHOR, seed=52)]
    for inp in cases:
        c = inp.cfg
        for b in range(c.B):
            for p_min, kb in ((0.0, c.top_k), (0.5, 2), (0.7, 1), (0.99, c.top_k)):
                full = orc.propose_block(replace(inp, cfg=replace(c, p_min=p_min)), b)
                g = orc.propose_block_gated(inp, b, p_min, kb)
                n = g["length"]
                assert n == full["length"]
                assert np.array_equal(g["conf"], full["conf"])
                assert np.array_equal(g["logits"], full["logits"])
                assert np.array_equal(g["tokens"][:n], full["tokens"][:n])
                assert np.all(g["tokens"][n:] == -1)
                assert np.array_equal(g["candidates"][:n, :kb], full["candidates"][:n, :kb])
                assert np.array_equal(g["cand_logits"][:n, :kb], full["cand_logits"][:n, :kb])
                assert np.all(g["candidates"][:, kb:] == -1) and np.all(g["candidates"][n:] == -1)
                assert np.all(np.isneginf(g["cand_logits"][:, kb:]))
                assert np.all(np.isneginf(g["cand_logits"][n:]))
    # the thresholds used above do cut some blocks early and keep others whole
    inp = cases[0]
    lens = [orc.propose_block_gated(inp, b, 0.5, 1, keep_logits=False)["length"] for b in range(4)]
    assert min(lens) < inp.cfg.n_pred


# --------------------------------------------------------------------------
# 4-bit head (GGUF plain 4-bit blocks; the reading is stated in oracle.c)
# --------------------------------------------------------------------------

def _golden_q4_row():
    """(row bytes uint8 [72], values float64 [128]) of golden/q4_row_h128.txt."""
    raw, vals = [], []
    with open(os.path.join(GOLDEN, "q4_row_h128.txt")) as f:
        for line in f:
            t = line.split()
            if not t or t[0].startswith("#"):
                continue
            if t[0] == "bytes":
                raw += [int(x, 16) for x in t[1:]]
            elif t[0] == "values":
                for x in t[1:]:
                    if "*2^" in x:
                        k, e = x.split("*2^")
                        vals.append(math.ldexp(float(k), int(e)))
                    else:
                        vals.append(float(x))
    return np.array(raw, dtype=np.uint8), np.array(vals, dtype=np.float64)


def _np_q4_dequant(q4: np.ndarray, H: int) -> np.ndarray:
    """[V, H] float64 weights of GGUF 4-bit blocks, decoded with numpy's binary16."""
    V = q4.shape[0]
    blk = q4.reshape(V, H // 32, 18)
    d = blk[:, :, :2].copy().view("<f2")[:, :, 0].astype(np.float64)
    qs = blk[:, :, 2:].astype(np.int64)
    codes = np.concatenate([qs & 15, qs >> 4], axis=2)        # elements j, then j + 16
    return (d[:, :, None] * (codes - 8)).reshape(V, H)


def _q4_custom(inp: Inputs, q4: np.ndarray) -> Q4Inputs:
    return Q4Inputs(cfg=inp.cfg, hidden=inp.hidden, lm_head_q4=np.ascontiguousarray(q4),
                    lm_head_bias=inp.lm_head_bias, markov_w1=inp.markov_w1, markov_w2=inp.markov_w2,
                    conf_w=inp.conf_w, anchors=inp.anchors, reachable=inp.reachable)


def pin_f16_value(orc):
    """binary16 decoding: hand values and numpy's float16 on all 65536 patterns."""
    for bits, want in {0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24,
                       0x0400: 2.0 ** -14, 0x03FF: 1023 * 2.0 ** -24, 0x3555: 0.333251953125,
                       0xC200: -3.0, 0x8001: -(2.0 ** -24), 0x7C00: math.inf}.items():
        got = orc.f16_value(bits)
        assert got == want, f"f16_value({bits:#06x}) = {got!r}, want {want!r}"
    assert math.copysign(1.0, orc.f16_value(0x8000)) == -1.0
    allbits = np.arange(1 << 16, dtype=np.uint16)
    ref = allbits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_value(int(b)) for b in allbits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), allbits[~same][:8]


def pin_q4_golden_row(orc):
    """The hand-decoded row, through the decoder and through the projection
    (one-hot hidden rows pick the weights out one by one)."""
    row, want = _golden_q4_row()
    H = 128
    assert row.size == H // 32 * 18 and want.size == H
    got = orc.q4_dequant_row(row.reshape(1, -1), H, 0)
    assert np.array_equal(got, want), np.nonzero(got != want)
    # row 1 is row 0 with its blocks in reverse order: the block stride shows
    q4 = np.stack([row, row.reshape(4, 18)[::-1].ravel()])
    hidden = np.zeros((1, H, H), dtype=np.uint16)
    hidden[0, np.arange(H), np.arange(H)] = 0x3F80            # bf16 1.0
    inp = _custom(1, H, H, 2, 0, hidden, np.zeros((2, H), np.uint16), None, None, [0])
    z = orc.block_logits(_q4_custom(inp, q4), 0)
    assert np.array_equal(z[:, 0], want)
    assert np.array_equal(z[:, 1], want.reshape(4, 32)[::-1].ravel())


def pin_q4_logits_vs_numpy(orc):
    """Random codes and scales (negative, zero and subnormal scales included),
    fp32 hidden: numpy decode + fp64 matmul."""
    for layout, f32 in (("anchor_first", True), (BONUS_ANCHOR, False)):
        inp = make_small(3, 6, 96, 211, 8, top_k=2, layout=layout, hidden_f32=f32, seed=61)
        q = quantize_q4(inp, "random")
        w = _np_q4_dequant(q.lm_head_q4, 96)
        assert np.any(w < 0) and np.any(w == 0)
        x = (bf16_bits_to_f32(f32_to_bf16_bits(inp.hidden)) if f32 else bf16_bits_to_f32(inp.hidden))
        x = x.astype(np.float64)[:, inp.cfg.i_first_pred:, :]
        want = x @ w.T
        for b in range(inp.cfg.B):
            z = orc.block_logits(q, b)
            assert np.allclose(z, want[b], rtol=1e-12, atol=1e-12), np.abs(z - want[b]).max()


def pin_q4_equals_bf16_when_weights_are_bf16(orc):
    """Power-of-two scales make every decoded weight a bf16 value: the q4
    proposal must then be the bf16 proposal of the decoded head, bit for bit
    (logits included: the same products summed in the same order)."""
    inp = make_small(4, 6, 128, 300, 8, top_k=3, conf=True, p_min=0.45, conf_trend=True, seed=62,
                     w_std=0.5, reachable=120)
    rng = np.random.default_rng(7)
    V, H = 300, 128
    codes = rng.integers(0, 16, size=(V, H), dtype=np.uint8)
    scales = np.ldexp(1.0, rng.integers(-9, -4, size=(V, H // 32))).astype(np.float16)
    scales[~np.isin(np.arange(V), inp.reachable)] = 0
    q4 = q4_blocks(codes, scales)
    w = _np_q4_dequant(q4, H)
    lm = f32_to_bf16_bits(w.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32(lm).astype(np.float64), w)
    ref = orc.propose(replace(inp, lm_head=lm))
    got = orc.propose(_q4_custom(inp, q4))
    for k in ("logits", "tokens", "candidates", "cand_logits", "conf", "lengths"):
        assert np.array_equal(got[k], ref[k]), k


def pin_q4_scale_linearity(orc):
    """Doubling every scale doubles every projection exactly (no bias)."""
    inp = make_small(2, 5, 64, 97, 0, seed=63)
    q = quantize_q4(inp, "round")
    q2 = q.lm_head_q4.reshape(97, 2, 18).copy()
    d = q2[:, :, :2].copy().view("<f2")
    assert np.all(np.abs(d.astype(np.float64)) < 16000)
    q2[:, :, :2] = (d * np.float16(2)).view(np.uint8)
    for b in range(2):
        z1 = orc.block_logits(q, b)
        z2 = orc.block_logits(_q4_custom(inp, q2.reshape(97, 36)), b)
        assert np.array_equal(z2, 2.0 * z1)


def pin_q4_zero_weights_give_bias(orc):
    """Code 8 everywhere (any scale) or scale 0 (any code): the projection is the bias."""
    inp = make_small(2, 4, 64, 50, 4, reachable=20, seed=64, w_std=0.5)
    rng = np.random.default_rng(8)
    eights = q4_blocks(np.full((50, 64), 8, np.uint8),
                       rng.standard_normal((50, 2)).astype(np.float16))
    zeros = q4_blocks(rng.integers(0, 16, (50, 64), dtype=np.uint8), np.zeros((50, 2), np.float16))
    for q4 in (eights, zeros):
        for b in range(2):
            z = orc.block_logits(_q4_custom(inp, q4), b)
            assert np.array_equal(z, np.broadcast_to(inp.lm_head_bias.astype(np.float64), z.shape))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
