"""The parity gate itself, pinned.

``oracle.check`` turns oracle scores into every GPU pass / fail verdict, so it
is tested here on its own, without a GPU:

* valid proposals must pass: the oracle's own outputs; a slot whose two best
  scores lie within the score tolerance resolved the other way, with the rest
  of the block conditioned on that choice (the re-conditioning rule: greedy
  drafting stays lossless whichever of two tied tokens is taken, llama.cpp
  commit 6fed9f6 "spec: add DSpark speculative decoding"); a confidence within
  its tolerance that crosses p_min and moves the cut by one slot; a proposal
  without its optional outputs;
* planted mistakes must be rejected, each by the rule written for it (the
  ParityError message names the rule): a wrong token, the runner-up taken
  outside the margin, swapped candidates, a repeated candidate, a head
  candidate that is not the token, an out-of-range token, a candidate score,
  a logit and a confidence moved past their tolerances, and cuts off by one;
* planted mistakes in the checker's own source (a dropped rule, a rule that
  re-conditions on the oracle's token instead of the GPU's, off-by-one cut
  windows, loosened tolerances) must each make one of those cases come out
  wrong.

The rule that an isolated candidate must carry the oracle's id is implied by
the candidate-score rule plus distinctness (a distinct id whose score lies
within the tolerance of an isolated rank's score cannot exist), so it has no
plant of its own; it is the backup that catches swapped candidates when the
score rule is removed.
"""
from __future__ import annotations

import copy
import types

import numpy as np
import pytest

import oracle.check as checker
from oracle import Oracle
from synthetic import make_small
from synthetic.inputs import with_config

TOL = checker.TOL_SCORE


def _inp():
    # strong Markov weights, so the previous token decides the next argmax
    return make_small(8, 6, 64, 300, 8, top_k=4, conf=True, p_min=0.5, conf_trend=True,
                      w_std=0.5, seed=91)


def _walk(orc, inp, z, prev, first=None):
    """The chain of one block over projections z (fp64 [n, V]) from prev, as
    the oracle's own steps take it; `first` forces slot 0's token."""
    n, k = z.shape[0], inp.cfg.top_k
    tok = np.empty(n, np.int32)
    cand = np.empty((n, k), np.int32)
    cval = np.empty((n, k), np.float32)
    for j in range(n):
        zp = orc.step_scores(inp, z[j], prev)
        idx, val = orc.topk(zp, k)
        if j == 0 and first is not None:
            rest = [int(i) for i in idx if int(i) != first][: k - 1]
            idx = np.array([first] + rest, np.int32)
            val = zp[idx]
        tok[j], cand[j], cval[j] = idx[0], idx, val
        prev = int(idx[0])
    return tok, cand, cval


class Scenario:
    """Oracle outputs for every block, shaped like the GPU binding's."""

    def __init__(self, orc):
        self.orc = orc
        self.inp = _inp()
        c = self.inp.cfg
        ref = orc.propose(self.inp)
        self.z = {b: ref["logits"][b] for b in range(c.B)}
        self.out = {
            "logits": np.concatenate([ref["logits"][b] for b in range(c.B)]).astype(np.float32),
            "tokens": ref["tokens"].copy(), "candidates": ref["candidates"].copy(),
            "cand_logits": ref["cand_logits"].copy(), "conf": ref["conf"].copy(),
            "lengths": ref["lengths"].copy(),
        }
        self.oc = {b: orc.conf(self.inp, b) for b in range(c.B)}

    def scores(self, b, j, prev=None):
        """Oracle biased scores of slot j of block b on the oracle's own chain."""
        if prev is None:
            prev = int(self.inp.anchors[b]) if j == 0 else int(self.out["tokens"][b, j - 1])
        return self.orc.step_scores(self.inp, self.z[b][j], prev)

    def find_slot(self, pred):
        c = self.inp.cfg
        for b in range(c.B):
            for j in range(c.n_pred):
                zp = self.scores(b, j)
                idx, val = self.orc.topk(zp, c.top_k + 1)
                if pred(b, j, idx, val):
                    return b, j, idx, val
        raise AssertionError("the scenario has no slot of the kind this case needs")


# A case: (inp, gpu outputs, {block: z}, blocks, expected message fragment or None).

def valid_cases(s: Scenario):
    orc, inp, c = s.orc, s.inp, s.inp.cfg
    cases = {"oracle_outputs": (inp, s.out, s.z, list(range(c.B)), None)}

    # A near tie at slot 0 taken the other way, the rest of the block
    # conditioned on that choice. Block chosen so that the choice matters for
    # slot 1 (a checker that re-conditions on the oracle's token fails here).
    for b in range(c.B):
        z = s.z[b].copy()
        prev0 = int(inp.anchors[b])
        zp = orc.step_scores(inp, z[0], prev0)
        idx, val = orc.topk(zp, 2)
        a, r = int(idx[0]), int(idx[1])
        z[0, r] += float(val[0]) - float(val[1]) - 0.005
        zp = orc.step_scores(inp, z[0], prev0)
        if not (0.0 < float(zp[a]) - float(zp[r]) < 0.01 and orc.argmax(zp) == a):
            continue
        if orc.argmax(orc.step_scores(inp, z[1], a)) == orc.argmax(orc.step_scores(inp, z[1], r)):
            continue
        tok, cand, cval = _walk(orc, inp, z, prev0, first=r)
        g = copy.deepcopy(s.out)
        g["logits"][b * c.n_pred:(b + 1) * c.n_pred] = z.astype(np.float32)
        g["tokens"][b], g["candidates"][b], g["cand_logits"][b] = tok, cand, cval
        cases["near_tie_reconditioned"] = (inp, g, {b: z}, [b], None)
        break
    assert "near_tie_reconditioned" in cases, "no block where the near tie changes the chain"

    # A confidence within its tolerance of the oracle's that crosses p_min: the
    # GPU's cut moves one slot later, and both cut points are accepted.
    for b in range(c.B):
        oc = s.oc[b]
        js = [j for j in range(1, c.n_pred) if oc[j] < oc[:j].min() - 3e-3]
        if not js:
            continue
        j = js[0]
        p_min = float(np.float32(oc[j]) + np.float32(4e-4))
        inp2 = with_config(inp, p_min=p_min)
        g = copy.deepcopy(s.out)
        g["conf"][b, j] = np.float32(p_min + 3e-4)
        g["lengths"][b] = next((i for i in range(c.n_pred) if g["conf"][b, i] < np.float32(p_min)),
                               c.n_pred)
        assert g["lengths"][b] > j
        cases["conf_within_tol_moves_cut"] = (inp2, g, s.z, [b], None)
        break
    assert "conf_within_tol_moves_cut" in cases

    g = copy.deepcopy(s.out)
    g["cand_logits"], g["conf"], g["logits"] = None, None, None
    cases["optional_outputs_absent"] = (inp, g, s.z, list(range(c.B)), None)
    return cases


def planted_cases(s: Scenario):
    orc, inp, c = s.orc, s.inp, s.inp.cfg
    cases = {}

    def plant(name, b, fn, expect, inp_=None):
        g = copy.deepcopy(s.out)
        fn(g)
        cases[name] = (inp_ or inp, g, s.z, [b], expect)

    # a token that is neither the argmax nor a tied runner-up
    b, j, idx, val = s.find_slot(lambda b, j, idx, val: j == 0 and val[0] - val[2] > 0.05)

    def f(g, b=b, j=j, idx=idx):
        g["tokens"][b, j] = idx[2]
        g["candidates"][b, j] = [idx[2], idx[0], idx[1], idx[3]]
    plant("wrong_token", b, f, "gpu token")

    # the runner-up taken outside the margin, candidates consistent with it
    b, j, idx, val = s.find_slot(lambda b, j, idx, val: j == 0 and val[0] - val[1] > 0.05)

    def f(g, b=b, j=j, idx=idx):
        g["tokens"][b, j] = idx[1]
        g["candidates"][b, j] = [idx[1], idx[0], idx[2], idx[3]]
        g["cand_logits"][b, j] = s.scores(b, j)[g["candidates"][b, j]]
    plant("runner_up_outside_margin", b, f, "gpu token")

    # ranks 1 and 2 swapped where both scores are isolated
    b, j, idx, val = s.find_slot(lambda b, j, idx, val: min(val[0] - val[1], val[1] - val[2],
                                                            val[2] - val[3]) > 2 * TOL)

    def f(g, b=b, j=j, idx=idx):
        g["candidates"][b, j, 1], g["candidates"][b, j, 2] = idx[2], idx[1]
        g["cand_logits"][b, j] = s.scores(b, j)[g["candidates"][b, j]]
    plant("swapped_isolated_candidates", b, f, "scores")

    b, j, idx, val = s.find_slot(lambda b, j, idx, val: val[1] - val[2] > 2 * TOL)

    def f(g, b=b, j=j):
        g["candidates"][b, j, 2] = g["candidates"][b, j, 1]
    plant("repeated_candidate", b, f, "repeated candidates")

    b, j, idx, val = s.find_slot(lambda b, j, idx, val: val[0] - val[1] > 2 * TOL)

    def f(g, b=b, j=j, idx=idx):
        g["candidates"][b, j, 0], g["candidates"][b, j, 1] = idx[1], idx[0]
    plant("head_candidate_not_token", b, f, "!= token")

    def f(g):
        g["tokens"][0, 0] = c.V
    plant("token_out_of_range", 0, f, "out of range")

    b, j, idx, val = s.find_slot(lambda b, j, idx, val: val[2] - val[3] > 2 * TOL
                                 and val[3] - val[4] > 2 * TOL)

    def f(g, b=b, j=j, idx=idx):
        g["candidates"][b, j, 3] = idx[4]   # the fifth best instead of the fourth
        g["cand_logits"][b, j, 3] = val[4]
    plant("wrong_last_candidate", b, f, "scores")

    def f(g):
        g["cand_logits"][1, 2, 1] += np.float32(0.03)
    plant("cand_logit_plus_0.03", 1, f, "cand_logit")

    def f(g):
        g["logits"][1 * c.n_pred + 3, 77] += np.float32(0.03)
    plant("logit_plus_0.03", 1, f, "logits[")

    # conf + 2e-3 on a slot far from p_min (the cut stays where it is)
    bj = [(b, j) for b in range(c.B) for j in range(c.n_pred) if abs(s.oc[b][j] - c.p_min) > 0.05]
    b, j = bj[0]

    def f(g, b=b, j=j):
        g["conf"][b, j] += np.float32(2e-3)
    plant("conf_plus_2e-3", b, f, ": conf [")

    # cuts off by one where the oracle's cut is clear
    bs = [b for b in range(c.B) if s.out["lengths"][b] < c.n_pred
          and s.oc[b][s.out["lengths"][b]] < c.p_min - 0.01]
    b = bs[0]

    def f(g, b=b):
        g["lengths"][b] += 1
    plant("length_plus_one", b, f, "its own conf cuts at")

    def f(g, b=b):
        g["lengths"][b] += 1
        g["conf"] = None
    plant("length_plus_one_without_conf", b, f, "accepts")

    bs = [b for b in range(c.B) if 0 < s.out["lengths"][b]
          and s.oc[b][s.out["lengths"][b] - 1] > c.p_min + 0.01]
    b = bs[0]

    def f(g, b=b):
        g["lengths"][b] -= 1
        g["conf"] = None
    plant("length_minus_one_without_conf", b, f, "accepts")
    return cases


def outcome(mod, orc, case):
    """None when the checker accepts, else the ParityError message."""
    inp, g, zs, blocks, _ = case
    try:
        for b in blocks:
            mod.check_block(orc, inp, b, g, z=zs.get(b))
    except mod.ParityError as e:
        return str(e)
    except Exception as e:   # a crash is a failed test too, but not the rule's verdict
        return f"crash {type(e).__name__}: {e}"
    return None


def wrong_outcomes(mod, orc, valid, planted):
    """Names of the cases the checker `mod` gets wrong."""
    bad = []
    for name, case in valid.items():
        if outcome(mod, orc, case) is not None:
            bad.append(name)
    for name, case in planted.items():
        msg = outcome(mod, orc, case)
        if msg is None or case[4] not in msg:
            bad.append(name)
    return bad


@pytest.fixture(scope="module")
def scenario(orc):
    s = Scenario(orc)
    return s, valid_cases(s), planted_cases(s)


def test_valid_proposals_pass(scenario, orc):
    s, valid, _ = scenario
    for name, case in valid.items():
        assert outcome(checker, orc, case) is None, name


@pytest.mark.parametrize("name", ["wrong_token", "runner_up_outside_margin",
                                  "swapped_isolated_candidates", "repeated_candidate",
                                  "head_candidate_not_token", "token_out_of_range",
                                  "wrong_last_candidate", "cand_logit_plus_0.03",
                                  "logit_plus_0.03", "conf_plus_2e-3", "length_plus_one",
                                  "length_plus_one_without_conf", "length_minus_one_without_conf"])
def test_planted_mistake_rejected_by_its_rule(scenario, orc, name):
    s, _, planted = scenario
    case = planted[name]
    msg = outcome(checker, orc, case)
    assert msg is not None, f"{name} was accepted"
    assert case[4] in msg, f"{name} rejected by another rule: {msg}"


CHECKER_MUTANTS = {
    "reconditions_on_oracle_token": ("        prev = gtok\n", "        prev = int(oidx[0])\n"),
    "near_tie_never_accepted": (
        "elif V > 1 and gtok == int(oidx[1]) and float(oval[0]) - float(oval[1]) < TOL_SCORE:",
        "elif False:"),
    "margin_dropped": (
        "elif V > 1 and gtok == int(oidx[1]) and float(oval[0]) - float(oval[1]) < TOL_SCORE:",
        "elif V > 1 and gtok == int(oidx[1]):"),
    "logits_unchecked": ('if rep["max_logit_err"] > TOL_LOGITS:', "if False:"),
    "distinctness_dropped": ("if len(set(gc)) != k:", "if False:"),
    "head_rule_dropped": ("if gc[0] != gtok:", "if False:"),
    "rank_score_dropped": ("if abs(float(zp[gc[t]]) - float(oval[t])) >= TOL_SCORE:", "if False:"),
    "cand_logits_unchecked": (
        "if cvals is not None and abs(float(cvals[j, t]) - float(zp[gc[t]])) >= TOL_SCORE:",
        "if False:"),
    "conf_unchecked": ('if rep["max_conf_err"] > TOL_CONF:', "if False:"),
    "own_cut_unchecked": ("if glen != own:", "if False:"),
    "cut_window_unchecked": ("if glen not in ok:", "if False:"),
    "cut_window_prefix_off_by_one": ("for j in range(ell))", "for j in range(ell + 1))"),
    "cut_window_cut_off_by_one": ("cut_ok = ell == n or float(oc[ell]) < c.p_min + TOL_CONF",
                                  "cut_ok = ell == n or float(oc[ell - 1]) < c.p_min + TOL_CONF"),
    "token_range_unchecked": ("if not (0 <= gtok < V):", "if False:"),
    "logit_tolerance_loose": ("TOL_LOGITS = 2e-2", "TOL_LOGITS = 2e-1"),
    "score_tolerance_loose": ("TOL_SCORE = 2e-2", "TOL_SCORE = 2e-1"),
    "conf_tolerance_loose": ("TOL_CONF = 1e-3", "TOL_CONF = 1e-2"),
}


def _checker_source():
    with open(checker.__file__) as f:
        return f.read()


def _load_mutant(src: str):
    mod = types.ModuleType("oracle._check_mutant")
    mod.__package__ = "oracle"
    mod.__file__ = "check_mutant.py"
    exec(compile(src, "check_mutant.py", "exec"), mod.__dict__)
    return mod


def test_unmutated_copy_gets_everything_right(scenario, orc):
    s, valid, planted = scenario
    assert wrong_outcomes(_load_mutant(_checker_source()), orc, valid, planted) == []


@pytest.mark.parametrize("name", sorted(CHECKER_MUTANTS))
def test_checker_mutant_is_caught(scenario, orc, name):
    s, valid, planted = scenario
    old, new = CHECKER_MUTANTS[name]
    src = _checker_source()
    assert src.count(old) == 1, f"mutation site of {name} not found exactly once"
    mod = _load_mutant(src.replace(old, new))
    assert wrong_outcomes(mod, orc, valid, planted), f"no case catches the checker mutant {name}"
