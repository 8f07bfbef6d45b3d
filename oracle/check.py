"""Re-conditioning checker: GPU proposals against the CPU oracle (test infrastructure).

The chain's argmax is decided on fp32 scores, and the GPU sums in another order
than the oracle, so a slot whose two best scores lie closer than the score
tolerance may legitimately resolve either way. The checker walks each block
slot by slot with prev = anchor, recomputes the oracle's biased scores under
that prev, and accepts the GPU token g when

* g is the oracle's argmax, or
* g is the oracle's runner-up and the oracle's top-2 margin is below TOL_SCORE;

it then conditions the next slot on g (the GPU's choice), so one near-tie does
not cascade. Everything else is compared on what is unique:

* logits: |gpu - oracle| <= TOL_LOGITS everywhere;
* candidates: distinct, candidates[..., 0] == token, and for each rank t the
  oracle score of the GPU's t-th candidate lies within TOL_SCORE of the
  oracle's t-th best score; where the oracle's t-th score is separated from
  its neighbours by more than TOL_SCORE the id itself must match;
* cand_logits: within TOL_SCORE of the oracle score of that id;
* conf: within TOL_CONF;
* lengths: the first slot whose GPU conf is below p_min (self-consistency),
  and equal to the oracle's unless a confidence in the prefix lies within
  TOL_CONF of p_min, where both cut points are accepted.

Tolerances: a bf16 x bf16 product is exact in fp32 and any fp32 summation
order of H terms is within gamma_H * sum|x_h w_h| of the exact sum (Higham);
at H = 5120 with the synthetic distributions sum|x w| is about 46, which
bounds the logit error by about 0.014 < 2e-2 (typical errors are ~1e-5). The
Markov term adds at most r * 2^-24 * sum|w2 u| (< 1e-5). The confidence moves
by at most a quarter of its logit's error (sigma' <= 1/4).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import Oracle

TOL_LOGITS = 2e-2
TOL_SCORE = 2e-2
TOL_CONF = 1e-3


class ParityError(AssertionError):
    pass


def check_block(orc: Oracle, inp, b: int, gpu: dict, z: Optional[np.ndarray] = None,
                check_logits: bool = True) -> dict:
    """Check every output of block b. ``gpu`` holds numpy arrays over all blocks:
    tokens [B, n], candidates [B, n, k], cand_logits [B, n, k] or None,
    conf [B, n] or None, lengths [B], logits [B*n, V] or None."""
    c = inp.cfg
    n, k, V = c.n_pred, c.top_k, c.V
    if z is None:
        z = orc.block_logits(inp, b)
    rep = {"block": b, "exact": 0, "near_tie": 0, "max_logit_err": 0.0, "max_conf_err": 0.0}

    if check_logits and gpu.get("logits") is not None:
        g = np.asarray(gpu["logits"][b * n:(b + 1) * n], dtype=np.float64)
        err = np.abs(g - z)
        if not np.all(np.isfinite(g)):
            raise ParityError(f"block {b}: non-finite GPU logits")
        rep["max_logit_err"] = float(err.max())
        if rep["max_logit_err"] > TOL_LOGITS:
            j, v = np.unravel_index(int(err.argmax()), err.shape)
            raise ParityError(f"block {b}: logits[{j},{v}] gpu={g[j, v]} oracle={z[j, v]}")

    tokens = np.asarray(gpu["tokens"][b])
    cands = np.asarray(gpu["candidates"][b])
    cvals = None if gpu.get("cand_logits") is None else np.asarray(gpu["cand_logits"][b])
    kk = min(V, k + 1 if k + 1 <= V else k)
    kk = max(kk, min(2, V))
    prev = int(inp.anchors[b])
    for j in range(n):
        zp = orc.step_scores(inp, z[j], prev)
        oidx, oval = orc.topk(zp, kk)
        gtok = int(tokens[j])
        if not (0 <= gtok < V):
            raise ParityError(f"block {b} slot {j}: token {gtok} out of range")
        if gtok == int(oidx[0]):
            rep["exact"] += 1
        elif V > 1 and gtok == int(oidx[1]) and float(oval[0]) - float(oval[1]) < TOL_SCORE:
            rep["near_tie"] += 1
        else:
            raise ParityError(
                f"block {b} slot {j} (prev {prev}): gpu token {gtok} (score {zp[gtok]}) vs oracle "
                f"{oidx[0]} ({oval[0]}), runner-up {oidx[1] if V > 1 else None}")
        gc = [int(x) for x in cands[j]]
        if len(set(gc)) != k:
            raise ParityError(f"block {b} slot {j}: repeated candidates {gc}")
        if gc[0] != gtok:
            raise ParityError(f"block {b} slot {j}: candidates[0]={gc[0]} != token {gtok}")
        for t in range(k):
            if not (0 <= gc[t] < V):
                raise ParityError(f"block {b} slot {j}: candidate {gc[t]} out of range")
            if abs(float(zp[gc[t]]) - float(oval[t])) >= TOL_SCORE:
                raise ParityError(f"block {b} slot {j} rank {t}: candidate {gc[t]} scores "
                                  f"{zp[gc[t]]}, oracle rank value {oval[t]}")
            lo_gap = float(oval[t - 1]) - float(oval[t]) if t > 0 else np.inf
            hi_gap = float(oval[t]) - float(oval[t + 1]) if t + 1 < kk else np.inf
            if t > 0 and lo_gap > TOL_SCORE and hi_gap > TOL_SCORE and gc[t] != int(oidx[t]):
                raise ParityError(f"block {b} slot {j} rank {t}: candidate {gc[t]} != oracle "
                                  f"{oidx[t]} though the oracle's score is isolated")
            if cvals is not None and abs(float(cvals[j, t]) - float(zp[gc[t]])) >= TOL_SCORE:
                raise ParityError(f"block {b} slot {j} rank {t}: cand_logit {cvals[j, t]} vs "
                                  f"oracle {zp[gc[t]]}")
        prev = gtok

    glen = int(gpu["lengths"][b])
    if inp.conf_w is None:
        if glen != n:
            raise ParityError(f"block {b}: length {glen} without a confidence head (want {n})")
        if gpu.get("conf") is not None and not np.all(np.asarray(gpu["conf"][b]) == 1.0):
            raise ParityError(f"block {b}: conf must be 1 without a confidence head")
    else:
        oc = orc.conf(inp, b)
        if gpu.get("conf") is not None:
            gcf = np.asarray(gpu["conf"][b], dtype=np.float32)
            err = np.abs(gcf.astype(np.float64) - oc)
            rep["max_conf_err"] = float(err.max())
            if rep["max_conf_err"] > TOL_CONF:
                raise ParityError(f"block {b}: conf {gcf} vs oracle {oc}")
            own = next((j for j in range(n) if gcf[j] < np.float32(c.p_min)), n)
            if glen != own:
                raise ParityError(f"block {b}: length {glen} but its own conf cuts at {own}")
        ok = set()
        for ell in range(n + 1):
            prefix_ok = all(float(oc[j]) >= c.p_min - TOL_CONF for j in range(ell))
            cut_ok = ell == n or float(oc[ell]) < c.p_min + TOL_CONF
            if prefix_ok and cut_ok:
                ok.add(ell)
        if glen not in ok:
            raise ParityError(f"block {b}: length {glen}, oracle conf {oc} accepts {sorted(ok)}")
    return rep


def check(orc: Oracle, inp, gpu: dict, blocks: Optional[Sequence[int]] = None,
          check_logits: bool = True) -> list:
    blocks = range(inp.cfg.B) if blocks is None else blocks
    return [check_block(orc, inp, int(b), gpu, check_logits=check_logits) for b in blocks]
