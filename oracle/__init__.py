"""CPU oracle for the DSpark proposal step (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path never touches it.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc, OpenMP over
the vocabulary); this module only marshals numpy arrays into it. What the C
code computes, and which passage of the pages each step follows, is written
at the top of ``oracle.c``.

Parity pins: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` against closed forms, library routines (numpy
argmax / lexsort / fp64 matmul), brute force at tiny vocabulary and
hand-worked examples under ``tests/golden/``. The end-to-end acceptance
behaviour of a trained drafter is parity unpinned (it needs trained weights
and a target model).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

GCC_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(src: str = SRC_PATH, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (no HIP involved)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


_LIB: Optional[ctypes.CDLL] = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p
_i = ctypes.c_int


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    lib.oracle_bf16_round.argtypes = [ctypes.c_float]
    lib.oracle_bf16_round.restype = ctypes.c_uint16
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_block_logits.argtypes = [_vp, _i, _u16p, _f32p, _i, _i, _i, _i, _i, _f64p]
    lib.oracle_block_logits.restype = _i
    lib.oracle_markov_bias.argtypes = [_u16p, _u16p, _i, _i, _i, _f64p]
    lib.oracle_markov_bias.restype = _i
    lib.oracle_step_scores.argtypes = [_f64p, _u16p, _u16p, _i, _i, _i, _f32p]
    lib.oracle_step_scores.restype = _i
    lib.oracle_argmax.argtypes = [_f32p, _i]
    lib.oracle_argmax.restype = _i
    lib.oracle_topk.argtypes = [_f32p, _i, _i, _i32p, _f32p]
    lib.oracle_topk.restype = _i
    lib.oracle_block_chain.argtypes = [_f64p, _u16p, _u16p, _i, _i, _i, _i, _i, _i32p, _i32p, _f32p]
    lib.oracle_block_chain.restype = _i
    lib.oracle_conf.argtypes = [_vp, _i, _u16p, _i, _i, _i, _i, _i]
    lib.oracle_conf.restype = ctypes.c_float
    lib.oracle_truncate.argtypes = [_f32p, _i, ctypes.c_float]
    lib.oracle_truncate.restype = _i
    lib.oracle_propose_block.argtypes = [_vp, _i, _u16p, _f32p, _u16p, _u16p, _u16p, _i32p,
                                         _i, _i, _i, _i, _i, _i, ctypes.c_float, _i, _f64p,
                                         _i32p, _i32p, _f32p, _f32p, _i32p]
    lib.oracle_propose_block.restype = _i
    lib.oracle_block_chain_d2t.argtypes = [_f64p, _u16p, _u16p, _i64p, _i, _i, _i, _i, _i, _i,
                                           _i32p, _i32p, _f32p]
    lib.oracle_block_chain_d2t.restype = _i
    lib.oracle_propose_block_d2t.argtypes = [_vp, _i, _u16p, _i64p, _u16p, _u16p, _u16p, _i32p,
                                             _i, _i, _i, _i, _i, _i, _i, ctypes.c_float, _i,
                                             _f64p, _i32p, _i32p, _f32p, _f32p, _i32p]
    lib.oracle_propose_block_d2t.restype = _i
    lib.oracle_propose_block_gated.argtypes = [_vp, _i, _u16p, _f32p, _u16p, _u16p, _u16p, _i32p,
                                               _i, _i, _i, _i, _i, _i, _i, ctypes.c_float, _i,
                                               _f64p, _i32p, _i32p, _f32p, _f32p, _i32p]
    lib.oracle_propose_block_gated.restype = _i
    lib.oracle_verify.argtypes = [_i32p, _i32p, _i32p, _i, _i, _i, _i, _i32p, _i64p]
    lib.oracle_verify.restype = _i
    lib.oracle_f16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_value.restype = ctypes.c_double
    lib.oracle_q4_dequant_row.argtypes = [_u8p, _i, ctypes.c_long, _f64p]
    lib.oracle_q4_dequant_row.restype = _i
    lib.oracle_block_logits_q4.argtypes = [_vp, _i, _u8p, _f32p, _i, _i, _i, _i, _i, _f64p]
    lib.oracle_block_logits_q4.restype = _i
    lib.oracle_propose_block_q4.argtypes = [_vp, _i, _u8p, _f32p, _u16p, _u16p, _u16p, _i32p,
                                            _i, _i, _i, _i, _i, _i, ctypes.c_float, _i, _f64p,
                                            _i32p, _i32p, _f32p, _f32p, _i32p]
    lib.oracle_propose_block_q4.restype = _i
    return lib


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liboracle.so, compiling it first if it is missing or older than its source.
    With DSPARK_ORACLE_LIB set, the default library is that prebuilt file
    instead (the test suite's sanitizer build)."""
    global _LIB
    if path == LIB_PATH and _LIB is not None:
        return _LIB
    override = os.environ.get("DSPARK_ORACLE_LIB")
    if path == LIB_PATH and override:
        _LIB = _declare(ctypes.CDLL(override))
        return _LIB
    if path == LIB_PATH and (not os.path.exists(path)
                             or os.path.getmtime(path) < os.path.getmtime(SRC_PATH)):
        build(out=path)
    elif not os.path.exists(path):
        build(out=path)
    lib = _declare(ctypes.CDLL(path))
    if path == LIB_PATH:
        _LIB = lib
    return lib


def _p(a: Optional[np.ndarray], t):
    if a is None:
        return ctypes.cast(None, t)
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(t)


class Oracle:
    """Thin numpy front-end over one loaded oracle library."""

    def __init__(self, lib: Optional[ctypes.CDLL] = None):
        self.lib = lib if lib is not None else load()

    # --- scalar helpers ---------------------------------------------------
    def bf16_round(self, x: float) -> int:
        return int(self.lib.oracle_bf16_round(ctypes.c_float(x)))

    def bf16_value(self, bits: int) -> float:
        return float(self.lib.oracle_bf16_value(ctypes.c_uint16(bits)))

    # --- method steps -----------------------------------------------------
    def block_logits(self, inp, b: int) -> np.ndarray:
        if hasattr(inp, "lm_head_q4"):
            return self.block_logits_q4(inp, b)
        c = inp.cfg
        z = np.empty((c.n_pred, c.V), dtype=np.float64)
        st = self.lib.oracle_block_logits(
            inp.hidden.ctypes.data, int(inp.hidden_f32), _p(inp.lm_head, _u16p),
            _p(inp.lm_head_bias, _f32p), c.L, c.H, c.V, c.i_first_pred, b, _p(z, _f64p))
        if st != 0:
            raise ValueError("oracle_block_logits rejected its arguments")
        return z

    def markov_bias(self, inp, prev: int) -> np.ndarray:
        c = inp.cfg
        m = np.empty(c.V, dtype=np.float64)
        st = self.lib.oracle_markov_bias(_p(inp.markov_w1, _u16p), _p(inp.markov_w2, _u16p),
                                         c.V, c.r, int(prev), _p(m, _f64p))
        if st != 0:
            raise ValueError("oracle_markov_bias rejected its arguments")
        return m

    def step_scores(self, inp, z_row: np.ndarray, prev: int) -> np.ndarray:
        c = inp.cfg
        z_row = np.ascontiguousarray(z_row, dtype=np.float64)
        zp = np.empty(c.V, dtype=np.float32)
        st = self.lib.oracle_step_scores(_p(z_row, _f64p), _p(inp.markov_w1, _u16p),
                                         _p(inp.markov_w2, _u16p), c.V, c.r, int(prev),
                                         _p(zp, _f32p))
        if st != 0:
            raise ValueError("oracle_step_scores rejected its arguments")
        return zp

    def argmax(self, zp: np.ndarray) -> int:
        zp = np.ascontiguousarray(zp, dtype=np.float32)
        return int(self.lib.oracle_argmax(_p(zp, _f32p), zp.size))

    def topk(self, zp: np.ndarray, k: int):
        zp = np.ascontiguousarray(zp, dtype=np.float32)
        idx = np.empty(k, dtype=np.int32)
        val = np.empty(k, dtype=np.float32)
        st = self.lib.oracle_topk(_p(zp, _f32p), zp.size, k, _p(idx, _i32p), _p(val, _f32p))
        if st != 0:
            raise ValueError("oracle_topk rejected its arguments")
        return idx, val

    def block_chain(self, inp, z: np.ndarray, anchor: int, top_k: Optional[int] = None):
        c = inp.cfg
        k = c.top_k if top_k is None else top_k
        z = np.ascontiguousarray(z, dtype=np.float64)
        n = z.shape[0]
        tokens = np.empty(n, dtype=np.int32)
        cand = np.empty((n, k), dtype=np.int32)
        cval = np.empty((n, k), dtype=np.float32)
        st = self.lib.oracle_block_chain(_p(z, _f64p), _p(inp.markov_w1, _u16p),
                                         _p(inp.markov_w2, _u16p), c.V, c.r, int(anchor), n, k,
                                         _p(tokens, _i32p), _p(cand, _i32p), _p(cval, _f32p))
        if st != 0:
            raise ValueError("oracle_block_chain rejected its arguments")
        return tokens, cand, cval

    def conf(self, inp, b: int) -> np.ndarray:
        c = inp.cfg
        out = np.empty(c.n_pred, dtype=np.float32)
        for j in range(c.n_pred):
            out[j] = self.lib.oracle_conf(inp.hidden.ctypes.data, int(inp.hidden_f32),
                                          _p(inp.conf_w, _u16p), c.L, c.H, c.i_first_pred, b, j)
        return out

    def truncate(self, conf: np.ndarray, p_min: float) -> int:
        conf = np.ascontiguousarray(conf, dtype=np.float32)
        return int(self.lib.oracle_truncate(_p(conf, _f32p), conf.size, ctypes.c_float(p_min)))

    def propose_block(self, inp, b: int, keep_logits: bool = True) -> dict:
        c = inp.cfg
        n, k = c.n_pred, c.top_k
        z = np.empty((n, c.V), dtype=np.float64) if keep_logits else None
        tokens = np.empty(n, dtype=np.int32)
        cand = np.empty((n, k), dtype=np.int32)
        cval = np.empty((n, k), dtype=np.float32)
        conf = np.empty(n, dtype=np.float32)
        length = np.zeros(1, dtype=np.int32)
        st = self.lib.oracle_propose_block(
            inp.hidden.ctypes.data, int(inp.hidden_f32), _p(inp.lm_head, _u16p),
            _p(inp.lm_head_bias, _f32p), _p(inp.markov_w1, _u16p), _p(inp.markov_w2, _u16p),
            _p(inp.conf_w, _u16p), _p(inp.anchors, _i32p), c.L, c.H, c.V, c.r,
            c.i_first_pred, k, ctypes.c_float(c.p_min), b,
            _p(z, _f64p) if z is not None else ctypes.cast(None, _f64p),
            _p(tokens, _i32p), _p(cand, _i32p), _p(cval, _f32p), _p(conf, _f32p),
            _p(length, _i32p))
        if st != 0:
            raise ValueError("oracle_propose_block rejected its arguments")
        return {"logits": z, "tokens": tokens, "candidates": cand, "cand_logits": cval,
                "conf": conf, "length": int(length[0])}

    def propose_block_gated(self, inp, b: int, p_min: float, kb: int,
                            keep_logits: bool = True) -> dict:
        """Block b under the adaptive gate with its own threshold and kb candidates."""
        c = inp.cfg
        n, k = c.n_pred, c.top_k
        z = np.empty((n, c.V), dtype=np.float64) if keep_logits else None
        tokens = np.empty(n, dtype=np.int32)
        cand = np.empty((n, k), dtype=np.int32)
        cval = np.empty((n, k), dtype=np.float32)
        conf = np.empty(n, dtype=np.float32)
        length = np.zeros(1, dtype=np.int32)
        st = self.lib.oracle_propose_block_gated(
            inp.hidden.ctypes.data, int(inp.hidden_f32), _p(inp.lm_head, _u16p),
            _p(inp.lm_head_bias, _f32p), _p(inp.markov_w1, _u16p), _p(inp.markov_w2, _u16p),
            _p(inp.conf_w, _u16p), _p(inp.anchors, _i32p), c.L, c.H, c.V, c.r,
            c.i_first_pred, k, int(kb), ctypes.c_float(p_min), b,
            _p(z, _f64p) if z is not None else ctypes.cast(None, _f64p),
            _p(tokens, _i32p), _p(cand, _i32p), _p(cval, _f32p), _p(conf, _f32p),
            _p(length, _i32p))
        if st != 0:
            raise ValueError("oracle_propose_block_gated rejected its arguments")
        return {"logits": z, "tokens": tokens, "candidates": cand, "cand_logits": cval,
                "conf": conf, "length": int(length[0])}

    def verify(self, candidates: np.ndarray, lengths: np.ndarray, target: np.ndarray,
               lattice: bool = False):
        """Accepted slots per block and (sum accepted, sum clamped lengths)."""
        cand = np.ascontiguousarray(candidates, dtype=np.int32)
        B, n, k = cand.shape
        lengths = np.ascontiguousarray(lengths, dtype=np.int32)
        target = np.ascontiguousarray(target, dtype=np.int32)
        acc = np.empty(B, dtype=np.int32)
        tot = np.zeros(2, dtype=np.int64)
        st = self.lib.oracle_verify(_p(cand, _i32p), _p(lengths, _i32p), _p(target, _i32p), B, n, k,
                                    k if lattice else 1, _p(acc, _i32p), _p(tot, _i64p))
        if st != 0:
            raise ValueError("oracle_verify rejected its arguments")
        return acc, (int(tot[0]), int(tot[1]))

    def propose_block_d2t(self, red, b: int, keep_logits: bool = True) -> dict:
        """Block b of a reduced-vocabulary input (``synthetic.ReducedInputs``)."""
        c = red.cfg
        n, k, D = c.n_pred, c.top_k, red.D
        z = np.empty((n, D), dtype=np.float64) if keep_logits else None
        tokens = np.empty(n, dtype=np.int32)
        cand = np.empty((n, k), dtype=np.int32)
        cval = np.empty((n, k), dtype=np.float32)
        conf = np.empty(n, dtype=np.float32)
        length = np.zeros(1, dtype=np.int32)
        st = self.lib.oracle_propose_block_d2t(
            red.hidden.ctypes.data, int(red.hidden_f32), _p(red.lm_head, _u16p), _p(red.d2t, _i64p),
            _p(red.markov_w1, _u16p), _p(red.markov_w2, _u16p), _p(red.conf_w, _u16p),
            _p(red.anchors, _i32p), c.L, c.H, c.V, D, c.r, c.i_first_pred, k,
            ctypes.c_float(c.p_min), b,
            _p(z, _f64p) if z is not None else ctypes.cast(None, _f64p),
            _p(tokens, _i32p), _p(cand, _i32p), _p(cval, _f32p), _p(conf, _f32p),
            _p(length, _i32p))
        if st != 0:
            raise ValueError("oracle_propose_block_d2t rejected its arguments")
        return {"logits": z, "tokens": tokens, "candidates": cand, "cand_logits": cval,
                "conf": conf, "length": int(length[0])}

    # --- quantized head (q4) -----------------------------------------------
    def f16_value(self, bits: int) -> float:
        return float(self.lib.oracle_f16_value(ctypes.c_uint16(bits)))

    def q4_dequant_row(self, q4: np.ndarray, H: int, v: int) -> np.ndarray:
        """Row v of a q4 head (uint8 [V, H/32*18] GGUF blocks) as exact float64."""
        q4 = np.ascontiguousarray(q4, dtype=np.uint8)
        w = np.empty(H, dtype=np.float64)
        st = self.lib.oracle_q4_dequant_row(_p(q4, _u8p), H, int(v), _p(w, _f64p))
        if st != 0:
            raise ValueError("oracle_q4_dequant_row rejected its arguments")
        return w

    def block_logits_q4(self, qinp, b: int) -> np.ndarray:
        """Projections of block b through the q4 head of ``qinp`` (synthetic.Q4Inputs)."""
        c = qinp.cfg
        z = np.empty((c.n_pred, c.V), dtype=np.float64)
        st = self.lib.oracle_block_logits_q4(
            qinp.hidden.ctypes.data, int(qinp.hidden_f32), _p(qinp.lm_head_q4, _u8p),
            _p(qinp.lm_head_bias, _f32p), c.L, c.H, c.V, c.i_first_pred, b, _p(z, _f64p))
        if st != 0:
            raise ValueError("oracle_block_logits_q4 rejected its arguments")
        return z

    def propose_block_q4(self, qinp, b: int, keep_logits: bool = True) -> dict:
        c = qinp.cfg
        n, k = c.n_pred, c.top_k
        z = np.empty((n, c.V), dtype=np.float64) if keep_logits else None
        tokens = np.empty(n, dtype=np.int32)
        cand = np.empty((n, k), dtype=np.int32)
        cval = np.empty((n, k), dtype=np.float32)
        conf = np.empty(n, dtype=np.float32)
        length = np.zeros(1, dtype=np.int32)
        st = self.lib.oracle_propose_block_q4(
            qinp.hidden.ctypes.data, int(qinp.hidden_f32), _p(qinp.lm_head_q4, _u8p),
            _p(qinp.lm_head_bias, _f32p), _p(qinp.markov_w1, _u16p), _p(qinp.markov_w2, _u16p),
            _p(qinp.conf_w, _u16p), _p(qinp.anchors, _i32p), c.L, c.H, c.V, c.r,
            c.i_first_pred, k, ctypes.c_float(c.p_min), b,
            _p(z, _f64p) if z is not None else ctypes.cast(None, _f64p),
            _p(tokens, _i32p), _p(cand, _i32p), _p(cval, _f32p), _p(conf, _f32p),
            _p(length, _i32p))
        if st != 0:
            raise ValueError("oracle_propose_block_q4 rejected its arguments")
        return {"logits": z, "tokens": tokens, "candidates": cand, "cand_logits": cval,
                "conf": conf, "length": int(length[0])}

    def propose(self, inp, blocks: Optional[Sequence[int]] = None, keep_logits: bool = True) -> dict:
        """Oracle outputs for the listed blocks (all blocks by default), stacked
        (a synthetic.Q4Inputs goes through the q4 head)."""
        c = inp.cfg
        blocks = list(range(c.B)) if blocks is None else list(blocks)
        one = self.propose_block_q4 if hasattr(inp, "lm_head_q4") else self.propose_block
        outs = [one(inp, b, keep_logits) for b in blocks]
        res = {
            "blocks": np.array(blocks, dtype=np.int64),
            "tokens": np.stack([o["tokens"] for o in outs]),
            "candidates": np.stack([o["candidates"] for o in outs]),
            "cand_logits": np.stack([o["cand_logits"] for o in outs]),
            "conf": np.stack([o["conf"] for o in outs]),
            "lengths": np.array([o["length"] for o in outs], dtype=np.int32),
        }
        if keep_logits:
            res["logits"] = np.stack([o["logits"] for o in outs])
        return res
