"""Seeded synthetic workloads at the shapes the DSpark pages describe.

Recipe (every tensor has its own random stream, so shapes that agree across
workloads share identical weights, and the draw order does not matter):

* stream(name, chunk) = numpy.random.default_rng(SeedSequence(seed,
  spawn_key=(TENSOR_CODE[name], chunk))); tensors with more than one row are
  drawn in chunks of ``CHUNK_ROWS`` rows, chunk c from stream(name, c).
* Gaussian draws are float32 ``standard_normal`` scaled by the std, then
  rounded to bf16 with round-to-nearest-even. N(0, s) always means std s.
* hidden ~ N(0, 1)                       [B, L, H] (float32 kept as is when the
                                           workload feeds fp32 hidden states)
* lm_head ~ N(0, 1/sqrt(H))              [V, H]
* markov_w1, markov_w2 ~ N(0, w_std)     [V, r]
* conf_w ~ N(0, 1/sqrt(H))               [H]
* anchors uniform in [0, V); with ``exclude_mask`` they are drawn in [0, V-1)
  and every value >= MASK_TOKEN_ID is shifted up by one, so the Qwen3.8 mask
  id never appears.
* reduced draft vocabulary (``reachable`` = D): the first D entries of a
  seeded permutation of range(V) are the reachable rows. Every other row of
  lm_head and markov_w2 is zero and carries an lm_head bias of -1e9; the
  reachable rows carry bias 0. markov_w1 is left untouched.
* q4 head (``quantize_q4``): the same lm_head requantized to 4-bit blocks of
  32 weights along H (the block format is described at ``Q4Inputs``). Mode
  "round": d = binary16(max |w| / 8) per block and code q = clip(rint(w / d)
  + 8, 0, 15) (code 8 where d = 0), in float64 from the bf16 weights. Mode
  "random": codes uniform in [0, 16) and d = binary16(N(0, 1/(8 sqrt(H))))
  from stream("q4", chunk), with every 97th block's scale set to 0, every
  89th to a subnormal binary16 (2^-20) and every 83rd to its negative. The
  requantizer is input preparation (the drafter ships already quantized);
  the proposal step only decodes.
* confidence trend (``conf_trend``): conf_w is rescaled to norm 0.5 and each
  prediction slot j of every block is shifted along conf_w so that
  conf_w . hidden = logit(p_j) + (conf_w . z), with p_j falling linearly from
  0.9 at the first prediction slot to 0.3 at the last, z ~ N(0, 1).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

MASK_TOKEN_ID = 248077  # Qwen3.8 DSpark drafter mask id (lucebox PR #626 description)

CHUNK_ROWS = 4096
TENSOR_CODE = {
    "hidden": 1,
    "lm_head": 2,
    "markov_w1": 3,
    "markov_w2": 4,
    "conf_w": 5,
    "anchors": 6,
    "reachable": 7,
    "q4": 8,
}

ANCHOR_FIRST = "anchor_first"
BONUS_ANCHOR = "bonus_anchor"


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    L: int
    H: int
    V: int
    r: int
    top_k: int
    layout: str = ANCHOR_FIRST
    hidden_f32: bool = False
    w_std: float = 0.05
    conf: bool = False
    p_min: float = 0.0
    exclude_mask: bool = False
    reachable: Optional[int] = None
    conf_trend: bool = False
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def i_first_pred(self) -> int:
        return 1 if self.layout == BONUS_ANCHOR else 0

    @property
    def n_pred(self) -> int:
        return self.L - self.i_first_pred

    @property
    def drafted_tokens(self) -> int:
        return self.B * self.n_pred


CONFIGS = {
    "tiny": Config(
        "tiny", B=1, L=4, H=64, V=512, r=8, top_k=1, hidden_f32=True, w_std=0.1,
        notes="tiny oracle case, fp32 hidden, no truncation"),
    "qwen3_8b": Config(
        "qwen3_8b", B=1, L=16, H=4096, V=151936, r=64, top_k=1, conf=True, p_min=0.0,
        notes="Qwen3-8B-shaped draft, confidence head present, gate off"),
    "qwen38_27b_tree": Config(
        "qwen38_27b_tree", B=8, L=16, H=5120, V=248320, r=128, top_k=4, exclude_mask=True,
        notes="Qwen3.8-27B-shaped tree proposal, top-4 lattice, no confidence head"),
    "gemma4_26b_a4b": Config(
        "gemma4_26b_a4b", B=4, L=7, H=2816, V=262144, r=64, top_k=1, layout=BONUS_ANCHOR,
        conf=True, p_min=0.5, reachable=32768, conf_trend=True,
        notes="Gemma-4-26B-A4B speculators-shaped draft, 1+6 bonus-anchor block, reduced vocab"),
    "qwen38_27b_throughput": Config(
        "qwen38_27b_throughput", B=64, L=16, H=5120, V=248320, r=128, top_k=4, conf=True,
        p_min=0.3, exclude_mask=True,
        notes="throughput case at the Qwen3.8-27B shape, top-4 lattice, p_min 0.3"),
}


@dataclass
class Inputs:
    cfg: Config
    hidden: np.ndarray            # uint16 bf16 bits [B, L, H], or float32 [B, L, H]
    lm_head: np.ndarray           # uint16 bf16 bits [V, H]
    lm_head_bias: Optional[np.ndarray]  # float32 [V] or None
    markov_w1: Optional[np.ndarray]     # uint16 bf16 bits [V, r] or None (r == 0)
    markov_w2: Optional[np.ndarray]     # uint16 bf16 bits [V, r] or None (r == 0)
    conf_w: Optional[np.ndarray]        # uint16 bf16 bits [H] or None
    anchors: np.ndarray           # int32 [B]
    reachable: Optional[np.ndarray] = None  # int64 sorted reachable ids, or None

    @property
    def hidden_f32(self) -> bool:
        return self.hidden.dtype == np.float32


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    u += np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))
    out = (u >> 16).astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _stream(seed: int, name: str, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(TENSOR_CODE[name], chunk)))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _gauss_bf16(seed: int, name: str, rows: int, cols: int, std: float) -> np.ndarray:
    """[rows, cols] bf16 bits of N(0, std), drawn chunk by chunk in parallel."""
    out = np.empty((rows, cols), dtype=np.uint16)
    n_chunks = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS
    s = np.float32(std)

    def fill(c: int) -> None:
        r0 = c * CHUNK_ROWS
        r1 = min(rows, r0 + CHUNK_ROWS)
        x = _stream(seed, name, c).standard_normal((r1 - r0, cols), dtype=np.float32)
        x *= s
        out[r0:r1] = f32_to_bf16_bits(x)

    if n_chunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def _gauss_f32(seed: int, name: str, rows: int, cols: int, std: float) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32)
    for c in range((rows + CHUNK_ROWS - 1) // CHUNK_ROWS):
        r0 = c * CHUNK_ROWS
        r1 = min(rows, r0 + CHUNK_ROWS)
        out[r0:r1] = _stream(seed, name, c).standard_normal((r1 - r0, cols), dtype=np.float32)
        out[r0:r1] *= np.float32(std)
    return out


_WEIGHT_CACHE: dict = {}


def _weights(cfg: Config):
    """lm_head, markov_w1, markov_w2, conf_w draws; cached per (seed, shape, std)."""
    key = (cfg.seed, cfg.V, cfg.H, cfg.r, cfg.w_std)
    hit = _WEIGHT_CACHE.get(key)
    if hit is not None:
        return hit
    lm = _gauss_bf16(cfg.seed, "lm_head", cfg.V, cfg.H, 1.0 / math.sqrt(cfg.H))
    if cfg.r > 0:
        w1 = _gauss_bf16(cfg.seed, "markov_w1", cfg.V, cfg.r, cfg.w_std)
        w2 = _gauss_bf16(cfg.seed, "markov_w2", cfg.V, cfg.r, cfg.w_std)
    else:
        w1 = w2 = None
    cw = _gauss_f32(cfg.seed, "conf_w", 1, cfg.H, 1.0 / math.sqrt(cfg.H))[0]
    hit = (lm, w1, w2, cw)
    # keep only the most recent large weight set in memory
    if lm.nbytes > (256 << 20):
        for k in [k for k, v in _WEIGHT_CACHE.items() if v[0].nbytes > (256 << 20)]:
            del _WEIGHT_CACHE[k]
    _WEIGHT_CACHE[key] = hit
    return hit


def make_inputs(cfg: Config) -> Inputs:
    B, L, H, V = cfg.B, cfg.L, cfg.H, cfg.V
    lm, w1, w2, cw_f32 = _weights(cfg)

    hid = _gauss_f32(cfg.seed, "hidden", B * L, H, 1.0).reshape(B, L, H)

    bias = None
    reachable = None
    if cfg.reachable is not None:
        perm = _stream(cfg.seed, "reachable").permutation(V)
        reachable = np.sort(perm[: cfg.reachable])
        keep = np.zeros(V, dtype=bool)
        keep[reachable] = True
        lm = lm.copy()
        lm[~keep] = 0
        if w2 is not None:
            w2 = w2.copy()
            w2[~keep] = 0
        bias = np.where(keep, np.float32(0.0), np.float32(-1e9)).astype(np.float32)

    conf_w = None
    if cfg.conf:
        if cfg.conf_trend:
            c = cw_f32 * np.float32(0.5 / float(np.linalg.norm(cw_f32.astype(np.float64))))
            conf_w = f32_to_bf16_bits(c)
            c_hat = bf16_bits_to_f32(conf_w).astype(np.float64)
            n = cfg.n_pred
            for j in range(n):
                p = 0.9 - 0.6 * (j / (n - 1) if n > 1 else 0.0)
                shift = math.log(p / (1.0 - p)) * c_hat / float(c_hat @ c_hat)
                slot = cfg.i_first_pred + j
                hid[:, slot, :] = (hid[:, slot, :].astype(np.float64) + shift).astype(np.float32)
        else:
            conf_w = f32_to_bf16_bits(cw_f32)

    hidden = hid if cfg.hidden_f32 else f32_to_bf16_bits(hid)

    ag = _stream(cfg.seed, "anchors")
    if cfg.exclude_mask and V > MASK_TOKEN_ID:
        anchors = ag.integers(0, V - 1, size=B, dtype=np.int64)
        anchors = np.where(anchors >= MASK_TOKEN_ID, anchors + 1, anchors)
    else:
        anchors = ag.integers(0, V, size=B, dtype=np.int64)

    return Inputs(cfg=cfg, hidden=np.ascontiguousarray(hidden), lm_head=lm, lm_head_bias=bias,
                  markov_w1=w1, markov_w2=w2, conf_w=conf_w,
                  anchors=anchors.astype(np.int32), reachable=reachable)


def make_small(B: int, L: int, H: int, V: int, r: int, top_k: int = 1, *,
               layout: str = ANCHOR_FIRST, hidden_f32: bool = False, w_std: float = 0.1,
               conf: bool = False, p_min: float = 0.0, reachable: Optional[int] = None,
               conf_trend: bool = False, seed: int = 0) -> Inputs:
    """A workload of arbitrary (small) shape with the same recipe."""
    cfg = Config(f"small_B{B}_L{L}_H{H}_V{V}_r{r}_k{top_k}_s{seed}", B=B, L=L, H=H, V=V, r=r,
                 top_k=top_k, layout=layout, hidden_f32=hidden_f32, w_std=w_std, conf=conf,
                 p_min=p_min, reachable=reachable, conf_trend=conf_trend, seed=seed)
    return make_inputs(cfg)


def with_config(inp: Inputs, **changes) -> Inputs:
    """Same tensors, different scalar parameters (top_k, p_min, ...)."""
    return replace(inp, cfg=replace(inp.cfg, **changes))


@dataclass
class ReducedInputs:
    """The same draft in the reduced-vocabulary form: the draft head has D rows,
    one per entry of d2t (int64 absolute target ids, increasing); markov_w2 has
    the same D rows; markov_w1 keeps its V target rows (it is indexed by the
    previous token, a target id); no bias."""
    cfg: Config                   # sizes of the target vocabulary (cfg.V)
    hidden: np.ndarray
    lm_head: np.ndarray           # uint16 bf16 bits [D, H]
    d2t: np.ndarray               # int64 [D]
    markov_w1: Optional[np.ndarray]     # uint16 [V, r] or None
    markov_w2: Optional[np.ndarray]     # uint16 [D, r] or None
    conf_w: Optional[np.ndarray]
    anchors: np.ndarray

    @property
    def D(self) -> int:
        return int(self.d2t.shape[0])

    @property
    def hidden_f32(self) -> bool:
        return self.hidden.dtype == np.float32


def reduce_vocab(inp: Inputs) -> ReducedInputs:
    """The reduced form of an input whose vocabulary was expanded: d2t lists the
    reachable target ids, and the head and markov_w2 keep only their rows (a row
    selection; the expanded form has zero rows and a -1e9 bias elsewhere)."""
    if inp.reachable is None:
        raise ValueError("the input has no reduced vocabulary")
    d2t = np.ascontiguousarray(inp.reachable, dtype=np.int64)
    w2 = None if inp.markov_w2 is None else np.ascontiguousarray(inp.markov_w2[d2t])
    return ReducedInputs(cfg=inp.cfg, hidden=inp.hidden, lm_head=np.ascontiguousarray(inp.lm_head[d2t]),
                         d2t=d2t, markov_w1=inp.markov_w1, markov_w2=w2, conf_w=inp.conf_w,
                         anchors=inp.anchors)


# ---------------------------------------------------------------------------
# 4-bit head
# ---------------------------------------------------------------------------

Q4_BLOCK = 32
Q4_BLOCK_BYTES = 18


@dataclass
class Q4Inputs:
    """The same draft with lm_head in a 4-bit block format (GGUF's plain
    4-bit type): each row is H/32 blocks of 18 bytes, a binary16 scale d (low
    byte first) and 16 code bytes; code byte j holds element j of the block
    in its low nibble and element j + 16 in its high nibble, and an element
    with code q is worth d * (q - 8)."""
    cfg: Config
    hidden: np.ndarray
    lm_head_q4: np.ndarray        # uint8 [V, H/32 * 18]
    lm_head_bias: Optional[np.ndarray]
    markov_w1: Optional[np.ndarray]
    markov_w2: Optional[np.ndarray]
    conf_w: Optional[np.ndarray]
    anchors: np.ndarray
    reachable: Optional[np.ndarray] = None

    @property
    def hidden_f32(self) -> bool:
        return self.hidden.dtype == np.float32


def q4_blocks(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """GGUF 4-bit blocks from codes uint8 [V, H] (values 0..15) and binary16
    scales [V, H/32]: uint8 [V, H/32 * 18]."""
    V, H = codes.shape
    nb = H // Q4_BLOCK
    c = np.asarray(codes, dtype=np.uint8).reshape(V, nb, Q4_BLOCK)
    qs = (c[:, :, :16] | (c[:, :, 16:] << 4)).astype(np.uint8)
    sb = np.ascontiguousarray(np.asarray(scales, dtype=np.float16)).view(np.uint8).reshape(V, nb, 2)
    return np.ascontiguousarray(np.concatenate([sb, qs], axis=2).reshape(V, nb * Q4_BLOCK_BYTES))


def _q4_round_rows(w_bits: np.ndarray) -> np.ndarray:
    """Round-to-nearest requantization of bf16 rows [n, H] into q4 blocks."""
    n, H = w_bits.shape
    w = bf16_bits_to_f32(w_bits).astype(np.float64).reshape(n, H // Q4_BLOCK, Q4_BLOCK)
    d = (np.abs(w).max(axis=2) / 8.0).astype(np.float16)
    d64 = d.astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(d64 != 0.0, np.clip(np.rint(w / np.where(d64 != 0.0, d64, 1.0)) + 8, 0, 15), 8)
    return q4_blocks(q.astype(np.uint8).reshape(n, H), d)


def _q4_random_rows(seed: int, chunk: int, n: int, H: int, row0: int) -> np.ndarray:
    g = _stream(seed, "q4", chunk)
    nb = H // Q4_BLOCK
    codes = g.integers(0, 16, size=(n, H), dtype=np.uint8)
    d = (g.standard_normal((n, nb)) / (8.0 * math.sqrt(H))).astype(np.float16)
    idx = (row0 + np.arange(n))[:, None] * nb + np.arange(nb)[None, :]
    d[idx % 83 == 0] = -d[idx % 83 == 0]
    d[idx % 89 == 0] = np.float16(2.0 ** -20)
    d[idx % 97 == 0] = np.float16(0.0)
    return q4_blocks(codes, d)


_Q4_CACHE: dict = {}


def quantize_q4(inp: Inputs, mode: str = "round") -> Q4Inputs:
    """``inp`` with its lm_head as q4 blocks (see the module recipe)."""
    c = inp.cfg
    if c.H % Q4_BLOCK != 0:
        raise ValueError("the 4-bit head needs H to be a multiple of 32")
    key = (c.seed, c.V, c.H, mode, c.reachable, inp.lm_head.ctypes.data if mode == "round" else 0)
    q4 = _Q4_CACHE.get(key)
    if q4 is None:
        V, H = c.V, c.H
        q4 = np.empty((V, H // Q4_BLOCK * Q4_BLOCK_BYTES), dtype=np.uint8)
        n_chunks = (V + CHUNK_ROWS - 1) // CHUNK_ROWS

        def fill(ch: int) -> None:
            r0 = ch * CHUNK_ROWS
            r1 = min(V, r0 + CHUNK_ROWS)
            if mode == "round":
                q4[r0:r1] = _q4_round_rows(inp.lm_head[r0:r1])
            elif mode == "random":
                q4[r0:r1] = _q4_random_rows(c.seed, ch, r1 - r0, H, r0)
            else:
                raise ValueError(f"unknown q4 mode {mode}")

        if n_chunks == 1:
            fill(0)
        else:
            with ThreadPoolExecutor(_threads()) as ex:
                list(ex.map(fill, range(n_chunks)))
        if mode == "random" and inp.reachable is not None:
            # unreachable rows stay zero weights (scale 0, code 8), as in the bf16 form
            keep = np.zeros(V, dtype=bool)
            keep[inp.reachable] = True
            zero_row = q4_blocks(np.full((1, H), 8, np.uint8), np.zeros((1, H // Q4_BLOCK), np.float16))
            q4[~keep] = zero_row
        if q4.nbytes > (256 << 20):
            for k in [k for k, v in _Q4_CACHE.items() if v.nbytes > (256 << 20)]:
                del _Q4_CACHE[k]
        _Q4_CACHE[key] = q4
    return Q4Inputs(cfg=c, hidden=inp.hidden, lm_head_q4=q4, lm_head_bias=inp.lm_head_bias,
                    markov_w1=inp.markov_w1, markov_w2=inp.markov_w2, conf_w=inp.conf_w,
                    anchors=inp.anchors, reachable=inp.reachable)
