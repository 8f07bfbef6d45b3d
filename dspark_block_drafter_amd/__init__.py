"""DSpark drafter proposal step on MI355X (gfx950).

Python binding of ``libdspark.so`` (C ABI declared in ``include/dspark.h``).
This module only marshals arguments: it turns torch tensors into device
pointers and the current HIP stream into a handle, and raises on a non-OK
status. Every step of the computation runs in the library's HIP kernels;
there is no Python or CPU fallback, and importing the binding fails loudly
when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# DSPARK_LIBRARY names another build of the library (the test suite's
# sanitizer build); by default the one built in the package directory.
LIB_PATH = os.environ.get("DSPARK_LIBRARY") or os.path.join(HERE, "libdspark.so")

ANCHOR_FIRST = 0
BONUS_ANCHOR = 1
LAYOUTS = {"anchor_first": ANCHOR_FIRST, "bonus_anchor": BONUS_ANCHOR,
           ANCHOR_FIRST: ANCHOR_FIRST, BONUS_ANCHOR: BONUS_ANCHOR}
HIDDEN_BF16 = 0
HIDDEN_F32 = 1

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_WORKSPACE = -3
ERR_HIP = -4
ERR_SCRATCH = -5
NOALLOC_SCRATCH_BYTES = 64 << 20

FLAG_BAD_ANCHOR = 1
FLAG_INTERNAL = 2
FLAG_BAD_D2T = 4

MAX_TOP_K = 16
MAX_RANK = 256

EXPORTS = ("dspark_workspace_bytes", "dspark_propose", "dspark_propose_marked",
           "dspark_propose_noalloc", "dspark_logits", "dspark_chain",
           "dspark_propose_d2t", "dspark_propose_adaptive", "dspark_q4_packed_bytes",
           "dspark_q4_pack", "dspark_q4_workspace_bytes", "dspark_logits_q4", "dspark_propose_q4",
           "dspark_verify", "dspark_read_flags", "dspark_status_string")


class DsparkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_LIB: Optional[ctypes.CDLL] = None
_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdspark.so (built by ``__graft_entry__.build()``); never builds or falls back."""
    global _LIB
    if _LIB is not None and path == LIB_PATH:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; "
                          f"g.build()'` (hipcc, gfx950); there is no fallback path")
    lib = ctypes.CDLL(path)
    lib.dspark_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
    lib.dspark_workspace_bytes.restype = _sz
    lib.dspark_propose.argtypes = [_vp, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _i, _i, _i, _i, _i, _i, _i, _f,
                                   _vp, _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.dspark_propose.restype = _i
    lib.dspark_propose_marked.argtypes = lib.dspark_propose.argtypes + [_vp, _vp, _vp]
    lib.dspark_propose_marked.restype = _i
    lib.dspark_propose_noalloc.argtypes = [_vp, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                           _i, _i, _i, _i, _i, _i, _i, _f,
                                           _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.dspark_propose_noalloc.restype = _i
    lib.dspark_logits.argtypes = [_vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp]
    lib.dspark_logits.restype = _i
    lib.dspark_chain.argtypes = [_vp, _vp, _i, _vp, _vp, _vp, _vp,
                                 _i, _i, _i, _i, _i, _i, _i, _f,
                                 _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.dspark_chain.restype = _i
    lib.dspark_propose_d2t.argtypes = [_vp, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _i, _i, _i, _i, _i, _i, _i, _i, _f,
                                       _vp, _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.dspark_propose_d2t.restype = _i
    lib.dspark_propose_adaptive.argtypes = [_vp, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _i, _i, _i, _i, _i, _i, _i, _vp, _vp,
                                            _vp, _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.dspark_propose_adaptive.restype = _i
    lib.dspark_q4_packed_bytes.argtypes = [_i, _i]
    lib.dspark_q4_packed_bytes.restype = _sz
    lib.dspark_q4_pack.argtypes = [_vp, _i, _i, _vp, _vp]
    lib.dspark_q4_pack.restype = _i
    lib.dspark_q4_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
    lib.dspark_q4_workspace_bytes.restype = _sz
    lib.dspark_logits_q4.argtypes = [_vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp]
    lib.dspark_logits_q4.restype = _i
    lib.dspark_propose_q4.argtypes = lib.dspark_propose.argtypes
    lib.dspark_propose_q4.restype = _i
    lib.dspark_verify.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp]
    lib.dspark_verify.restype = _i
    lib.dspark_read_flags.argtypes = [_vp, ctypes.POINTER(ctypes.c_uint32), _vp]
    lib.dspark_read_flags.restype = _i
    lib.dspark_status_string.argtypes = [_i]
    lib.dspark_status_string.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load_library().dspark_status_string(int(status)).decode()


def workspace_bytes(B: int, L: int, V: int, top_k: int, layout="anchor_first") -> int:
    return int(load_library().dspark_workspace_bytes(B, L, V, top_k, LAYOUTS[layout]))


def n_pred_of(L: int, layout) -> int:
    return L - (1 if LAYOUTS[layout] == BONUS_ANCHOR else 0)


# ---------------------------------------------------------------------------
# torch front-end (device memory and streams only)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(t, stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _check_dev(name, t, dtype, shape=None):
    torch = _torch()
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    del torch


def _hidden_dtype(hidden) -> int:
    torch = _torch()
    if hidden.dtype == torch.bfloat16:
        return HIDDEN_BF16
    if hidden.dtype == torch.float32:
        return HIDDEN_F32
    raise ValueError(f"hidden must be bfloat16 or float32, got {hidden.dtype}")


class Outputs:
    """Device buffers of one proposal (reusable across calls of the same shape)."""

    def __init__(self, B: int, L: int, V: int, top_k: int, layout, device, *,
                 with_cand_logits: bool = True, with_conf: bool = True):
        torch = _torch()
        n = n_pred_of(L, layout)
        self.logits = torch.empty((B * n, V), dtype=torch.float32, device=device)
        self.tokens = torch.empty((B, n), dtype=torch.int32, device=device)
        self.candidates = torch.empty((B, n, top_k), dtype=torch.int32, device=device)
        self.cand_logits = (torch.empty((B, n, top_k), dtype=torch.float32, device=device)
                            if with_cand_logits else None)
        self.conf = torch.empty((B, n), dtype=torch.float32, device=device) if with_conf else None
        self.lengths = torch.empty((B,), dtype=torch.int32, device=device)
        nbytes = workspace_bytes(B, L, V, top_k, layout)
        self.workspace = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=device)

    def as_dict(self) -> dict:
        return {"logits": self.logits, "tokens": self.tokens, "candidates": self.candidates,
                "cand_logits": self.cand_logits, "conf": self.conf, "lengths": self.lengths}


def _event_handle(ev) -> Optional[int]:
    """The hipEvent_t of a torch.cuda.Event (created by its first record)."""
    if ev is None:
        return None
    if not ev.cuda_event:
        ev.record()
    return int(ev.cuda_event)


def propose(hidden, lm_head, markov_w1, markov_w2, anchors, *, layout="anchor_first", top_k=1,
            p_min=0.0, lm_head_bias=None, conf_w=None, out: Optional[Outputs] = None,
            stream=None, marks=None) -> Outputs:
    """Run dspark_propose on device tensors; returns the Outputs holding the results.
    With ``marks`` = (init, projected, chained) torch.cuda.Events (any may be
    None) the call is dspark_propose_marked, which records them on the stream
    between its launches."""
    torch = _torch()
    lib = load_library()
    B, L, H = hidden.shape
    V = lm_head.shape[0]
    r = 0 if markov_w1 is None else markov_w1.shape[1]
    _check_dev("hidden", hidden, hidden.dtype)
    _check_dev("lm_head", lm_head, torch.bfloat16, (V, H))
    _check_dev("lm_head_bias", lm_head_bias, torch.float32, (V,))
    _check_dev("markov_w1", markov_w1, torch.bfloat16, (V, r))
    _check_dev("markov_w2", markov_w2, torch.bfloat16, (V, r))
    _check_dev("conf_w", conf_w, torch.bfloat16, (H,))
    _check_dev("anchors", anchors, torch.int32, (B,))
    if out is None:
        out = Outputs(B, L, V, top_k, layout, hidden.device)
    args = (_ptr(hidden), _hidden_dtype(hidden), _ptr(lm_head), _ptr(lm_head_bias), _ptr(markov_w1),
            _ptr(markov_w2), _ptr(conf_w), _ptr(anchors), B, L, H, V, r, LAYOUTS[layout], top_k,
            float(p_min), _ptr(out.logits), _ptr(out.workspace), out.workspace.numel(),
            _ptr(out.tokens), _ptr(out.candidates), _ptr(out.cand_logits), _ptr(out.conf),
            _ptr(out.lengths), _stream(hidden, stream))
    if marks is None:
        st = lib.dspark_propose(*args)
    else:
        st = lib.dspark_propose_marked(*args, *[_event_handle(e) for e in marks])
    if st != OK:
        raise DsparkError(st, "dspark_propose_marked" if marks is not None else "dspark_propose")
    return out


def propose_noalloc(hidden, lm_head, markov_w1, markov_w2, anchors, *, layout="anchor_first",
                    top_k=1, p_min=0.0, lm_head_bias=None, conf_w=None,
                    out: Optional[Outputs] = None, stream=None) -> Outputs:
    """Run dspark_propose_noalloc (the library's static scratch as workspace;
    ``out.workspace`` is not used). Returns the Outputs holding the results."""
    torch = _torch()
    lib = load_library()
    B, L, H = hidden.shape
    V = lm_head.shape[0]
    r = 0 if markov_w1 is None else markov_w1.shape[1]
    _check_dev("hidden", hidden, hidden.dtype)
    _check_dev("lm_head", lm_head, torch.bfloat16, (V, H))
    _check_dev("lm_head_bias", lm_head_bias, torch.float32, (V,))
    _check_dev("markov_w1", markov_w1, torch.bfloat16, (V, r))
    _check_dev("markov_w2", markov_w2, torch.bfloat16, (V, r))
    _check_dev("conf_w", conf_w, torch.bfloat16, (H,))
    _check_dev("anchors", anchors, torch.int32, (B,))
    if out is None:
        out = Outputs(B, L, V, top_k, layout, hidden.device)
    st = lib.dspark_propose_noalloc(
        _ptr(hidden), _hidden_dtype(hidden), _ptr(lm_head), _ptr(lm_head_bias), _ptr(markov_w1),
        _ptr(markov_w2), _ptr(conf_w), _ptr(anchors), B, L, H, V, r, LAYOUTS[layout], top_k,
        float(p_min), _ptr(out.logits), _ptr(out.tokens), _ptr(out.candidates),
        _ptr(out.cand_logits), _ptr(out.conf), _ptr(out.lengths), _stream(hidden, stream))
    if st != OK:
        raise DsparkError(st, "dspark_propose_noalloc")
    return out


def propose_adaptive(hidden, lm_head, markov_w1, markov_w2, anchors, conf_w, p_min, *,
                     layout="anchor_first", top_k=1, block_top_k=None, lm_head_bias=None,
                     out: Optional[Outputs] = None, stream=None) -> Outputs:
    """Run dspark_propose_adaptive: ``p_min`` is a device fp32 [B] tensor of
    per-block thresholds, ``block_top_k`` an optional device int32 [B]."""
    torch = _torch()
    lib = load_library()
    B, L, H = hidden.shape
    V = lm_head.shape[0]
    r = 0 if markov_w1 is None else markov_w1.shape[1]
    _check_dev("hidden", hidden, hidden.dtype)
    _check_dev("lm_head", lm_head, torch.bfloat16, (V, H))
    _check_dev("lm_head_bias", lm_head_bias, torch.float32, (V,))
    _check_dev("markov_w1", markov_w1, torch.bfloat16, (V, r))
    _check_dev("markov_w2", markov_w2, torch.bfloat16, (V, r))
    _check_dev("conf_w", conf_w, torch.bfloat16, (H,))
    _check_dev("anchors", anchors, torch.int32, (B,))
    _check_dev("p_min", p_min, torch.float32, (B,))
    _check_dev("block_top_k", block_top_k, torch.int32, (B,))
    if out is None:
        out = Outputs(B, L, V, top_k, layout, hidden.device)
    st = lib.dspark_propose_adaptive(
        _ptr(hidden), _hidden_dtype(hidden), _ptr(lm_head), _ptr(lm_head_bias), _ptr(markov_w1),
        _ptr(markov_w2), _ptr(conf_w), _ptr(anchors), B, L, H, V, r, LAYOUTS[layout], top_k,
        _ptr(p_min), _ptr(block_top_k), _ptr(out.logits), _ptr(out.workspace),
        out.workspace.numel(), _ptr(out.tokens), _ptr(out.candidates), _ptr(out.cand_logits),
        _ptr(out.conf), _ptr(out.lengths), _stream(hidden, stream))
    if st != OK:
        raise DsparkError(st, "dspark_propose_adaptive")
    return out


def propose_d2t(hidden, lm_head, d2t, markov_w1, markov_w2, anchors, *, vocab: int,
                layout="anchor_first", top_k=1, p_min=0.0, conf_w=None,
                out: Optional[Outputs] = None, stream=None) -> Outputs:
    """Run dspark_propose_d2t: a draft head over D draft ids (``lm_head`` [D, H],
    ``markov_w2`` [D, r]) whose ids map to target ids through ``d2t`` (int64 [D],
    strictly increasing, in [0, vocab)); ``markov_w1`` is [vocab, r]. The Outputs
    must be sized for D columns; tokens and candidates come back as target ids."""
    torch = _torch()
    lib = load_library()
    B, L, H = hidden.shape
    D = lm_head.shape[0]
    r = 0 if markov_w1 is None else markov_w1.shape[1]
    _check_dev("hidden", hidden, hidden.dtype)
    _check_dev("lm_head", lm_head, torch.bfloat16, (D, H))
    _check_dev("d2t", d2t, torch.int64, (D,))
    _check_dev("markov_w1", markov_w1, torch.bfloat16, (vocab, r))
    _check_dev("markov_w2", markov_w2, torch.bfloat16, (D, r))
    _check_dev("conf_w", conf_w, torch.bfloat16, (H,))
    _check_dev("anchors", anchors, torch.int32, (B,))
    if out is None:
        out = Outputs(B, L, D, top_k, layout, hidden.device)
    st = lib.dspark_propose_d2t(
        _ptr(hidden), _hidden_dtype(hidden), _ptr(lm_head), _ptr(d2t), _ptr(markov_w1),
        _ptr(markov_w2), _ptr(conf_w), _ptr(anchors), B, L, H, int(vocab), D, r,
        LAYOUTS[layout], top_k, float(p_min), _ptr(out.logits), _ptr(out.workspace),
        out.workspace.numel(), _ptr(out.tokens), _ptr(out.candidates), _ptr(out.cand_logits),
        _ptr(out.conf), _ptr(out.lengths), _stream(hidden, stream))
    if st != OK:
        raise DsparkError(st, "dspark_propose_d2t")
    return out


def q4_packed_bytes(V: int, H: int) -> int:
    return int(load_library().dspark_q4_packed_bytes(V, H))


def q4_workspace_bytes(B: int, L: int, H: int, V: int, top_k: int, layout="anchor_first") -> int:
    return int(load_library().dspark_q4_workspace_bytes(B, L, H, V, top_k, LAYOUTS[layout]))


def q4_pack(blocks, V: int, H: int, *, out=None, stream=None):
    """Run dspark_q4_pack: ``blocks`` is the device uint8 [V, H/32*18] GGUF 4-bit
    head; returns the packed head (device uint8, dspark_q4_packed_bytes bytes)."""
    torch = _torch()
    lib = load_library()
    _check_dev("blocks", blocks, torch.uint8, (V, H // 32 * 18))
    nbytes = q4_packed_bytes(V, H)
    if nbytes == 0:
        raise ValueError(f"no 4-bit packing for V={V}, H={H} (H must be a multiple of 32)")
    if out is None:
        out = torch.empty((nbytes,), dtype=torch.uint8, device=blocks.device)
    _check_dev("out", out, torch.uint8, (nbytes,))
    st = lib.dspark_q4_pack(_ptr(blocks), V, H, _ptr(out), _stream(blocks, stream))
    if st != OK:
        raise DsparkError(st, "dspark_q4_pack")
    return out


class OutputsQ4(Outputs):
    """Outputs of a 4-bit head call: the workspace also holds the per-call
    preparation of the hidden rows."""

    def __init__(self, B: int, L: int, H: int, V: int, top_k: int, layout, device, **kw):
        super().__init__(B, L, V, top_k, layout, device, **kw)
        torch = _torch()
        nbytes = q4_workspace_bytes(B, L, H, V, top_k, layout)
        self.workspace = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=device)


def _check_q4_head(lm_head_q4, V, H):
    torch = _torch()
    nbytes = q4_packed_bytes(V, H)
    if nbytes == 0:
        raise ValueError(f"no 4-bit head for V={V}, H={H} (H must be a multiple of 32)")
    _check_dev("lm_head_q4", lm_head_q4, torch.uint8, (nbytes,))


def propose_q4(hidden, lm_head_q4, markov_w1, markov_w2, anchors, *, V: int,
               layout="anchor_first", top_k=1, p_min=0.0, lm_head_bias=None, conf_w=None,
               out: Optional[OutputsQ4] = None, stream=None) -> OutputsQ4:
    """Run dspark_propose_q4 with a packed 4-bit head (``q4_pack``) of V rows."""
    torch = _torch()
    lib = load_library()
    B, L, H = hidden.shape
    r = 0 if markov_w1 is None else markov_w1.shape[1]
    _check_dev("hidden", hidden, hidden.dtype)
    _check_q4_head(lm_head_q4, V, H)
    _check_dev("lm_head_bias", lm_head_bias, torch.float32, (V,))
    _check_dev("markov_w1", markov_w1, torch.bfloat16, (V, r))
    _check_dev("markov_w2", markov_w2, torch.bfloat16, (V, r))
    _check_dev("conf_w", conf_w, torch.bfloat16, (H,))
    _check_dev("anchors", anchors, torch.int32, (B,))
    if out is None:
        out = OutputsQ4(B, L, H, V, top_k, layout, hidden.device)
    st = lib.dspark_propose_q4(
        _ptr(hidden), _hidden_dtype(hidden), _ptr(lm_head_q4), _ptr(lm_head_bias), _ptr(markov_w1),
        _ptr(markov_w2), _ptr(conf_w), _ptr(anchors), B, L, H, V, r, LAYOUTS[layout], top_k,
        float(p_min), _ptr(out.logits), _ptr(out.workspace), out.workspace.numel(),
        _ptr(out.tokens), _ptr(out.candidates), _ptr(out.cand_logits), _ptr(out.conf),
        _ptr(out.lengths), _stream(hidden, stream))
    if st != OK:
        raise DsparkError(st, "dspark_propose_q4")
    return out


def logits_q4(hidden, lm_head_q4, *, V: int, layout="anchor_first", lm_head_bias=None, out=None,
              workspace=None, stream=None):
    """Run dspark_logits_q4 (the 4-bit projection alone); returns fp32 [B*n_pred, V]."""
    torch = _torch()
    lib = load_library()
    B, L, H = hidden.shape
    _check_dev("hidden", hidden, hidden.dtype)
    _check_q4_head(lm_head_q4, V, H)
    _check_dev("lm_head_bias", lm_head_bias, torch.float32, (V,))
    n = n_pred_of(L, layout)
    if out is None:
        out = torch.empty((B * n, V), dtype=torch.float32, device=hidden.device)
    _check_dev("out", out, torch.float32, (B * n, V))
    if workspace is None:
        workspace = torch.empty((q4_workspace_bytes(B, L, H, V, 1, layout),), dtype=torch.uint8,
                                device=hidden.device)
    st = lib.dspark_logits_q4(_ptr(hidden), _hidden_dtype(hidden), _ptr(lm_head_q4),
                              _ptr(lm_head_bias), B, L, H, V, LAYOUTS[layout], _ptr(out),
                              _ptr(workspace), workspace.numel(), _stream(hidden, stream))
    if st != OK:
        raise DsparkError(st, "dspark_logits_q4")
    return out


def logits(hidden, lm_head, *, layout="anchor_first", lm_head_bias=None, out=None, stream=None):
    """Run dspark_logits (the lm_head projection alone); returns fp32 [B*n_pred, V]."""
    torch = _torch()
    lib = load_library()
    B, L, H = hidden.shape
    V = lm_head.shape[0]
    _check_dev("hidden", hidden, hidden.dtype)
    _check_dev("lm_head", lm_head, torch.bfloat16, (V, H))
    _check_dev("lm_head_bias", lm_head_bias, torch.float32, (V,))
    n = n_pred_of(L, layout)
    if out is None:
        out = torch.empty((B * n, V), dtype=torch.float32, device=hidden.device)
    _check_dev("out", out, torch.float32, (B * n, V))
    st = lib.dspark_logits(_ptr(hidden), _hidden_dtype(hidden), _ptr(lm_head), _ptr(lm_head_bias),
                           B, L, H, V, LAYOUTS[layout], _ptr(out), _stream(hidden, stream))
    if st != OK:
        raise DsparkError(st, "dspark_logits")
    return out


def chain(logits_in, markov_w1, markov_w2, anchors, *, B, L, layout="anchor_first", top_k=1,
          p_min=0.0, hidden=None, conf_w=None, out: Optional[Outputs] = None, stream=None) -> Outputs:
    """Run dspark_chain on caller-provided projections ``logits_in`` [B*n_pred, V]."""
    torch = _torch()
    lib = load_library()
    V = logits_in.shape[1]
    r = 0 if markov_w1 is None else markov_w1.shape[1]
    H = hidden.shape[2] if hidden is not None else (conf_w.shape[0] if conf_w is not None else 8)
    n = n_pred_of(L, layout)
    _check_dev("logits", logits_in, torch.float32, (B * n, V))
    _check_dev("markov_w1", markov_w1, torch.bfloat16, (V, r))
    _check_dev("markov_w2", markov_w2, torch.bfloat16, (V, r))
    _check_dev("conf_w", conf_w, torch.bfloat16, (H,))
    _check_dev("anchors", anchors, torch.int32, (B,))
    if out is None:
        out = Outputs(B, L, V, top_k, layout, logits_in.device)
    hd = _hidden_dtype(hidden) if hidden is not None else HIDDEN_BF16
    st = lib.dspark_chain(
        _ptr(logits_in), _ptr(hidden), hd, _ptr(markov_w1), _ptr(markov_w2), _ptr(conf_w),
        _ptr(anchors), B, L, H, V, r, LAYOUTS[layout], top_k, float(p_min), _ptr(out.workspace),
        out.workspace.numel(), _ptr(out.tokens), _ptr(out.candidates), _ptr(out.cand_logits),
        _ptr(out.conf), _ptr(out.lengths), _stream(logits_in, stream))
    if st != OK:
        raise DsparkError(st, "dspark_chain")
    return out


def verify(candidates, lengths, target, *, lattice: bool = False, accepted=None, totals=None,
           stream=None):
    """Run dspark_verify; returns (accepted [B], totals [2]) as device int32 tensors."""
    torch = _torch()
    lib = load_library()
    B, n, k = candidates.shape
    _check_dev("candidates", candidates, torch.int32)
    _check_dev("lengths", lengths, torch.int32, (B,))
    _check_dev("target", target, torch.int32, (B, n))
    if accepted is None:
        accepted = torch.empty((B,), dtype=torch.int32, device=candidates.device)
    if totals is None:
        totals = torch.empty((2,), dtype=torch.int32, device=candidates.device)
    _check_dev("accepted", accepted, torch.int32, (B,))
    _check_dev("totals", totals, torch.int32, (2,))
    st = lib.dspark_verify(_ptr(candidates), _ptr(lengths), _ptr(target), B, n, k, int(bool(lattice)),
                           _ptr(accepted), _ptr(totals), _stream(candidates, stream))
    if st != OK:
        raise DsparkError(st, "dspark_verify")
    return accepted, totals


def read_flags(out: Outputs, stream=None) -> int:
    """Flags word of the workspace after the stream drains (synchronises the stream)."""
    lib = load_library()
    flags = ctypes.c_uint32(0)
    st = lib.dspark_read_flags(_ptr(out.workspace), ctypes.byref(flags),
                               _stream(out.workspace, stream))
    if st != OK:
        raise DsparkError(st, "dspark_read_flags")
    return int(flags.value)
