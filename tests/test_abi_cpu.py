"""The C-ABI library loads without a GPU, exports every declared entry point,
and rejects bad arguments on the host before anything is enqueued."""
import ctypes
import os
import re

import pytest

import dspark_block_drafter_amd as dsp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")


@pytest.fixture(scope="module")
def lib():
    return dsp.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(dspark_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(dsp.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4):
        assert lib.dspark_status_string(st).decode() not in ("", "unknown status")
    assert lib.dspark_status_string(17).decode() == "unknown status"


def test_workspace_bytes_layout(lib):
    # [256 B flags][n_pred*8*roundup(B, 32)*8 winners (8 ways per block), 256-aligned]
    # [B*n_pred*4 k-th slab maxima, 256-aligned]
    # [B*n_pred*ceil(V/64)*4 slab maxima, 256-aligned]
    # [n_pred*B*nwg*top_k*8 partials, 256-aligned, top_k > 1]
    def al(x):
        return (x + 255) // 256 * 256
    for B, L, V, k, lay in [(64, 16, 248320, 4, 0), (1, 16, 151936, 1, 0), (4, 7, 262144, 1, 1),
                            (3, 5, 1000, 3, 0), (5, 7, 777, 16, 1)]:
        n = L - lay
        # chain workgroups: pipelined kernel (V % 4 == 0) runs at most min(ceil(V/64), 512)
        # (two per CU in its two-stage form), the direct kernel one per 128 columns
        nwg = min((V + 63) // 64, 512) if V % 4 == 0 else (V + 127) // 128
        Bp = (B + 31) // 32 * 32
        want = (256 + al(n * 8 * Bp * 8) + al(B * n * 4) + al(B * n * ((V + 63) // 64) * 4)
                + (al(n * B * nwg * k * 8) if k > 1 else 0))
        assert lib.dspark_workspace_bytes(B, L, V, k, lay) == want


@pytest.mark.parametrize("args", [(0, 4, 100, 1, 0), (2, 0, 100, 1, 0), (2, 4, 0, 1, 0), (2, 4, 100, 0, 0),
                                  (2, 4, 100, 17, 0), (2, 4, 100, 1, 2), (2, 1, 100, 1, 1)])
def test_workspace_bytes_invalid(lib, args):
    assert lib.dspark_workspace_bytes(*args) == 0


# Non-null, 256-byte aligned fake device addresses: validation must reject the
# call before any of them is dereferenced or anything is enqueued.
P = 1 << 20


def propose(lib, **kw):
    a = dict(hidden=P, hidden_dtype=0, lm_head=P, bias=None, w1=P, w2=P, conf_w=P, anchors=P,
             B=2, L=4, H=64, V=512, r=8, layout=0, top_k=2, p_min=0.5, logits=P, ws=P,
             ws_bytes=1 << 30, tokens=P, cand=P, cand_logits=P, conf=P, lengths=P, stream=None)
    a.update(kw)
    return lib.dspark_propose(a["hidden"], a["hidden_dtype"], a["lm_head"], a["bias"], a["w1"], a["w2"],
                              a["conf_w"], a["anchors"], a["B"], a["L"], a["H"], a["V"], a["r"],
                              a["layout"], a["top_k"], ctypes.c_float(a["p_min"]), a["logits"], a["ws"],
                              a["ws_bytes"], a["tokens"], a["cand"], a["cand_logits"], a["conf"],
                              a["lengths"], a["stream"])


INVALID = [dict(B=0), dict(L=0), dict(H=0), dict(V=0), dict(B=-3), dict(layout=2), dict(layout=-1),
           dict(layout=1, L=1), dict(top_k=0), dict(top_k=17), dict(V=3, top_k=4), dict(r=-8),
           dict(w1=None), dict(w2=None), dict(r=0), dict(hidden_dtype=2), dict(p_min=float("nan")),
           dict(hidden=None), dict(lm_head=None), dict(logits=None), dict(anchors=None),
           dict(tokens=None), dict(cand=None), dict(lengths=None)]


@pytest.mark.parametrize("kw", INVALID, ids=[",".join(f"{k}={v}" for k, v in d.items()) for d in INVALID])
def test_propose_rejects_invalid(lib, kw):
    assert propose(lib, **kw) == dsp.ERR_INVALID_ARG


UNSUPPORTED = [dict(H=60), dict(r=12), dict(r=264), dict(hidden=P + 4), dict(lm_head=P + 2),
               dict(w1=P + 8), dict(logits=P + 4)]


@pytest.mark.parametrize("kw", UNSUPPORTED, ids=[",".join(f"{k}={v}" for k, v in d.items()) for d in UNSUPPORTED])
def test_propose_rejects_unsupported(lib, kw):
    assert propose(lib, **kw) == dsp.ERR_UNSUPPORTED


def test_propose_rejects_workspace(lib):
    need = lib.dspark_workspace_bytes(2, 4, 512, 2, 0)
    assert propose(lib, ws=None) == dsp.ERR_WORKSPACE
    assert propose(lib, ws_bytes=need - 1) == dsp.ERR_WORKSPACE
    assert propose(lib, ws=P + 64) == dsp.ERR_WORKSPACE


def propose_d2t(lib, **kw):
    a = dict(hidden=P, hidden_dtype=0, lm_head=P, d2t=P, w1=P, w2=P, conf_w=P, anchors=P,
             B=2, L=4, H=64, V=4096, D=512, r=8, layout=0, top_k=2, p_min=0.5, logits=P, ws=P,
             ws_bytes=1 << 30, tokens=P, cand=P, cand_logits=P, conf=P, lengths=P, stream=None)
    a.update(kw)
    return lib.dspark_propose_d2t(a["hidden"], a["hidden_dtype"], a["lm_head"], a["d2t"], a["w1"],
                                  a["w2"], a["conf_w"], a["anchors"], a["B"], a["L"], a["H"], a["V"],
                                  a["D"], a["r"], a["layout"], a["top_k"], ctypes.c_float(a["p_min"]),
                                  a["logits"], a["ws"], a["ws_bytes"], a["tokens"], a["cand"],
                                  a["cand_logits"], a["conf"], a["lengths"], a["stream"])


INVALID_D2T = [dict(D=0), dict(V=0), dict(D=4097), dict(d2t=None), dict(D=3, top_k=4),
               dict(lm_head=None), dict(w2=None), dict(layout=3), dict(p_min=float("nan"))]


@pytest.mark.parametrize("kw", INVALID_D2T, ids=[",".join(f"{k}={v}" for k, v in d.items()) for d in INVALID_D2T])
def test_propose_d2t_rejects_invalid(lib, kw):
    assert propose_d2t(lib, **kw) == dsp.ERR_INVALID_ARG


def test_propose_d2t_rejects_unsupported_and_workspace(lib):
    assert propose_d2t(lib, d2t=P + 4) == dsp.ERR_UNSUPPORTED     # int64 table misaligned
    assert propose_d2t(lib, H=60) == dsp.ERR_UNSUPPORTED
    # the workspace is sized for the D draft columns
    need = lib.dspark_workspace_bytes(2, 4, 512, 2, 0)
    assert propose_d2t(lib, ws_bytes=need - 1) == dsp.ERR_WORKSPACE
    assert propose_d2t(lib, ws=None) == dsp.ERR_WORKSPACE


def test_verify_rejects_invalid(lib):
    def v(**kw):
        a = dict(cand=P, lengths=P, target=P, B=4, n=8, k=2, lattice=1, acc=P, tot=P)
        a.update(kw)
        return lib.dspark_verify(a["cand"], a["lengths"], a["target"], a["B"], a["n"], a["k"],
                                 a["lattice"], a["acc"], a["tot"], None)
    for kw in (dict(B=0), dict(n=0), dict(k=0), dict(k=17), dict(lattice=2), dict(cand=None),
               dict(lengths=None), dict(target=None), dict(acc=None), dict(tot=None)):
        assert v(**kw) == dsp.ERR_INVALID_ARG, kw
    assert v(B=1 << 20, n=1 << 8, k=16) == dsp.ERR_UNSUPPORTED


def test_r0_needs_null_markov(lib):
    # r == 0 is valid only with both Markov pointers NULL; r > 0 needs both
    assert propose(lib, r=0, w1=P, w2=None) == dsp.ERR_INVALID_ARG
    assert propose(lib, r=8, w1=P, w2=None) == dsp.ERR_INVALID_ARG


def test_logits_and_chain_reject_invalid(lib):
    f = ctypes.c_float
    assert lib.dspark_logits(P, 0, P, None, 0, 4, 64, 512, 0, P, None) == dsp.ERR_INVALID_ARG
    assert lib.dspark_logits(None, 0, P, None, 2, 4, 64, 512, 0, P, None) == dsp.ERR_INVALID_ARG
    assert lib.dspark_logits(P, 0, P, None, 2, 4, 60, 512, 0, P, None) == dsp.ERR_UNSUPPORTED
    assert lib.dspark_chain(P, P, 0, P, P, P, P, 2, 4, 64, 512, 8, 0, 20, f(0.0), P, 1 << 30,
                            P, P, None, None, P, None) == dsp.ERR_INVALID_ARG
    assert lib.dspark_chain(P, None, 0, P, P, P, P, 2, 4, 64, 512, 8, 0, 2, f(0.0), P, 1 << 30,
                            P, P, None, None, P, None) == dsp.ERR_INVALID_ARG  # conf_w needs hidden
    assert lib.dspark_chain(P, P, 0, P, P, P, P, 2, 4, 64, 512, 8, 0, 2, f(0.0), P, 16,
                            P, P, None, None, P, None) == dsp.ERR_WORKSPACE


def test_read_flags_rejects_null(lib):
    flags = ctypes.c_uint32()
    assert lib.dspark_read_flags(None, ctypes.byref(flags), None) == dsp.ERR_INVALID_ARG


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(ImportError):
        dsp.load_library(str(tmp_path / "libdspark.so"))


def test_noalloc_validates_before_anything(lib):
    """dspark_propose_noalloc rejects bad arguments like dspark_propose, and
    sizes whose workspace exceeds its static scratch with DSPARK_ERR_SCRATCH,
    all before any HIP call (no GPU here)."""
    def call(**kw):
        a = dict(hidden=P, hidden_dtype=0, lm_head=P, bias=None, w1=P, w2=P, conf_w=P, anchors=P,
                 B=2, L=4, H=64, V=512, r=8, layout=0, top_k=2, p_min=0.5, logits=P, tokens=P,
                 cand=P, cand_logits=P, conf=P, lengths=P, stream=None)
        a.update(kw)
        return lib.dspark_propose_noalloc(
            a["hidden"], a["hidden_dtype"], a["lm_head"], a["bias"], a["w1"], a["w2"], a["conf_w"],
            a["anchors"], a["B"], a["L"], a["H"], a["V"], a["r"], a["layout"], a["top_k"],
            ctypes.c_float(a["p_min"]), a["logits"], a["tokens"], a["cand"], a["cand_logits"],
            a["conf"], a["lengths"], a["stream"])
    assert call(B=0) == dsp.ERR_INVALID_ARG
    assert call(top_k=17) == dsp.ERR_INVALID_ARG
    assert call(tokens=None) == dsp.ERR_INVALID_ARG
    assert call(H=12) == dsp.ERR_UNSUPPORTED
    assert call(B=512, L=64, V=248320, top_k=4) == dsp.ERR_SCRATCH
    assert dsp.workspace_bytes(512, 64, 248320, 4) > dsp.NOALLOC_SCRATCH_BYTES
    assert "static scratch" in dsp.status_string(dsp.ERR_SCRATCH)


def test_q4_sizes(lib):
    """Packed 4-bit head: (ceil(V/16) tiles) x (ceil(H/128) quads) x (1024 + 128) bytes;
    the 4-bit workspace adds M x 128 ceil(H/128) bf16 (256-aligned) after the
    chain's."""
    def al(x):
        return (x + 255) // 256 * 256
    for V, H in [(512, 64), (151936, 4096), (248320, 5120), (262144, 2816), (37, 96)]:
        assert lib.dspark_q4_packed_bytes(V, H) == (V + 15) // 16 * ((H // 32 + 3) // 4) * 1152
    for V, H in [(0, 64), (10, 0), (10, 48), (10, -32)]:
        assert lib.dspark_q4_packed_bytes(V, H) == 0
    for B, L, H, V, k, lay in [(64, 16, 5120, 248320, 4, 0), (4, 7, 2816, 262144, 1, 1), (1, 4, 64, 512, 1, 0)]:
        M = B * (L - lay)
        assert lib.dspark_q4_workspace_bytes(B, L, H, V, k, lay) == (
            al(M * 128 * ((H // 32 + 3) // 4) * 2) + lib.dspark_workspace_bytes(B, L, V, k, lay))
    assert lib.dspark_q4_workspace_bytes(2, 4, 48, 512, 1, 0) == 0
    assert lib.dspark_q4_workspace_bytes(2, 4, 64, 512, 17, 0) == 0


def propose_q4(lib, **kw):
    a = dict(hidden=P, hidden_dtype=0, lm_head=P, bias=None, w1=P, w2=P, conf_w=P, anchors=P,
             B=2, L=4, H=64, V=512, r=8, layout=0, top_k=2, p_min=0.5, logits=P, ws=P,
             ws_bytes=1 << 30, tokens=P, cand=P, cand_logits=P, conf=P, lengths=P, stream=None)
    a.update(kw)
    return lib.dspark_propose_q4(a["hidden"], a["hidden_dtype"], a["lm_head"], a["bias"], a["w1"],
                                 a["w2"], a["conf_w"], a["anchors"], a["B"], a["L"], a["H"], a["V"],
                                 a["r"], a["layout"], a["top_k"], ctypes.c_float(a["p_min"]),
                                 a["logits"], a["ws"], a["ws_bytes"], a["tokens"], a["cand"],
                                 a["cand_logits"], a["conf"], a["lengths"], a["stream"])


@pytest.mark.parametrize("kw", INVALID, ids=[",".join(f"{k}={v}" for k, v in d.items()) for d in INVALID])
def test_propose_q4_rejects_invalid(lib, kw):
    assert propose_q4(lib, **kw) == dsp.ERR_INVALID_ARG


def test_q4_rejects_unsupported_and_workspace(lib):
    assert propose_q4(lib, H=48) == dsp.ERR_UNSUPPORTED           # not a multiple of 32
    assert propose_q4(lib, lm_head=P + 8) == dsp.ERR_UNSUPPORTED  # packed head misaligned
    assert propose_q4(lib, hidden=P + 4) == dsp.ERR_UNSUPPORTED
    need = lib.dspark_q4_workspace_bytes(2, 4, 64, 512, 2, 0)
    assert propose_q4(lib, ws_bytes=need - 1) == dsp.ERR_WORKSPACE
    assert propose_q4(lib, ws=None) == dsp.ERR_WORKSPACE
    assert propose_q4(lib, ws=P + 64) == dsp.ERR_WORKSPACE
    # the bf16 workspace alone is not enough for the 4-bit call
    assert propose_q4(lib, ws_bytes=lib.dspark_workspace_bytes(2, 4, 512, 2, 0)) == dsp.ERR_WORKSPACE
    lq = lib.dspark_logits_q4
    assert lq(P, 0, P, None, 0, 4, 64, 512, 0, P, P, 1 << 30, None) == dsp.ERR_INVALID_ARG
    assert lq(None, 0, P, None, 2, 4, 64, 512, 0, P, P, 1 << 30, None) == dsp.ERR_INVALID_ARG
    assert lq(P, 0, P, None, 2, 4, 48, 512, 0, P, P, 1 << 30, None) == dsp.ERR_UNSUPPORTED
    assert lq(P, 0, P, None, 2, 4, 64, 512, 0, P, P, 16, None) == dsp.ERR_WORKSPACE
    pk = lib.dspark_q4_pack
    assert pk(None, 512, 64, P, None) == dsp.ERR_INVALID_ARG
    assert pk(P, 0, 64, P, None) == dsp.ERR_INVALID_ARG
    assert pk(P, 512, 48, P, None) == dsp.ERR_UNSUPPORTED
    assert pk(P, 512, 64, P + 4, None) == dsp.ERR_UNSUPPORTED
