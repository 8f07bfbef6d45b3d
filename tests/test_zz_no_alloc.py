"""The allocation-free entry point (dspark_propose_noalloc) against
dspark_propose: the same kernels on the library's static scratch instead of a
caller workspace, so every output must be identical, bit for bit; two calls
in a row, the second with a smaller input (the scratch keeps the first call's
contents)."""
import numpy as np
import pytest

from synthetic import make_small

pytestmark = pytest.mark.gpu


def _host(res):
    return {k: (None if v is None else v.cpu().numpy()) for k, v in res.as_dict().items()}


def test_noalloc_matches_propose_on_two_calls():
    import torch

    import dspark_block_drafter_amd as dsp
    from devutil import run_propose, to_device
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cases = [
        make_small(40, 6, 256, 30000, 64, top_k=4, conf=True, p_min=0.4, seed=71),   # two block groups
        make_small(5, 4, 128, 5000, 16, top_k=2, conf=True, p_min=0.5, seed=72),     # smaller, pruned form
    ]
    for inp in cases:
        c = inp.cfg
        d = to_device(inp)
        want = _host(run_propose(inp, dev=d))
        got = dsp.propose_noalloc(d["hidden"], d["lm_head"], d["markov_w1"], d["markov_w2"],
                                  d["anchors"], layout=c.layout, top_k=c.top_k, p_min=c.p_min,
                                  lm_head_bias=d["lm_head_bias"], conf_w=d["conf_w"])
        torch.cuda.synchronize()
        got = _host(got)
        for k in want:
            assert np.array_equal(want[k], got[k]), (c.name, k)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    import torch

    import dspark_block_drafter_amd as dsp
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    # the workspace of B = 512 blocks of 64 slots over a 248320-id vocabulary
    # at top-4 is far above the static scratch: refused, nothing enqueued
    B, L, V, k = 512, 64, 248320, 4
    assert dsp.workspace_bytes(B, L, V, k) > dsp.NOALLOC_SCRATCH_BYTES
    lib = dsp.load_library()
    P = 1 << 20   # never dereferenced: the call stops before enqueuing
    st = lib.dspark_propose_noalloc(P, 0, P, None, P, P, None, P, B, L, 64, V, 8, 0, k, 0.0,
                                    P, P, P, None, None, P, None)
    assert st == dsp.ERR_SCRATCH
    assert "static scratch" in dsp.status_string(st)
