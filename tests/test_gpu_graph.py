"""A proposal step captured in a HIP graph. dspark_propose_noalloc allocates
nothing and needs no host synchronisation, so a caller can capture it once
and replay it. Every replay must equal the eager call bit for bit, with other
eager work (another proposal on the same library scratch, torch operations,
synchronisations) between the replays."""
import numpy as np
import pytest

from synthetic import make_small

pytestmark = pytest.mark.gpu

CASES = {
    "top1_one_group": lambda: make_small(1, 9, 256, 40000, 64, top_k=1, conf=True, p_min=0.3, seed=81),
    "top4_two_groups": lambda: make_small(40, 5, 256, 30000, 64, top_k=4, conf=True, p_min=0.4, seed=82),
    "top4_pruned": lambda: make_small(8, 6, 128, 50000, 128, top_k=4, seed=83),
}


def _host(out):
    return {k: (None if v is None else v.cpu().numpy()) for k, v in out.as_dict().items()}


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_equal_the_eager_call(name):
    import torch

    import dspark_block_drafter_amd as dsp
    from devutil import to_device
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    inp = CASES[name]()
    c = inp.cfg
    d = to_device(inp)
    other = make_small(3, 4, 128, 7000, 16, top_k=2, conf=True, p_min=0.5, seed=84)
    od = to_device(other)

    def call(out=None):
        return dsp.propose_noalloc(d["hidden"], d["lm_head"], d["markov_w1"], d["markov_w2"],
                                   d["anchors"], layout=c.layout, top_k=c.top_k, p_min=c.p_min,
                                   lm_head_bias=d["lm_head_bias"], conf_w=d["conf_w"], out=out)

    eager = call()
    torch.cuda.synchronize()
    want = _host(eager)
    out = dsp.Outputs(c.B, c.L, c.V, c.top_k, c.layout, "cuda:0")
    call(out)   # warm-up on the capture's buffers
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    torch.cuda.synchronize()
    for rep in range(3):
        for v in out.as_dict().values():
            if v is not None:
                v.fill_(-7)   # stale outputs must be overwritten by the replay
        g.replay()
        torch.cuda.synchronize()
        got = _host(out)
        for k in want:
            if want[k] is not None:
                assert np.array_equal(want[k], got[k]), (name, rep, k)
        # eager work between replays: another proposal on the same scratch
        dsp.propose_noalloc(od["hidden"], od["lm_head"], od["markov_w1"], od["markov_w2"],
                            od["anchors"], layout=other.cfg.layout, top_k=other.cfg.top_k,
                            p_min=other.cfg.p_min, lm_head_bias=od["lm_head_bias"], conf_w=od["conf_w"])
        torch.zeros(1 << 20, device="cuda:0").add_(1.0).sum().item()
        torch.cuda.synchronize()
    del g
