"""pi_layer captured into a HIP graph: every replay, with other (eager) work
on the same workspace between replays, must give the bits of the eager call
on the same input.  Covers the counters the layer kernels clear themselves
(the fused single-token kernel's segment words, the many-token predictor's
list words), which must not depend on anything a previous call left behind.
"""

import pytest
import torch

import activation_sparse_rank_amd as pi
import workload
from helpers import DeviceLayer, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("name,n_tok", [("falcon40b", 1), ("falcon40b", 8), ("falcon40b", 64), ("falcon40b", 70),
                                        ("falcon40b_q4", 1), ("falcon40b_q4", 8), ("llama70b", 1), ("tiny", 3)])
def test_layer_graph_replays_match_eager(name, n_tok):
    cfg = workload.get_config(name)
    dl = DeviceLayer(cfg, layer=1)
    d = cfg.d_model
    xs = [workload.make_tokens(cfg, 1, n_tok, "cuda", stream=s + 4) for s in range(3)]
    ws = pi.alloc_workspace(dl.pred, dl.ffn, n_tok)
    refs = []
    for x in xs:
        y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
        pi.layer(dl.pred, dl.ffn, x, cfg.tau, y, ws=ws)
        refs.append(y)
    torch.cuda.synchronize()

    x_stage = xs[0].clone()
    y_g = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        pi.layer(dl.pred, dl.ffn, x_stage, cfg.tau, y_g, ws=ws)      # warm-up before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        pi.layer(dl.pred, dl.ffn, x_stage, cfg.tau, y_g, ws=ws)
    torch.cuda.synchronize()

    y_e = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    for rep in range(6):
        k = rep % 3
        x_stage.copy_(xs[k])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, refs[k]), f"{name} n={n_tok}: replay {rep} differs from the eager call"
        # eager work on the same workspace between replays
        pi.layer(dl.pred, dl.ffn, xs[(k + 1) % 3], cfg.tau, y_e, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(y_e, refs[(k + 1) % 3])
    assert pi.read_flags(ws) == 0, "fault flags raised"
