"""pi_layer_noalloc -- the layer call whose scratch is the library's static
device array -- against pi_layer with a caller workspace, through the C ABI.

The two share every kernel, so the outputs must be identical bit for bit.
Each case makes two calls in a row, the second with a smaller input, so the
second call runs on scratch that still holds the first call's contents.
"""

import pytest
import torch

import activation_sparse_rank_amd as pi
import workload
from activation_sparse_rank_amd import _lib as L
from helpers import DeviceLayer, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _both(dl, n_tok, stream_id):
    cfg = dl.cfg
    x = workload.make_tokens(cfg, 0, n_tok, "cuda", stream=stream_id)
    y_ref = torch.empty((n_tok, cfg.d_model), dtype=torch.float32, device="cuda")
    ws = pi.alloc_workspace(dl.pred, dl.ffn, n_tok)
    pi.layer(dl.pred, dl.ffn, x, cfg.tau, y_ref, ws=ws)
    y = torch.full_like(y_ref, float("nan"))
    pi.layer_noalloc(dl.pred, dl.ffn, x, cfg.tau, y)
    torch.cuda.synchronize()
    assert pi.read_flags(ws) == 0
    return y, y_ref


@pytest.mark.parametrize("name,first,second", [
    ("falcon40b", 8, 1),        # matrix-core predictor and FFN, then the fused kernel
    ("falcon40b", 2, 1),        # fused kernel, 2-token tile then 1
    ("falcon40b_q4", 16, 2),    # Q4_0 matrix-core path, then the fused Q4_0 tile of 2
    ("llama70b", 32, 3),        # ReGLU, 32 then 3 tokens on the matrix cores
    ("tiny", 8, 1),             # fp32 fused tiles
])
def test_noalloc_matches_layer(name, first, second):
    cfg = workload.get_config(name)
    dl = DeviceLayer(cfg, layer=0)
    for n_tok, sid in ((first, 0), (second, 1)):
        y, y_ref = _both(dl, n_tok, sid)
        assert torch.equal(y, y_ref), f"{name} n={n_tok}: pi_layer_noalloc differs from pi_layer"


def test_noalloc_smaller_layer_after_larger():
    # A Falcon-shaped 8-token call leaves its lists and partial sums in the
    # scratch; a tiny layer's single token must not see any of them.
    big = DeviceLayer(workload.get_config("falcon40b"), layer=1)
    small = DeviceLayer(workload.get_config("tiny"), layer=0)
    y, y_ref = _both(big, 8, 2)
    assert torch.equal(y, y_ref)
    y, y_ref = _both(small, 1, 3)
    assert torch.equal(y, y_ref)


def test_noalloc_rejects_oversize():
    cfg = workload.get_config("falcon40b")
    dl = DeviceLayer(cfg, layer=0)
    n = 64                                      # needs far more than the static scratch
    assert pi.workspace_bytes(dl.pred, dl.ffn, n) > L.PI_NOALLOC_SCRATCH_BYTES
    x = workload.make_tokens(cfg, 0, n, "cuda")
    y = torch.zeros((n, cfg.d_model), dtype=torch.float32, device="cuda")
    with pytest.raises(pi.PiError) as err:
        pi.layer_noalloc(dl.pred, dl.ffn, x, cfg.tau, y)
    assert err.value.status == L.PI_E_WORKSPACE
    assert "static scratch" in str(err.value)
    torch.cuda.synchronize()
    assert torch.all(y == 0), "a rejected call must launch nothing"
