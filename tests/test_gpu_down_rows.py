"""GPU: the workspace header's counts of w_down and w_up rows read.

The list-path down projection (up to one token tile of 8; Q4_0: the tile
whose fp16 x fits 32 KB) reads only the listed rows whose h is nonzero for
some token of the tile, since a row whose h is exactly zero for every token
adds nothing to y.  The matrix-core path reads every listed row once per
token tile.  The up projections read the up row of every listed neuron once
per token tile, except pi_layer's fused kernel with ReGLU, which reads the
up row only of the listed neurons whose gate is positive for some token.
The expected counts are built from the oracle's dense FFN (its firing flags:
a ReLU / squared-ReLU neuron fires when its pre-activation is positive, a
ReGLU neuron when its gate is), and the list from pi_compact, which the
parity tests hold bit-exact to the oracle.
"""

import numpy as np
import pytest
import torch

import activation_sparse_rank_amd as pi
import oracle
import workload
from helpers import DeviceLayer, host, require_gpu

pytestmark = pytest.mark.gpu

# A neuron whose pre-activation lies within fp32 rounding of zero may count
# on either side; with random inputs that is rare (well under one per case).
SLACK = 2
LIST_TILE = 8     # list-path token tile at these widths (Q4_0 too: 8 * 1024 * 2 B <= 32 KB)
MFMA_TILE = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _cfg(wtype, act):
    return workload.get_config("falcon40b").with_(name=f"rows_{wtype}_{act}", d_model=1024, d_ff=6144, rank=128,
                                                 n_layers=1, wtype=wtype, act=act, rho=0.2)


def _mfma(wtype, n_tok):
    return (wtype == "f16" and n_tok > 2) or (wtype == "q4_0" and n_tok > LIST_TILE)


def _expected(fired, idx, n_tok, wtype):
    """Rows the down projection reads: per token tile, the listed rows that
    fire for a token of the tile (list path) or every listed row (matrix
    cores)."""
    if _mfma(wtype, n_tok):
        return len(idx) * ((n_tok + MFMA_TILE - 1) // MFMA_TILE)
    total = 0
    for t0 in range(0, n_tok, LIST_TILE):
        total += int(fired[t0:t0 + LIST_TILE][:, idx].any(axis=0).sum())
    return total


def _tiles(wtype, n_tok):
    t = MFMA_TILE if _mfma(wtype, n_tok) else LIST_TILE
    return (n_tok + t - 1) // t


def _expected_up(fired, idx, n_tok, wtype, act, layer):
    """w_up rows the up projections read: every listed row once per token
    tile, or, in pi_layer's fused kernel (one tile, no matrix cores) with
    ReGLU, the listed rows whose gate fires for some token."""
    fused = layer and n_tok <= LIST_TILE and not _mfma(wtype, n_tok)
    if fused and act == "reglu":
        return int(fired[:n_tok][:, idx].any(axis=0).sum())
    return len(idx) * _tiles(wtype, n_tok)


@pytest.mark.parametrize("wtype", ["f32", "f16", "q4_0"])
@pytest.mark.parametrize("act", ["relu", "reglu", "relu2"])
@pytest.mark.parametrize("n_tok", [1, 2, 9])
def test_rows_read(wtype, act, n_tok):
    cfg = _cfg(wtype, act)
    dl = DeviceLayer(cfg)
    f, d = cfg.d_ff, cfg.d_model
    x = workload.make_tokens(cfg, 0, n_tok, "cuda")
    mask = torch.empty((n_tok, f), dtype=torch.uint8, device="cuda")
    pi.predict(dl.pred, x, cfg.tau, mask)
    idx = torch.zeros(f, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    pi.compact(mask, idx, cnt)
    c = int(cnt.item())
    listed = host(idx)[:c].astype(np.int64)
    _, fired = oracle.dense_ffn(host(x), **dl.oracle_args()["ffn"])
    want = _expected(fired, listed, n_tok, wtype)
    what = f"{wtype} {act} n={n_tok} count={c}"
    if not _mfma(wtype, n_tok) and n_tok <= LIST_TILE:
        assert 0 < want < c, f"{what}: the case should have listed rows that do not fire"

    y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    ws = pi.alloc_workspace(None, dl.ffn, n_tok)
    assert pi.read_down_rows(ws) == 0 and pi.read_up_rows(ws) == 0
    pi.sparse_ffn(dl.ffn, x, idx, cnt, y, ws=ws)
    got = pi.read_down_rows(ws)
    assert abs(got - want) <= SLACK, f"{what}: pi_sparse_ffn read {got} rows, expected {want}"
    up = pi.read_up_rows(ws)
    want_up = _expected_up(fired, listed, n_tok, wtype, act, layer=False)
    assert up == want_up, f"{what}: pi_sparse_ffn read {up} up rows, expected {want_up}"
    pi.sparse_ffn(dl.ffn, x, idx, cnt, y, ws=ws)
    assert pi.read_down_rows(ws) == 2 * got, f"{what}: the count does not add up over calls"
    assert pi.read_up_rows(ws) == 2 * up, f"{what}: the up count does not add up over calls"
    pi.clear_flags(ws)
    assert pi.read_down_rows(ws) == 0 and pi.read_up_rows(ws) == 0

    # the layer call lists the same neurons (fused path: by slots)
    wl = pi.alloc_workspace(dl.pred, dl.ffn, n_tok)
    pi.layer(dl.pred, dl.ffn, x, cfg.tau, y, ws=wl)
    got_l = pi.read_down_rows(wl)
    assert abs(got_l - want) <= SLACK, f"{what}: pi_layer read {got_l} rows, expected {want}"
    up_l = pi.read_up_rows(wl)
    want_up = _expected_up(fired, listed, n_tok, wtype, act, layer=True)
    assert abs(up_l - want_up) <= SLACK, f"{what}: pi_layer read {up_l} up rows, expected {want_up}"
    if act == "reglu" and n_tok <= 2:
        assert want_up < c, f"{what}: the case should have listed neurons whose gate does not fire"
    assert pi.read_flags(wl) == 0


def test_all_zero_h_reads_nothing():
    # Every listed neuron's pre-activation is negative (bias -1e4): h is zero
    # everywhere, no down row is read and y is exactly zero.
    cfg = _cfg("f16", "relu")
    dl = DeviceLayer(cfg)
    f, d = cfg.d_ff, cfg.d_model
    dl.ffn = pi.FFN(dl.L["w_up"], dl.L["w_down_t"], "relu",
                    b_up=torch.full((f,), -1e4, dtype=torch.float32, device="cuda"))
    x = workload.make_tokens(cfg, 0, 1, "cuda")
    idx = torch.arange(f, dtype=torch.int32, device="cuda")
    cnt = torch.tensor([f], dtype=torch.int32, device="cuda")
    y = torch.full((1, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = pi.alloc_workspace(None, dl.ffn, 1)
    pi.sparse_ffn(dl.ffn, x, idx, cnt, y, ws=ws)
    assert pi.read_down_rows(ws) == 0
    assert pi.read_up_rows(ws) == f      # every listed up row is read; none passes h != 0
    assert torch.all(y == 0)


def test_reglu_gate_never_fires_reads_no_up_row():
    # pi_layer's fused kernel with ReGLU and a gate bias of -1e4: every gate is
    # negative, so no up row and no down row is read and y is exactly zero.
    cfg = _cfg("f16", "reglu")
    dl = DeviceLayer(cfg)
    f, d = cfg.d_ff, cfg.d_model
    dl.ffn = pi.FFN(dl.L["w_up"], dl.L["w_down_t"], "reglu", w_gate=dl.L["w_gate"],
                    b_gate=torch.full((f,), -1e4, dtype=torch.float32, device="cuda"))
    x = workload.make_tokens(cfg, 0, 1, "cuda")
    y = torch.full((1, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = pi.alloc_workspace(dl.pred, dl.ffn, 1)
    pi.layer(dl.pred, dl.ffn, x, 0.5, y, ws=ws)
    assert pi.read_up_rows(ws) == 0
    assert pi.read_down_rows(ws) == 0
    assert pi.read_flags(ws) == 0
    assert torch.all(y == 0)
