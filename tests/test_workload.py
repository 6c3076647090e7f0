"""CPU checks of the seeded input generator.

The generator must reproduce its stated recipe: the Zipf constants, neurons
that fire (and are predicted) with the calibrated probabilities, identical
bits for identical seeds, and Q4_0 blocks that decode to the weights it meant.
"""

import numpy as np
import pytest
import torch

import oracle
import workload
from workload import CONFIGS, zipf_profile


@pytest.mark.parametrize("name,C,n_on", [
    ("tiny", 59.58, 41),
    ("opt30b", 547.9, 308),
    ("falcon40b", 1558.6, 798),
    ("llama70b", 1345.7, 699),
])
def test_zipf_constants(name, C, n_on):
    cfg = CONFIGS[name]
    p, c, on = zipf_profile(cfg.d_ff, cfg.rho, cfg.zipf_s, seed=0)
    assert abs(c - C) / C < 1e-3
    assert on == n_on
    assert abs(p.mean() - cfg.rho) < 1e-6
    assert p.max() < 1.0 and p.min() > 0.0


def test_zipf_concentration_matches_pages_scale():
    # Share of neurons that carry 80% of the firings: the pages report 26%
    # (OPT-30B, one layer) and 43% (LLaMA(ReGLU)-70B); the profile gives ~26%/~32%.
    for name, lo, hi in (("opt30b", 0.24, 0.28), ("falcon40b", 0.30, 0.35)):
        cfg = CONFIGS[name]
        p, _, _ = zipf_profile(cfg.d_ff, cfg.rho, cfg.zipf_s, seed=0)
        s = np.sort(p)[::-1]
        k = int(np.searchsorted(np.cumsum(s) / s.sum(), 0.8)) + 1
        assert lo < k / cfg.d_ff < hi


def test_same_seed_same_bits():
    cfg = CONFIGS["tiny"]
    a = workload.make_layer(cfg, 0)
    b = workload.make_layer(cfg, 0)
    for k in ("p1", "p2", "c", "w_up", "w_down_t", "b_up"):
        assert torch.equal(a[k], b[k]), k
    c = workload.make_layer(cfg, 1)
    assert not torch.equal(a["w_up"], c["w_up"])
    x1 = workload.make_tokens(cfg, 0, 4)
    x2 = workload.make_tokens(cfg, 0, 4)
    assert torch.equal(x1, x2) and x1.dtype == torch.float32
    assert not torch.equal(x1, workload.make_tokens(cfg, 0, 4, stream=1))


def _rates(cfg, L, n_tok):
    xs = workload.make_tokens(cfg, 0, n_tok).numpy()
    w_up = oracle.Q4_0Matrix(L["w_up"].numpy(), cfg.d_model) if cfg.wtype == "q4_0" else L["w_up"].numpy()
    w_dt = oracle.Q4_0Matrix(L["w_down_t"].numpy(), cfg.d_model) if cfg.wtype == "q4_0" else L["w_down_t"].numpy()
    kw = {}
    if cfg.act == "reglu":
        wg = L["w_gate"].numpy()
        kw = dict(w_gate=oracle.Q4_0Matrix(wg, cfg.d_model) if cfg.wtype == "q4_0" else wg,
                  b_gate=L["b_gate"].numpy())
    else:
        kw = dict(b_up=L["b_up"].numpy())
    _, fired = oracle.dense_ffn(xs, w_up, w_dt, cfg.act, **kw)
    _, mask = oracle.predict(xs, L["p1"].numpy(), L["p2"].numpy(), L["c"].numpy(), cfg.tau, decide=None)
    return fired.mean(axis=0), mask.mean(axis=0)


@pytest.mark.parametrize("cfg", [
    CONFIGS["tiny"],
    CONFIGS["llama70b"].with_(name="reglu_small", d_model=512, d_ff=1536, rank=64),
    CONFIGS["falcon40b_q4"].with_(name="q4_small", d_model=512, d_ff=1024, rank=64),
], ids=lambda c: c.name)
def test_calibrated_firing_rates(cfg):
    n_tok = 2000
    L = workload.make_layer(cfg, 0)
    fire_rate, pred_rate = _rates(cfg, L, n_tok)
    p = L["p"]
    # Mean over neurons: tight.  Per neuron: 5 sigma binomial band.
    assert abs(fire_rate.mean() - p.mean()) < 0.01
    assert abs(pred_rate.mean() - p.mean()) < 0.01
    band = 5.0 * np.sqrt(p * (1 - p) / n_tok) + 1.0 / n_tok
    assert np.mean(np.abs(fire_rate - p) <= band) > 0.995
    assert np.mean(np.abs(pred_rate - p) <= band) > 0.995


def test_q4_0_packer_decodes_to_its_codes():
    rng = np.random.default_rng(0)
    rows, nb = 5, 3
    d = torch.from_numpy((rng.standard_normal((rows, nb)) * 0.05).astype(np.float16))
    q = torch.from_numpy(rng.integers(0, 16, size=(rows, nb * 32)).astype(np.uint8))
    blocks = workload.q4_0_pack(d, q).numpy()
    assert blocks.shape == (rows, nb * 18)
    w = oracle.q4_0_dequant(blocks, nb * 32)
    expect = d.numpy().astype(np.float64).repeat(32, axis=1) * (q.numpy().astype(np.float64) - 8.0)
    assert np.array_equal(w, expect)


def test_q4_0_quantizer_error_bound():
    gen = torch.Generator().manual_seed(3)
    w = torch.randn((4, 256), generator=gen) * 0.02
    w[1, :32] = 0.0
    d, q = workload.q4_0_quantize(w)
    deq = oracle.q4_0_dequant(workload.q4_0_pack(d, q).numpy(), 256)
    err = np.abs(deq - w.numpy().astype(np.float64)).reshape(4, 8, 32).max(axis=2)
    assert np.all(err <= d.numpy().astype(np.float64) * 0.5 * (1 + 1e-3) + 1e-7)
    assert np.all(deq[1, :32] == 0.0)


def test_bernoulli_mask_rate():
    p = np.linspace(0.01, 0.9, 300)
    m = workload.bernoulli_mask(p, 4000, seed=1).numpy()
    assert m.dtype == np.uint8 and set(np.unique(m)) <= {0, 1}
    assert np.max(np.abs(m.mean(axis=0) - p)) < 5 * np.sqrt(0.25 / 4000) + 1e-3
