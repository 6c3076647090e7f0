"""GPU parity: every step of the hot path against the CPU oracle.

Inputs are seeded and synthetic.  Small cases span several tiles and ragged
tails and are checked element by element; the model-sized layers are run in
the same per-token launch configuration the benchmark times and checked on
sampled tokens.  Every call goes through the C ABI (via the ctypes binding).
"""

import numpy as np
import pytest
import torch

import activation_sparse_rank_amd as pi
import oracle
import workload
from helpers import (TOL, DeviceLayer, check_layer_vs_calls, check_mask, check_y, host, host_ffn, layer_is_fused,
                     oracle_sparse_chunked, rand_ffn, require_gpu, wtag)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _i32(n):
    return torch.zeros(n, dtype=torch.int32, device="cuda")


# ---------------------------------------------------------------------------
# Compaction: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d_ff", [1, 15, 16, 17, 1000, 16384, 16385, 32768, 40000])
@pytest.mark.parametrize("n_tok", [1, 3, 8])
def test_compact_bitexact(d_ff, n_tok):
    g = torch.Generator(device="cuda").manual_seed(d_ff * 31 + n_tok)
    for density in (0.0, 0.03, 0.1, 1.0):
        mask = (torch.rand((n_tok, d_ff), generator=g, device="cuda") < density).to(torch.uint8)
        if d_ff > 5 and density > 0:
            mask[0, 5] = 200        # any nonzero byte marks its neuron
        idx = torch.full((d_ff,), -7, dtype=torch.int32, device="cuda")
        cnt = _i32(1)
        pi.compact(mask, idx, cnt)
        torch.cuda.synchronize()
        ref_idx, ref_cnt = oracle.compact(host(mask))
        c = int(cnt.item())
        assert c == ref_cnt
        assert np.array_equal(host(idx)[:c], ref_idx)


@pytest.mark.parametrize("d_ff", [65536, 98320])
@pytest.mark.parametrize("n_tok", [17, 64])
def test_compact_many_tiles(d_ff, n_tok):
    # 16-byte aligned rows: one workgroup per 4096-neuron tile, each counting
    # the tiles before it itself (up to 24 of them, 64 token rows).
    g = torch.Generator(device="cuda").manual_seed(d_ff + n_tok)
    for density in (0.0, 0.004, 0.05, 1.0):
        mask = (torch.rand((n_tok, d_ff), generator=g, device="cuda") < density).to(torch.uint8)
        idx = torch.full((d_ff,), -7, dtype=torch.int32, device="cuda")
        cnt = _i32(1)
        pi.compact(mask, idx, cnt)
        ref_idx, ref_cnt = oracle.compact(host(mask))
        c = int(cnt.item())
        assert c == ref_cnt
        assert np.array_equal(host(idx)[:c], ref_idx)


def test_compact_unaligned_rows():
    # d_ff not a multiple of 16: rows of the mask are not 16-byte aligned.
    d_ff, n_tok = 1001, 5
    mask = (torch.rand((n_tok, d_ff), device="cuda") < 0.2).to(torch.uint8)
    idx, cnt = _i32(d_ff), _i32(1)
    pi.compact(mask, idx, cnt)
    ref_idx, ref_cnt = oracle.compact(host(mask))
    assert int(cnt.item()) == ref_cnt and np.array_equal(host(idx)[:ref_cnt], ref_idx)


# ---------------------------------------------------------------------------
# Predictor: masks agree outside the +-1e-3 logit band
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d,r,f", [
    (torch.float32, 256, 32, 1024),      # the tiny fp32 shape
    (torch.float16, 200, 40, 999),       # ragged everywhere
    (torch.float16, 9216, 136, 3001),    # two passes over p1 rows, ragged rank
    (torch.float16, 512, 2048, 700),     # long p2 rows (two passes)
])
@pytest.mark.parametrize("n_tok", [1, 5, 9])
@pytest.mark.parametrize("tau", [0.5, 0.3])
def test_predict(dtype, d, r, f, n_tok, tau):
    g = torch.Generator(device="cuda").manual_seed(d + r + f + n_tok)
    p1 = (torch.randn((r, d), generator=g, device="cuda") * 0.02).to(dtype)
    p2 = (torch.randn((f, r), generator=g, device="cuda") * 0.02).to(dtype)
    c = (torch.randn(f, generator=g, device="cuda") * 0.01).float()
    x = torch.randn((n_tok, d), generator=g, device="cuda").to(dtype)
    pred = pi.Predictor(p1, p2, c)
    mask = torch.empty((n_tok, f), dtype=torch.uint8, device="cuda")
    logits = torch.empty((n_tok, f), dtype=torch.float32, device="cuda")
    pi.predict(pred, x, tau, mask, logits)
    ref_l, _ = oracle.predict(host(x), host(p1), host(p2), host(c), tau)
    err = np.abs(host(logits).astype(np.float64) - ref_l)
    assert err.max() <= 1e-5 + 1e-5 * np.abs(ref_l).max()
    check_mask(host(mask), ref_l, tau, "predict")
    assert set(np.unique(host(mask))) <= {0, 1}


@pytest.mark.parametrize("d,r,f", [(1024, 128, 1001), (8192, 1024, 4000)])
@pytest.mark.parametrize("n_tok", [3, 16, 17, 64, 70])
def test_predict_mfma(d, r, f, n_tok):
    # fp16 predictor with 3 or more tokens: the matrix-core predictor (t split
    # into fp16 high and low parts for the second product).
    tau = 0.4
    g = torch.Generator(device="cuda").manual_seed(d + r + f + 3 * n_tok)
    p1 = (torch.randn((r, d), generator=g, device="cuda") * 0.02).half()
    p2 = (torch.randn((f, r), generator=g, device="cuda") * 0.02).half()
    c = (torch.randn(f, generator=g, device="cuda") * 0.01).float()
    x = torch.randn((n_tok, d), generator=g, device="cuda").half()
    pred = pi.Predictor(p1, p2, c)
    mask = torch.empty((n_tok, f), dtype=torch.uint8, device="cuda")
    logits = torch.empty((n_tok, f), dtype=torch.float32, device="cuda")
    pi.predict(pred, x, tau, mask, logits)
    mask2 = torch.empty_like(mask)
    pi.predict(pred, x, tau, mask2)                 # without logits: same masks
    ref_l, _ = oracle.predict(host(x), host(p1), host(p2), host(c), tau)
    err = np.abs(host(logits).astype(np.float64) - ref_l)
    assert err.max() <= 1e-5 + 1e-5 * np.abs(ref_l).max()
    check_mask(host(mask), ref_l, tau, "predict mfma")
    assert torch.equal(mask, mask2)


# ---------------------------------------------------------------------------
# Sparse FFN over a given list
# ---------------------------------------------------------------------------

SHAPES = [
    (torch.float32, 256, 1024),     # tiny fp32 shape
    (torch.float16, 200, 999),      # ragged columns (< one 512-column slice)
    (torch.float16, 1032, 3000),    # ragged second slice, two chunks per lane
    (torch.float16, 9216, 700),     # rows longer than one pass of the up kernel
]


@pytest.mark.parametrize("dtype,d,f", SHAPES)
@pytest.mark.parametrize("act", ["relu", "reglu", "relu2"])
@pytest.mark.parametrize("n_tok", [1, 3, 8, 11])
def test_sparse_ffn(dtype, d, f, act, n_tok):
    kw = rand_ffn(d, f, act, dtype, seed=d + f + n_tok)
    ffn = pi.FFN(**kw)
    hk = host_ffn(kw)
    g = torch.Generator(device="cuda").manual_seed(7 * n_tok + f)
    x = torch.randn((n_tok, d), generator=g, device="cuda").to(dtype)
    for density in (0.1, 0.6):
        sel = torch.rand(f, generator=g, device="cuda") < density
        idx_list = torch.nonzero(sel).flatten().to(torch.int32)
        n = idx_list.numel()
        idx = _i32(f)
        idx[:n] = idx_list
        cnt = torch.tensor([n], dtype=torch.int32, device="cuda")
        for ytype in (torch.float32, torch.float16):
            y = torch.empty((n_tok, d), dtype=ytype, device="cuda")
            pi.sparse_ffn(ffn, x, idx, cnt, y)
            ref = oracle.sparse_ffn(host(x), host(idx_list), **hk)
            tol = TOL[wtag(dtype)]
            if ytype == torch.float16:
                ref_r = ref.astype(np.float16).astype(np.float64)    # compare the decoded value
                tol = max(tol, 2e-3)
                check_y(host(y), ref_r, tol + 1e-3, f"{act} d={d} f={f} n={n_tok} y16")
            else:
                check_y(host(y), ref, tol, f"{act} d={d} f={f} n={n_tok}")


# Multi-token path (matrix cores): more tokens than one list-path pass.
MFMA_SHAPES = [
    (128, 300),      # one 128-wide k step: three of the four k-split waves have no work
    (1024, 1000),    # ragged list tail (count not a multiple of 32 or 64)
    (8192, 700),     # model width
]


@pytest.mark.parametrize("d,f", MFMA_SHAPES)
@pytest.mark.parametrize("act", ["relu", "reglu", "relu2"])
@pytest.mark.parametrize("n_tok", [9, 16, 17, 40, 64, 65, 130])
def test_sparse_ffn_mfma(d, f, act, n_tok):
    dtype = torch.float16
    kw = rand_ffn(d, f, act, dtype, seed=d + f + n_tok + 1)
    ffn = pi.FFN(**kw)
    hk = host_ffn(kw)
    g = torch.Generator(device="cuda").manual_seed(3 * n_tok + f)
    x = torch.randn((n_tok, d), generator=g, device="cuda").to(dtype)
    for density in (0.05, 0.5, 1.0):
        sel = torch.rand(f, generator=g, device="cuda") < density
        idx_list = torch.nonzero(sel).flatten().to(torch.int32)
        n = idx_list.numel()
        idx = torch.full((f,), -3, dtype=torch.int32, device="cuda")      # entries past the count are junk
        idx[:n] = idx_list
        cnt = torch.tensor([n], dtype=torch.int32, device="cuda")
        y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
        pi.sparse_ffn(ffn, x, idx, cnt, y)
        ref = oracle.sparse_ffn(host(x), host(idx_list), **hk)
        check_y(host(y), ref, TOL["f16"], f"mfma {act} d={d} f={f} n={n_tok} density={density}")


def test_mfma_empty_clamped_deterministic():
    d, f, n_tok = 1024, 800, 24
    kw = rand_ffn(d, f, "reglu", torch.float16, seed=5)
    ffn, hk = pi.FFN(**kw), host_ffn(kw)
    x = torch.randn((n_tok, d), device="cuda").to(torch.float16)
    s = np.flatnonzero(np.random.default_rng(2).random(f) < 0.4).astype(np.int32)
    idx = _i32(f)
    idx[:len(s)] = torch.as_tensor(s, device="cuda")

    def run(count, max_count=None, ytype=torch.float32):
        cnt = torch.tensor([count], dtype=torch.int32, device="cuda")
        y = torch.full((n_tok, d), float("nan"), dtype=ytype, device="cuda")
        pi.sparse_ffn(ffn, x, idx, cnt, y, max_count=max_count)
        return y

    assert torch.all(run(0) == 0)                                       # empty list: exact zeros
    check_y(host(run(len(s), max_count=37)), oracle.sparse_ffn(host(x), s[:37], **hk), TOL["f16"], "clamped")
    y1, y2 = run(len(s)), run(len(s))
    assert torch.equal(y1, y2)                                          # bitwise reproducible
    y16 = run(len(s), ytype=torch.float16)
    ref = oracle.sparse_ffn(host(x), s, **hk)
    check_y(host(y16), ref.astype(np.float16).astype(np.float64), TOL["f16"] + 1e-3, "fp16 out")


@pytest.mark.parametrize("act", ["relu", "reglu"])
def test_superset_all_empty_partition(act):
    dtype, d, f, n_tok = torch.float16, 1024, 2048, 2
    kw = rand_ffn(d, f, act, dtype, seed=3)
    ffn, hk = pi.FFN(**kw), host_ffn(kw)
    x = torch.randn((n_tok, d), device="cuda").to(dtype)
    y_dense, fired = oracle.dense_ffn(host(x), **hk)

    def run(idx_list, max_count=None):
        idx = _i32(f)
        idx[:len(idx_list)] = torch.as_tensor(np.asarray(idx_list, dtype=np.int32), device="cuda")
        cnt = torch.tensor([len(idx_list)], dtype=torch.int32, device="cuda")
        y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
        pi.sparse_ffn(ffn, x, idx, cnt, y, max_count=max_count)
        return host(y).astype(np.float64)

    # superset of the union of firing sets -> dense
    extra = np.random.default_rng(0).random(f) < 0.2
    sup = np.flatnonzero(fired.any(axis=0) | extra)
    check_y(run(sup), y_dense, TOL["f16"], "superset")
    check_y(run(np.arange(f)), y_dense, TOL["f16"], "all ones")
    # empty list: exact zeros
    assert np.all(run([]) == 0.0)
    # partition: two calls add up to one call
    s = np.flatnonzero(np.random.default_rng(1).random(f) < 0.3)
    a, b = s[::2], s[1::2]
    check_y(run(a) + run(b), run(s), 1e-5, "partition")
    # the pages' worked example: {3, 5} + {4} = {3, 4, 5}
    check_y(run([3, 5]) + run([4]), run([3, 4, 5]), 1e-6, "worked example")
    # a device count above max_count is clamped to max_count
    check_y(run(s, max_count=10), oracle.sparse_ffn(host(x), s[:10], **hk), TOL["f16"], "clamped count")


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------

def _layer_check(dl: DeviceLayer, n_tok: int, tokens_checked=None, stream_id=0, what=""):
    cfg = dl.cfg
    x = workload.make_tokens(cfg, 0, n_tok, "cuda", stream=stream_id)
    f, d = cfg.d_ff, cfg.d_model
    # the three calls one by one
    mask = torch.empty((n_tok, f), dtype=torch.uint8, device="cuda")
    logits = torch.empty((n_tok, f), dtype=torch.float32, device="cuda")
    pi.predict(dl.pred, x, cfg.tau, mask, logits)
    idx, cnt = _i32(f), _i32(1)
    pi.compact(mask, idx, cnt)
    y_sep = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    pi.sparse_ffn(dl.ffn, x, idx, cnt, y_sep)
    # and the fused layer call
    y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    ws = pi.alloc_workspace(dl.pred, dl.ffn, n_tok)
    pi.layer(dl.pred, dl.ffn, x, cfg.tau, y, ws=ws)
    assert pi.read_flags(ws) == 0, f"{what}: fault flags raised"
    check_layer_vs_calls(y, y_sep, layer_is_fused(cfg.wtype, d, cfg.rank, n_tok), what)

    h = dl.oracle_args()
    xs = host(x)
    ref_l, _ = oracle.predict(xs, h["p1"], h["p2"], h["c"], cfg.tau)
    in_band = check_mask(host(mask), ref_l, cfg.tau, what)
    c = int(cnt.item())
    ref_idx, ref_c = oracle.compact(host(mask))
    assert c == ref_c and np.array_equal(host(idx)[:c], ref_idx), f"{what}: list differs"
    rows = list(range(n_tok)) if tokens_checked is None else tokens_checked
    ref_y = oracle_sparse_chunked(xs[rows], ref_idx, h["ffn"])
    worst = check_y(host(y)[rows], ref_y, TOL[cfg.wtype], what)
    print(f"{what}: count={c} in-band mask flips={in_band} worst err={worst:.2e}", flush=True)


def test_layer_tiny():
    cfg = workload.get_config("tiny")
    _layer_check(DeviceLayer(cfg), n_tok=8, what="tiny n=8")
    dl = DeviceLayer(cfg)
    for s in range(3):
        _layer_check(dl, n_tok=1, stream_id=s + 1, what=f"tiny b1 #{s}")


@pytest.mark.parametrize("name", ["falcon40b", "opt30b", "llama70b"])
def test_layer_model_shape_b1(name):
    # One token per call: the launch configuration the benchmark times.
    cfg = workload.get_config(name)
    dl = DeviceLayer(cfg, layer=0)
    for s in range(2):
        _layer_check(dl, n_tok=1, stream_id=s, what=f"{name} b1 #{s}")


def test_layer_falcon_prompt64():
    cfg = workload.get_config("falcon40b")
    dl = DeviceLayer(cfg, layer=1)
    _layer_check(dl, n_tok=64, tokens_checked=[0, 17, 63], what="falcon prompt 64")


def test_layer_falcon_b2():
    # The fused single-tile kernel at 2 tokens and an ordinary threshold: the
    # union of two partly active masks is listed in-kernel.
    cfg = workload.get_config("falcon40b")
    dl = DeviceLayer(cfg, layer=3)
    for s in range(2):
        _layer_check(dl, n_tok=2, stream_id=s, what=f"falcon b2 #{s}")


@pytest.mark.parametrize("name,n_tok,rows", [
    ("tiny_relu2", 1, None), ("tiny_relu2", 2, None), ("tiny_relu2", 8, None),
    ("falcon40b_relu2", 1, None), ("falcon40b_relu2", 2, None), ("falcon40b_relu2", 8, [0, 3, 7]),
    ("falcon40b_relu2", 64, [0, 31, 63]),
])
def test_layer_relu2(name, n_tok, rows):
    # Squared ReLU through pi_layer: the fused kernel (1-2 tokens; tiny fp32 up
    # to 8) and the matrix-core path (8 and 64 fp16 tokens).
    cfg = workload.get_config(name)
    dl = DeviceLayer(cfg, layer=0)
    _layer_check(dl, n_tok=n_tok, tokens_checked=rows, what=f"{name} n={n_tok}")


@pytest.mark.parametrize("d", [1000, 1024])
@pytest.mark.parametrize("n_tok", [3, 4, 5, 8])
@pytest.mark.parametrize("act", ["relu", "reglu", "relu2"])
def test_layer_rank64_tiles(d, n_tok, act):
    # An fp16 predictor of rank 64 (not a multiple of 128: the VALU predictor
    # at any token count).  d = 1000: the FFN has no matrix-core path either,
    # so pi_layer runs the fused kernel on a tile of 3-8 tokens; d = 1024: the
    # FFN takes the matrix cores and pi_layer runs the three calls.
    f, r, tau = 2500, 64, 0.45
    g = torch.Generator(device="cuda").manual_seed(d + 13 * n_tok + len(act))
    p1 = (torch.randn((r, d), generator=g, device="cuda") * 0.05).half()
    p2 = (torch.randn((f, r), generator=g, device="cuda") * 0.2).half()
    c = (torch.randn(f, generator=g, device="cuda") * 0.5 - 1.2).float()
    kw = rand_ffn(d, f, act, torch.float16, seed=n_tok + d)
    pred, ffn, hk = pi.Predictor(p1, p2, c), pi.FFN(**kw), host_ffn(kw)
    x = torch.randn((n_tok, d), generator=g, device="cuda").half()
    mask = torch.empty((n_tok, f), dtype=torch.uint8, device="cuda")
    pi.predict(pred, x, tau, mask)
    idx, cnt = _i32(f), _i32(1)
    pi.compact(mask, idx, cnt)
    y_sep = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    pi.sparse_ffn(ffn, x, idx, cnt, y_sep)
    y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    ws = pi.alloc_workspace(pred, ffn, n_tok)
    pi.layer(pred, ffn, x, tau, y, ws=ws)
    assert pi.read_flags(ws) == 0
    check_layer_vs_calls(y, y_sep, layer_is_fused("f16", d, r, n_tok), f"rank64 d={d} n={n_tok}")
    ref_l, _ = oracle.predict(host(x), host(p1), host(p2), host(c), tau)
    check_mask(host(mask), ref_l, tau, f"rank64 n={n_tok}")
    c_ = int(cnt.item())
    ref_idx, ref_c = oracle.compact(host(mask))
    assert c_ == ref_c and np.array_equal(host(idx)[:c_], ref_idx)
    assert 0 < c_ < f
    check_y(host(y), oracle.sparse_ffn(host(x), ref_idx, **hk), TOL["f16"], f"rank64 d={d} n={n_tok} {act}")


@pytest.mark.parametrize("n_tok", [3, 5, 8, 20, 64, 70, 130])
@pytest.mark.parametrize("act", ["relu", "reglu"])
def test_layer_many_tokens(n_tok, act):
    # pi_layer with fp16 weights past the single-token tile: the matrix-core
    # predictor (its union mask, OR-ed over token tiles beyond 64 tokens), the
    # compaction of that one row, then the list path (<= 8 tokens) or the
    # matrix-core FFN; checked against predict + compact + sparse_ffn and the oracle.
    d, f, r, tau = 1024, 3000, 128, 0.45
    g = torch.Generator(device="cuda").manual_seed(17 * n_tok + len(act))
    p1 = (torch.randn((r, d), generator=g, device="cuda") * 0.05).half()
    p2 = (torch.randn((f, r), generator=g, device="cuda") * 0.05).half()
    c = (torch.randn(f, generator=g, device="cuda") * 0.5 - 1.0).float()
    kw = rand_ffn(d, f, act, torch.float16, seed=n_tok)
    pred, ffn, hk = pi.Predictor(p1, p2, c), pi.FFN(**kw), host_ffn(kw)
    x = torch.randn((n_tok, d), generator=g, device="cuda").half()
    mask = torch.empty((n_tok, f), dtype=torch.uint8, device="cuda")
    pi.predict(pred, x, tau, mask)
    idx, cnt = _i32(f), _i32(1)
    pi.compact(mask, idx, cnt)
    y_sep = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    pi.sparse_ffn(ffn, x, idx, cnt, y_sep)
    y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    pi.layer(pred, ffn, x, tau, y)
    torch.cuda.synchronize()
    assert torch.equal(y, y_sep), "pi_layer differs from predict + compact + sparse_ffn"
    ref_l, _ = oracle.predict(host(x), host(p1), host(p2), host(c), tau)
    check_mask(host(mask), ref_l, tau, f"layer n={n_tok}")
    c_ = int(cnt.item())
    ref_idx, ref_c = oracle.compact(host(mask))
    assert c_ == ref_c and np.array_equal(host(idx)[:c_], ref_idx)
    assert 0 < c_ < f
    check_y(host(y), oracle.sparse_ffn(host(x), ref_idx, **hk), TOL["f16"], f"layer n={n_tok} {act}")


@pytest.mark.parametrize("n_tok", [1, 2, 9])
def test_layer_degenerate_threshold(n_tok):
    # tau -> 0: every neuron is listed and pi_layer equals the dense FFN;
    # tau -> 1: nothing is listed and y is exactly zero.
    d, f, r = 512, 1536, 64
    g = torch.Generator(device="cuda").manual_seed(5 + n_tok)
    p1 = (torch.randn((r, d), generator=g, device="cuda") * 0.02).half()
    p2 = (torch.randn((f, r), generator=g, device="cuda") * 0.02).half()
    c = torch.zeros(f, dtype=torch.float32, device="cuda")
    kw = rand_ffn(d, f, "relu", torch.float16, seed=40 + n_tok)
    pred, ffn, hk = pi.Predictor(p1, p2, c), pi.FFN(**kw), host_ffn(kw)
    x = torch.randn((n_tok, d), generator=g, device="cuda").half()
    y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    pi.layer(pred, ffn, x, 1e-6, y)                 # theta = ln(1e-6 / (1 - 1e-6)), about -13.8
    y_dense, _ = oracle.dense_ffn(host(x), **hk)
    check_y(host(y), y_dense, TOL["f16"], "tau -> 0")
    y.fill_(float("nan"))
    pi.layer(pred, ffn, x, 1.0 - 1e-6, y)           # theta about +13.8
    torch.cuda.synchronize()
    assert torch.all(y == 0), "tau -> 1: nothing listed, y must be exact zeros"


@pytest.mark.parametrize("name,n_tok", [("falcon40b", 1), ("falcon40b", 8), ("falcon40b", 64),
                                         ("falcon40b_q4", 8)])
def test_determinism(name, n_tok):
    # Every sum has a fixed order, whatever grid numbering and k-walk start
    # each workgroup takes: repeated calls give the same bits (1 token: the
    # fused kernel; 8: k_mup / k_mdown; 64: k_mup_wide / k_mdown_w4).
    cfg = workload.get_config(name)
    dl = DeviceLayer(cfg, layer=2)
    x = workload.make_tokens(cfg, 2, n_tok, "cuda")
    ys = []
    for _ in range(3):
        y = torch.empty((n_tok, cfg.d_model), dtype=torch.float32, device="cuda")
        pi.layer(dl.pred, dl.ffn, x, cfg.tau, y)
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.isfinite(ys[0]).all()
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])


def test_binding_rejects_bad_tensors():
    cfg = workload.get_config("tiny")
    dl = DeviceLayer(cfg)
    x = workload.make_tokens(cfg, 0, 2, "cuda")
    y = torch.empty((2, cfg.d_model), dtype=torch.float32, device="cuda")
    with pytest.raises(pi.PiError):
        pi.layer(dl.pred, dl.ffn, x, 1.5, y)                    # tau out of range
    with pytest.raises(pi.PiError):
        ws = torch.empty(16, dtype=torch.uint8, device="cuda")
        pi.layer(dl.pred, dl.ffn, x, 0.5, y, ws=ws)             # workspace too small
    with pytest.raises(ValueError):
        pi.layer(dl.pred, dl.ffn, x.t(), 0.5, y)                # not contiguous / wrong shape
    with pytest.raises(TypeError):
        pi.layer(dl.pred, dl.ffn, x.half(), 0.5, y)             # wrong dtype
