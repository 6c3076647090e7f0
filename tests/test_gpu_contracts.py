"""GPU checks of the contracts include/pi.h states beyond plain parity:

  * a NaN logit is inactive (pi_predict and pi_layer, VALU and matrix-core
    predictors);
  * an in-count idx entry outside [0, d_ff) adds nothing (pi_sparse_ffn on
    the list path, the matrix-core path and Q4_0 rows);
  * the fault flags: a bounded in-kernel wait that runs out (forced from the
    host through the workspace's test hooks, so every kernel still exits
    normally) raises PI_FLAG_WAIT_EXPIRED and makes y all NaN; a value of the
    matrix-core path that leaves the fp16 range raises PI_FLAG_FP16_RANGE;
    ordinary calls raise nothing; the fused single-tile path has no waits;
  * a call given a stream and no workspace allocates its temporary workspace
    on that stream.

Every call goes through the C ABI (the ctypes binding).
"""

import numpy as np
import pytest
import torch

import activation_sparse_rank_amd as pi
import oracle
from activation_sparse_rank_amd import _lib as L
from helpers import TOL, check_mask, check_y, host, host_ffn, rand_ffn, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _i32(n):
    return torch.zeros(n, dtype=torch.int32, device="cuda")


def _predictor(d, r, f, seed, p1_scale=0.05, c_shift=-1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    p1 = (torch.randn((r, d), generator=g, device="cuda") * p1_scale).half()
    p2 = (torch.randn((f, r), generator=g, device="cuda") * 0.1).half()
    c = (torch.randn(f, generator=g, device="cuda") * 0.5 + c_shift).float()
    return p1, p2, c


# ---------------------------------------------------------------------------
# A NaN logit is inactive
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n_tok", [1, 2, 8])
def test_nan_logit_inactive(n_tok):
    # n_tok 1-2: the VALU predictor and the fused layer kernel; 8: the
    # matrix-core predictor and its in-kernel list.
    d, r, f, tau = 1024, 128, 3000, 0.4
    p1, p2, c = _predictor(d, r, f, seed=31 + n_tok, c_shift=2.0)     # most neurons active
    nan_at = np.arange(5, f, 7)
    c[torch.as_tensor(nan_at, device="cuda")] = float("nan")
    kw = rand_ffn(d, f, "relu", torch.float16, seed=9)
    pred, ffn, hk = pi.Predictor(p1, p2, c), pi.FFN(**kw), host_ffn(kw)
    x = torch.randn((n_tok, d), device="cuda").half()
    mask = torch.empty((n_tok, f), dtype=torch.uint8, device="cuda")
    logits = torch.empty((n_tok, f), dtype=torch.float32, device="cuda")
    pi.predict(pred, x, tau, mask, logits)
    m = host(mask)
    assert np.isnan(host(logits)[:, nan_at]).all()
    assert not m[:, nan_at].any(), "a NaN logit was predicted active"
    ref_l, _ = oracle.predict(host(x), host(p1), host(p2), host(c), tau)
    check_mask(m, ref_l, tau, "nan logits")
    # the layer lists none of them and matches the oracle over its own list
    y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    ws = pi.alloc_workspace(pred, ffn, n_tok)
    pi.layer(pred, ffn, x, tau, y, ws=ws)
    assert pi.read_flags(ws) == 0
    ref_idx, ref_c = oracle.compact(m)
    assert not np.isin(nan_at, ref_idx).any() and ref_c > f // 2
    check_y(host(y), oracle.sparse_ffn(host(x), ref_idx, **hk), TOL["f16"], f"nan logits layer n={n_tok}")


# ---------------------------------------------------------------------------
# An in-count idx entry outside [0, d_ff) adds nothing
# ---------------------------------------------------------------------------

def _q4_ffn(d, f, seed, bias_shift=0.0):
    import workload
    rng = np.random.default_rng(seed)
    canon = {}
    for k in ("w_up", "w_down_t"):
        scales = (rng.standard_normal((f, d // 32)) * 0.01).astype(np.float16)
        codes = rng.integers(0, 16, size=(f, d), dtype=np.uint8)
        canon[k] = workload.q4_0_pack(torch.from_numpy(scales), torch.from_numpy(codes)).numpy()
    b = (rng.standard_normal(f) * 0.3 + bias_shift).astype(np.float32)
    dev = {k: pi.q4_0_repack(torch.from_numpy(v).cuda(), f, d) for k, v in canon.items()}
    ffn = pi.FFN(dev["w_up"], dev["w_down_t"], "relu", b_up=torch.from_numpy(b).cuda(), d_model=d)
    hk = dict(w_up=oracle.Q4_0Matrix(canon["w_up"], d), w_down_t=oracle.Q4_0Matrix(canon["w_down_t"], d),
              act="relu", b_up=b)
    return ffn, hk


@pytest.mark.parametrize("kind,n_tok", [("f32", 1), ("f16", 1), ("f16", 2), ("f16", 16), ("f16", 40),
                                        ("q4_0", 1), ("q4_0", 2), ("q4_0", 16)])
def test_out_of_range_entries_add_nothing(kind, n_tok):
    # The biases are shifted up so that the five good neurons fire well away
    # from zero: with so few rows, a neuron whose pre-activation is near zero
    # carries the fp16 rounding of the matrix-core path (H and Q4_0 weights in
    # fp16) into y unscaled, which a bound relative to max|y| does not cover.
    d, f = 1024, 900
    if kind == "q4_0":
        ffn, hk = _q4_ffn(d, f, seed=3 + n_tok, bias_shift=6.0)
        xdt = torch.float16
    else:
        dt = torch.float32 if kind == "f32" else torch.float16
        kw = rand_ffn(d, f, "relu", dt, seed=17 + n_tok)
        kw["b_up"] = kw["b_up"] + 6.0
        ffn, hk = pi.FFN(**kw), host_ffn(kw)
        xdt = dt
    g = torch.Generator(device="cuda").manual_seed(29 + n_tok)
    x = torch.randn((n_tok, d), generator=g, device="cuda").to(xdt)
    good = np.array([3, 5, 77, 400, 899], dtype=np.int32)
    lst = np.array([3, -1, 5, f, 77, -2147483648, 400, f + 12345, 899], dtype=np.int32)

    def run(entries):
        idx = torch.as_tensor(entries, device="cuda")
        cnt = torch.tensor([entries.size], dtype=torch.int32, device="cuda")
        y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
        pi.sparse_ffn(ffn, x, idx, cnt, y, max_count=entries.size)
        return y

    y, y_good = run(lst), run(good)
    ref = oracle.sparse_ffn(host(x), good, **hk)
    check_y(host(y), ref, TOL[kind], f"out-of-range entries {kind} n={n_tok}")
    # against the good entries alone: the same rows' terms, summed in another
    # grouping at most (the bad entries take list positions)
    check_y(host(y), host(y_good).astype(np.float64), 1e-6, f"out-of-range vs good only {kind} n={n_tok}")


# ---------------------------------------------------------------------------
# Fault flags
# ---------------------------------------------------------------------------

def _set_hooks(ws, polls, skip):
    w = ws.view(torch.int32)
    w[L.PI_WS_WAIT_POLLS] = polls
    w[L.PI_WS_SKIP_PUBLISH] = skip


def _expiry_layer(wtype, n_tok, seed):
    d, r, f = 1024, 128, 4096
    p1, p2, c = _predictor(d, r, f, seed=seed)
    pred = pi.Predictor(p1, p2, c)
    if wtype == "q4_0":
        ffn, _ = _q4_ffn(d, f, seed=5)
    else:
        ffn = pi.FFN(**rand_ffn(d, f, "relu", torch.float16, seed=8))
    x = torch.randn((n_tok, d), device="cuda").half()
    return pred, ffn, x


@pytest.mark.parametrize("n_tok", [8, 40])
def test_wait_expiry_is_reported(n_tok):
    # The matrix-core predictor lists the union in-kernel: one workgroup of
    # that list leaves its count unpublished and the waits are bounded to 4
    # polls, so every later workgroup gives up.  The call must raise
    # PI_FLAG_WAIT_EXPIRED and write NaN to all of y; after the flags are
    # cleared, the same call gives the normal result again.  (8 tokens: then
    # k_mup; 40: k_mup_wide.)
    tau = 0.45
    pred, ffn, x = _expiry_layer("f16", n_tok, seed=77 + n_tok)
    ws = pi.alloc_workspace(pred, ffn, n_tok)
    y_ok = torch.empty((n_tok, x.shape[1]), dtype=torch.float32, device="cuda")
    pi.layer(pred, ffn, x, tau, y_ok, ws=ws)
    assert pi.read_flags(ws) == 0
    assert torch.isfinite(y_ok).all()

    _set_hooks(ws, polls=4, skip=1 + 9)              # workgroup 9 never publishes
    y = torch.empty_like(y_ok)
    pi.layer(pred, ffn, x, tau, y, ws=ws)
    flags = pi.read_flags(ws)                        # synchronises: every kernel has exited
    assert flags & L.PI_FLAG_WAIT_EXPIRED, f"flags {flags:#x}"
    assert torch.isnan(y).all(), "y must be all NaN after a wait gave up"

    # the flag is sticky: a normal call leaves it set until it is cleared
    _set_hooks(ws, polls=0, skip=0)
    pi.layer(pred, ffn, x, tau, y, ws=ws)
    assert pi.read_flags(ws) & L.PI_FLAG_WAIT_EXPIRED
    assert torch.equal(y, y_ok)
    pi.clear_flags(ws)
    pi.layer(pred, ffn, x, tau, y, ws=ws)
    assert pi.read_flags(ws) == 0
    assert torch.equal(y, y_ok)


@pytest.mark.parametrize("wtype,n_tok", [("f16", 1), ("f16", 2), ("q4_0", 1)])
def test_fused_layer_never_waits(wtype, n_tok):
    # The fused single-tile path writes per-neuron slots and no workgroup
    # waits on another: the wait hooks change nothing, y stays bitwise the
    # same and no flag is raised.
    tau = 0.45
    pred, ffn, x = _expiry_layer(wtype, n_tok, seed=91 + n_tok)
    ws = pi.alloc_workspace(pred, ffn, n_tok)
    y_ok = torch.empty((n_tok, x.shape[1]), dtype=torch.float32, device="cuda")
    pi.layer(pred, ffn, x, tau, y_ok, ws=ws)
    _set_hooks(ws, polls=4, skip=1 + 9)
    y = torch.full_like(y_ok, float("nan"))
    pi.layer(pred, ffn, x, tau, y, ws=ws)
    assert pi.read_flags(ws) == 0
    assert torch.equal(y, y_ok)


@pytest.mark.parametrize("n_tok", [16, 40])
def test_fp16_range_flag_ffn(n_tok):
    # Squared ReLU of pre-activations of a few hundred exceeds fp16: the
    # matrix-core path's H (k_mup at 16 tokens, k_mfin at 40) is inf.
    d, f = 1024, 256
    g = torch.Generator(device="cuda").manual_seed(n_tok)
    w_up = (torch.randn((f, d), generator=g, device="cuda") * 3.0).half()
    w_dt = (torch.randn((f, d), generator=g, device="cuda") * 0.05).half()
    ffn = pi.FFN(w_up, w_dt, "relu2")
    x = torch.randn((n_tok, d), generator=g, device="cuda").half()
    idx = torch.arange(f, dtype=torch.int32, device="cuda")
    cnt = torch.tensor([f], dtype=torch.int32, device="cuda")
    y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    ws = pi.alloc_workspace(None, ffn, n_tok)
    pi.sparse_ffn(ffn, x, idx, cnt, y, ws=ws)
    assert pi.read_flags(ws) & L.PI_FLAG_FP16_RANGE
    assert not torch.isfinite(y).all()
    # the same products in range raise nothing
    ffn_ok = pi.FFN((w_up * 0.01).contiguous(), w_dt, "relu2")
    pi.clear_flags(ws)
    pi.sparse_ffn(ffn_ok, x, idx, cnt, y, ws=ws)
    assert pi.read_flags(ws) == 0 and torch.isfinite(y).all()


def test_fp16_range_flag_predictor():
    # t = p1 x of about 3e4 sigma: its fp16 split overflows on the matrix-core predictor.
    d, r, f, n_tok = 1024, 128, 500, 4
    p1, p2, c = _predictor(d, r, f, seed=3, p1_scale=1000.0)
    pred = pi.Predictor(p1, p2, c)
    x = torch.randn((n_tok, d), device="cuda").half()
    mask = torch.empty((n_tok, f), dtype=torch.uint8, device="cuda")
    ws = pi.alloc_workspace(pred, None, n_tok)
    pi.predict(pred, x, 0.5, mask, ws=ws)
    assert pi.read_flags(ws) & L.PI_FLAG_FP16_RANGE
    pred_ok = pi.Predictor((p1 * 0.001).contiguous(), p2, c)
    pi.clear_flags(ws)
    pi.predict(pred_ok, x, 0.5, mask, ws=ws)
    assert pi.read_flags(ws) == 0


# ---------------------------------------------------------------------------
# Temporary workspace on the call's stream
# ---------------------------------------------------------------------------

def test_side_stream_without_workspace():
    import workload
    cfg = workload.get_config("tiny")
    Lw = workload.make_layer(cfg, 0, "cuda")
    pred = pi.Predictor(Lw["p1"], Lw["p2"], Lw["c"])
    ffn = pi.FFN(Lw["w_up"], Lw["w_down_t"], "relu", b_up=Lw["b_up"])
    x = workload.make_tokens(cfg, 0, 3, "cuda")
    y_ref = torch.empty((3, cfg.d_model), dtype=torch.float32, device="cuda")
    pi.layer(pred, ffn, x, cfg.tau, y_ref, ws=pi.alloc_workspace(pred, ffn, 3))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ys = [torch.empty_like(y_ref) for _ in range(8)]
    for y in ys:
        pi.layer(pred, ffn, x, cfg.tau, y, stream=side)          # temporary workspace on `side`
        junk = torch.full((1 << 20,), 7, dtype=torch.uint8, device="cuda")   # reuses freed blocks on the current stream
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for y in ys:
        assert torch.equal(y, y_ref)
