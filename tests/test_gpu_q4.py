"""GPU parity for Q4_0 weights: the repacked layout (bit-exact against the
layout's definition), the sparse FFN over random Q4_0 blocks, and whole
layers of the Q4_0 model shapes, all against the CPU oracle.

Q4_0 ([GN] "Lượng tử hóa và tương thích"): blocks of 32 weights with one fp16
scale d; code q stands for d*(q-8).
"""

import numpy as np
import pytest
import torch

import activation_sparse_rank_amd as pi
import oracle
import workload
from helpers import (TOL, DeviceLayer, check_layer_vs_calls, check_mask, check_y, host, layer_is_fused,
                     oracle_sparse_chunked, require_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _i32(n):
    return torch.zeros(n, dtype=torch.int32, device="cuda")


def rand_q4(rows, cols, seed, zero_blocks=True):
    """Canonical Q4_0 blocks with uniform codes and mixed-sign fp16 scales
    (some zero), built with the workload packer."""
    rng = np.random.default_rng(seed)
    nb = cols // 32
    scales = (rng.standard_normal((rows, nb)) * 0.01).astype(np.float16)
    if zero_blocks:
        scales[rng.random((rows, nb)) < 0.02] = 0
    codes = rng.integers(0, 16, size=(rows, cols), dtype=np.uint8)
    return workload.q4_0_pack(torch.from_numpy(scales), torch.from_numpy(codes)).numpy()


def expected_repack(blocks: np.ndarray, cols: int) -> np.ndarray:
    """The repacked layout written out from its definition: code groups
    [rows][nb][16] (word k holds pairs 4k+u: code 2p at bits 4u, code 2p+1 at
    bits 16+4u), then scales [rows][nb]."""
    rows = blocks.shape[0]
    nb = cols // 32
    b = blocks.reshape(rows, nb, 18)
    scale_bytes = b[:, :, :2].reshape(rows * nb * 2)
    lo, hi = b[:, :, 2:] & 0xF, b[:, :, 2:] >> 4
    codes = np.concatenate([lo, hi], axis=2).astype(np.uint32)      # code j, j = 0..31
    words = np.zeros((rows, nb, 4), dtype=np.uint32)
    for k in range(4):
        for u in range(4):
            p = 4 * k + u
            words[:, :, k] |= codes[:, :, 2 * p] << (4 * u)
            words[:, :, k] |= codes[:, :, 2 * p + 1] << (16 + 4 * u)
    return np.concatenate([words.astype("<u4").view(np.uint8).reshape(-1), scale_bytes])


@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 96), (300, 1056), (33, 8192)])
def test_repack_layout(rows, cols):
    blocks = rand_q4(rows, cols, seed=rows + cols)
    dst = pi.q4_0_repack(torch.from_numpy(blocks).cuda(), rows, cols)
    torch.cuda.synchronize()
    assert np.array_equal(host(dst).reshape(-1), expected_repack(blocks, cols))


def _q4_ffn(d, f, act, seed):
    rng = np.random.default_rng(seed)
    canon = {k: rand_q4(f, d, seed + i) for i, k in enumerate(["w_up", "w_down_t"] + (["w_gate"] if act == "reglu" else []))}
    b = (rng.standard_normal(f) * 0.3).astype(np.float32)
    dev = {k: pi.q4_0_repack(torch.from_numpy(v).cuda(), f, d) for k, v in canon.items()}
    bias = torch.from_numpy(b).cuda()
    ffn = pi.FFN(dev["w_up"], dev["w_down_t"], act, b_up=None if act == "reglu" else bias, w_gate=dev.get("w_gate"),
                 b_gate=bias if act == "reglu" else None, d_model=d)
    hk = dict(w_up=oracle.Q4_0Matrix(canon["w_up"], d), w_down_t=oracle.Q4_0Matrix(canon["w_down_t"], d), act=act,
              b_up=None if act == "reglu" else b,
              w_gate=oracle.Q4_0Matrix(canon["w_gate"], d) if act == "reglu" else None,
              b_gate=b if act == "reglu" else None)
    return ffn, hk, dev


Q4_SHAPES = [
    (256, 1000),     # one partial slice of the down kernel
    (1056, 700),     # 33 blocks: a full 1024-column slice plus a ragged one
    (8192, 300),     # model width: x tiles of 2 tokens in LDS
    (16416, 200),    # 513 blocks: two passes of the up kernel, x read from global memory
]


@pytest.mark.parametrize("d,f", Q4_SHAPES)
@pytest.mark.parametrize("act", ["relu", "reglu", "relu2"])
@pytest.mark.parametrize("n_tok", [1, 2, 3, 8, 11])
def test_sparse_ffn_q4(d, f, act, n_tok):
    ffn, hk, _ = _q4_ffn(d, f, act, seed=d + f + n_tok)
    g = torch.Generator(device="cuda").manual_seed(5 * n_tok + f)
    x = torch.randn((n_tok, d), generator=g, device="cuda").to(torch.float16)
    for density in (0.1, 0.7):
        sel = torch.rand(f, generator=g, device="cuda") < density
        idx_list = torch.nonzero(sel).flatten().to(torch.int32)
        n = idx_list.numel()
        idx = _i32(f)
        idx[:n] = idx_list
        cnt = torch.tensor([n], dtype=torch.int32, device="cuda")
        y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
        pi.sparse_ffn(ffn, x, idx, cnt, y)
        ref = oracle.sparse_ffn(host(x), host(idx_list), **hk)
        check_y(host(y), ref, TOL["q4_0"], f"q4 {act} d={d} f={f} n={n_tok} density={density}")


@pytest.mark.parametrize("d,f", [(1024, 900), (8192, 500), (640, 300)])
@pytest.mark.parametrize("act", ["relu", "reglu"])
@pytest.mark.parametrize("n_tok", [3, 8, 9, 16, 17, 32, 33, 64, 70])
def test_sparse_ffn_q4_mfma(d, f, act, n_tok):
    # More tokens than one list-path pass: the matrix-core path (k_mup +
    # k_mdown up to 16 tokens, the wide kernels from 17, two tiles past 64).
    # d = 640 leaves the last column tile of the down projections part
    # empty (256 and 512 columns per tile), so those lanes read a stand-in
    # column and add nothing.
    ffn, hk, _ = _q4_ffn(d, f, act, seed=d + 7 * f + n_tok)
    g = torch.Generator(device="cuda").manual_seed(11 * n_tok + f)
    x = torch.randn((n_tok, d), generator=g, device="cuda").to(torch.float16)
    for density in (0.05, 0.4):
        sel = torch.rand(f, generator=g, device="cuda") < density
        idx_list = torch.nonzero(sel).flatten().to(torch.int32)
        n = idx_list.numel()
        idx = _i32(f)
        idx[:n] = idx_list
        cnt = torch.tensor([n], dtype=torch.int32, device="cuda")
        y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
        pi.sparse_ffn(ffn, x, idx, cnt, y)
        ref = oracle.sparse_ffn(host(x), host(idx_list), **hk)
        check_y(host(y), ref, TOL["q4_0"], f"q4 mfma {act} d={d} f={f} n={n_tok} density={density}")


@pytest.mark.parametrize("d", [1152, 2048, 4096])
@pytest.mark.parametrize("act", ["relu", "reglu"])
@pytest.mark.parametrize("n_tok", [9, 16])
def test_q4_mup_chunking(d, act, n_tok):
    # The matrix-core up projection at up to 16 tokens walks each wave's
    # quarter of d in chunks of k steps (8, or 4 with gate rows), with the
    # chunk's scales in one load and the code groups by transposed loads;
    # quarters that are not whole chunks, or rows whose scales are not
    # 16-byte aligned (d % 256 != 0), take the step-by-step loads instead.
    # d = 1152: 9 steps, ragged quarters, unaligned scales; 2048: quarters of
    # 4 steps (one gated chunk, step-by-step without gate); 4096: quarters of
    # 8 steps (one chunk, or two gated chunks).
    f = 600
    ffn, hk, _ = _q4_ffn(d, f, act, seed=3 * d + n_tok)
    g = torch.Generator(device="cuda").manual_seed(d + n_tok)
    x = torch.randn((n_tok, d), generator=g, device="cuda").to(torch.float16)
    sel = torch.rand(f, generator=g, device="cuda") < 0.3
    idx_list = torch.nonzero(sel).flatten().to(torch.int32)
    n = idx_list.numel()
    idx = _i32(f)
    idx[:n] = idx_list
    cnt = torch.tensor([n], dtype=torch.int32, device="cuda")
    y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    pi.sparse_ffn(ffn, x, idx, cnt, y)
    ref = oracle.sparse_ffn(host(x), host(idx_list), **hk)
    check_y(host(y), ref, TOL["q4_0"], f"q4 mup chunking {act} d={d} n={n_tok}")


def test_q4_empty_and_all():
    d, f, n_tok = 1024, 512, 3
    ffn, hk, _ = _q4_ffn(d, f, "reglu", seed=11)
    x = torch.randn((n_tok, d), device="cuda").to(torch.float16)
    y_dense, _ = oracle.dense_ffn(host(x), **hk)
    for lst, ref in ((np.arange(f), y_dense), (np.zeros(0, dtype=np.int64), np.zeros_like(y_dense))):
        idx = _i32(f)
        idx[:len(lst)] = torch.as_tensor(lst.astype(np.int32), device="cuda")
        cnt = torch.tensor([len(lst)], dtype=torch.int32, device="cuda")
        y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
        pi.sparse_ffn(ffn, x, idx, cnt, y)
        check_y(host(y), ref, TOL["q4_0"], f"q4 list of {len(lst)}")


def _layer_check(dl, n_tok, rows=None, stream_id=0, what=""):
    cfg = dl.cfg
    x = workload.make_tokens(cfg, 0, n_tok, "cuda", stream=stream_id)
    f, d = cfg.d_ff, cfg.d_model
    mask = torch.empty((n_tok, f), dtype=torch.uint8, device="cuda")
    logits = torch.empty((n_tok, f), dtype=torch.float32, device="cuda")
    pi.predict(dl.pred, x, cfg.tau, mask, logits)
    idx, cnt = _i32(f), _i32(1)
    pi.compact(mask, idx, cnt)
    y_sep = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    pi.sparse_ffn(dl.ffn, x, idx, cnt, y_sep)
    y = torch.empty((n_tok, d), dtype=torch.float32, device="cuda")
    ws = pi.alloc_workspace(dl.pred, dl.ffn, n_tok)
    pi.layer(dl.pred, dl.ffn, x, cfg.tau, y, ws=ws)
    assert pi.read_flags(ws) == 0, f"{what}: fault flags raised"
    check_layer_vs_calls(y, y_sep, layer_is_fused(cfg.wtype, d, cfg.rank, n_tok), what)
    h = dl.oracle_args()
    xs = host(x)
    ref_l, _ = oracle.predict(xs, h["p1"], h["p2"], h["c"], cfg.tau)
    check_mask(host(mask), ref_l, cfg.tau, what)
    c = int(cnt.item())
    ref_idx, ref_c = oracle.compact(host(mask))
    assert c == ref_c and np.array_equal(host(idx)[:c], ref_idx), f"{what}: list differs"
    rows = list(range(n_tok)) if rows is None else rows
    worst = check_y(host(y)[rows], oracle_sparse_chunked(xs[rows], ref_idx, h["ffn"]), TOL["q4_0"], what)
    print(f"{what}: count={c} worst err={worst:.2e}", flush=True)


@pytest.mark.parametrize("name", ["falcon40b_q4", "llama70b_q4"])
def test_layer_q4_model_shape(name):
    cfg = workload.get_config(name)
    dl = DeviceLayer(cfg, layer=0)
    _layer_check(dl, n_tok=1, what=f"{name} b1")
    # two tokens: the fused kernel's Q4_0 tile of 2 (x of both tokens in LDS)
    _layer_check(dl, n_tok=2, stream_id=2, what=f"{name} b2")
    _layer_check(dl, n_tok=8, rows=[0, 5, 7], stream_id=1, what=f"{name} b8")


@pytest.mark.parametrize("n_tok", [17, 64])
def test_layer_q4_wide(n_tok):
    # Many tokens: the matrix-core predictor leaves the token tile in the
    # block order Q4_0 rows meet, and the wide FFN kernels read that copy;
    # the separate calls copy the tokens themselves.  Both must give the
    # same bits, and the sampled tokens must match the oracle.
    cfg = workload.get_config("falcon40b_q4")
    dl = DeviceLayer(cfg, layer=0)
    _layer_check(dl, n_tok=n_tok, rows=[0, n_tok - 1], stream_id=3, what=f"falcon40b_q4 n={n_tok}")
