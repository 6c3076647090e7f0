"""Shared helpers for the GPU parity tests: device inputs, host copies for the
oracle, and the comparison rules.

Comparison rules (applied per token):
  * index lists and counts: bit-exact;
  * predictor masks: equal wherever the oracle's float64 logit is farther
    than 1e-3 from the threshold logit;
  * FFN outputs: max_j |y_gpu - y_oracle| <= tol * max_j |y_oracle|, with
    tol = 2e-3 for fp16 weights, 5e-3 for Q4_0 and 1e-5 for fp32 (fp32
    accumulation of at most a few thousand terms is good to ~1e-6); when the
    oracle's y is exactly zero the GPU must write exact zeros.
"""

from __future__ import annotations

import numpy as np
import torch

import activation_sparse_rank_amd as pi
import oracle
import workload

TOL = {"f32": 1e-5, "f16": 2e-3, "q4_0": 5e-3}
BAND = 1e-3


def require_gpu():
    assert torch.cuda.is_available(), "GPU parity tests need an MI355X with ROCm"
    pi.load_library()


def host(t: torch.Tensor) -> np.ndarray:
    """Exact host copy of a device tensor."""
    return t.detach().cpu().numpy()


def wtag(dtype) -> str:
    return {torch.float32: "f32", torch.float16: "f16"}[dtype]


class DeviceLayer:
    """One generated layer on the GPU plus its bindings and host copies."""

    def __init__(self, cfg, layer=0, base_seed=0, device="cuda"):
        self.cfg = cfg
        self.L = workload.make_layer(cfg, layer, device, base_seed)
        L = self.L
        self.pred = pi.Predictor(L["p1"], L["p2"], L["c"])
        if cfg.wtype == "q4_0":
            d = cfg.d_model
            self.q = {k: pi.q4_0_repack(L[k], cfg.d_ff, d) for k in ("w_up", "w_down_t", "w_gate") if k in L}
            self.ffn = pi.FFN(self.q["w_up"], self.q["w_down_t"], cfg.act, b_up=L.get("b_up"),
                              w_gate=self.q.get("w_gate"), b_gate=L.get("b_gate"), d_model=d)
        else:
            self.ffn = pi.FFN(L["w_up"], L["w_down_t"], cfg.act, b_up=L.get("b_up"), w_gate=L.get("w_gate"),
                              b_gate=L.get("b_gate"))
        self._host = None

    def oracle_args(self):
        """Host copies (exact bits) in the form the oracle takes."""
        if self._host is None:
            L, cfg = self.L, self.cfg

            def w(k):
                if k not in L:
                    return None
                a = host(L[k])
                return oracle.Q4_0Matrix(a, cfg.d_model) if cfg.wtype == "q4_0" else a

            self._host = dict(
                p1=host(L["p1"]), p2=host(L["p2"]), c=host(L["c"]),
                ffn=dict(w_up=w("w_up"), w_down_t=w("w_down_t"), act=cfg.act,
                         b_up=host(L["b_up"]) if "b_up" in L else None,
                         w_gate=w("w_gate"), b_gate=host(L["b_gate"]) if "b_gate" in L else None),
            )
        return self._host


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, tol: float, what=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64).reshape(y_ref.shape)
    worst = 0.0
    for t in range(y_ref.shape[0]):
        scale = np.abs(y_ref[t]).max()
        if scale == 0.0:
            assert np.all(y_gpu[t] == 0.0), f"{what}: token {t}: oracle y is zero, GPU is not"
            continue
        err = np.abs(y_gpu[t] - y_ref[t]).max() / scale
        worst = max(worst, err)
        assert err <= tol, f"{what}: token {t}: max|err|/|y|inf = {err:.3e} > {tol:.1e}"
    return worst


def check_mask(mask_gpu: np.ndarray, logits_ref: np.ndarray, tau: float, what=""):
    """GPU mask vs the oracle's decision, ignoring the +-1e-3 logit band."""
    theta = oracle.logit_threshold(tau)
    mask_ref = logits_ref.astype(np.float32) > np.float32(theta)
    outside = np.abs(logits_ref - theta) > BAND
    bad = (mask_gpu.astype(bool) != mask_ref) & outside
    assert not bad.any(), f"{what}: {int(bad.sum())} mask entries differ outside the band"
    return int(((mask_gpu.astype(bool) != mask_ref) & ~outside).sum())


def oracle_sparse_chunked(x, idx, ffn_args, chunk=4096):
    """Oracle sparse FFN over a long list, summed over consecutive pieces of
    the list (the partition rule pinned in the oracle's own tests)."""
    idx = np.asarray(idx)
    y = None
    for s in range(0, max(1, idx.size), chunk):
        part = oracle.sparse_ffn(x, idx[s:s + chunk], **ffn_args)
        y = part if y is None else y + part
    return y


def rand_ffn(d, f, act, dtype, device="cuda", seed=0, with_bias=True):
    g = torch.Generator(device=device).manual_seed(seed)

    def m():
        return (torch.randn((f, d), generator=g, device=device) * 0.05).to(dtype)

    w_up, w_dt = m(), m()
    w_gate = m() if act == "reglu" else None
    b = (torch.randn(f, generator=g, device=device) * 0.3).float() if with_bias else None
    return dict(w_up=w_up, w_down_t=w_dt, act=act, b_up=None if act == "reglu" else b, w_gate=w_gate,
                b_gate=b if act == "reglu" else None)


def host_ffn(kw):
    return {k: (host(v) if isinstance(v, torch.Tensor) else v) for k, v in kw.items()}


def layer_is_fused(wtype: str, d: int, rank: int, n_tok: int) -> bool:
    """Whether pi_layer takes its fused single-tile path for these shapes (the
    dispatch rule the library documents): one token tile of the list path
    (8 tokens; Q4_0: x tile within 32 KB) within one predictor tile (t of
    the tile within 64 KB), where neither stand-alone call would use the
    matrix cores (fp16 / Q4_0 rows with d % 128 == 0 beyond 2 fp16 tokens or
    one Q4_0 tile; an fp16 predictor with d and rank multiples of 128 beyond
    2 tokens)."""
    tile = 8
    if wtype == "q4_0":
        while tile > 1 and tile * d * 2 > 32768:
            tile //= 2
    ptile = 8
    while ptile > 1 and ptile * rank > 16384:
        ptile //= 2
    pred_wtype = "f16" if wtype == "q4_0" else wtype
    pred_mfma = pred_wtype == "f16" and d % 128 == 0 and rank % 128 == 0 and n_tok > 2
    ffn_mfma = wtype in ("f16", "q4_0") and d % 128 == 0 and n_tok > (2 if wtype == "f16" else tile)
    return n_tok <= tile and n_tok <= ptile and not pred_mfma and not ffn_mfma


def check_layer_vs_calls(y: torch.Tensor, y_sep: torch.Tensor, fused: bool, what=""):
    """pi_layer against pi_predict + pi_compact + pi_sparse_ffn on the same
    input.  Off the fused path both run the same kernels on the same list:
    identical bits.  The fused path groups the down projection's chunks by
    segments of neurons instead of list positions, so its fp32 sums are
    added in another order: equal to about 1e-6 of max|y|."""
    if not fused:
        assert torch.equal(y, y_sep), f"{what}: pi_layer differs from predict+compact+sparse_ffn"
        return
    check_y(host(y), host(y_sep).astype(np.float64), 1e-5, f"{what}: pi_layer vs predict+compact+sparse_ffn")
