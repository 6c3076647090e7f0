"""Seeded generators for weights, biases, decode tokens and masks.

Recipe (stated once here, used for every workload):

* Layer ``l`` of a stack with base seed ``s`` has seed ``s * 1_000_003 + l``;
  each generator is seeded with a SplitMix64 mix of (layer seed, purpose,
  stream) so weights, tokens and masks come from unrelated streams.
  Weights are i.i.d. normal with standard deviation 0.02 (``torch``
  generator on the target device, drawn in fixed 2048-row chunks in
  float32), rounded once to the storage type.  Draw order: ``p1``,
  ``p2``, ``w_gate`` (ReGLU only), ``w_up``, ``w_down_t``.
* Firing profile: neuron ``i`` gets a Zipf rank from a seeded permutation, and
  probability ``p_i = min(1, C * rank_i**-s)`` with ``C`` found by bisection so
  that ``mean(p) = rho``; ``p`` is capped at ``1 - 2**-20``.
* Biases place each neuron's firing probability at ``p_i`` for inputs
  ``x ~ N(0, I)``: the pre-activation of neuron ``i`` is then normal with
  standard deviation ``||w_i||``, so the bias ``||w_i|| * Phi^-1(p_i)`` makes
  it positive with probability ``p_i``; likewise the predictor bias is offset
  from the logit threshold by ``sigma_i * Phi^-1(p_i)`` with
  ``sigma_i**2 = p2_i^T (p1 p1^T) p2_i``.  Norms are taken in float64 from the
  stored (rounded, or quantized) weights; biases are then rounded to float32.
* Q4_0 weights: each 32-weight block of a float32 draw is quantized with scale
  ``d = fp16(amax / 7)`` and codes ``clamp(round_half_even(w / d) + 8, 0, 15)``
  (an all-zero block gets ``d = 0`` and codes 8), then packed into 18-byte
  blocks: little-endian fp16 scale, then 16 bytes, byte ``j`` holding code
  ``j`` in its low nibble and code ``j + 16`` in its high nibble.
* Decode tokens ``x ~ N(0, 1)``, per (layer, token), rounded once to the
  activation storage type; a separate generator stream per layer.
"""

from __future__ import annotations

import math

import numpy as np
import torch
from scipy.special import ndtri

from .configs import Config

_CHUNK_ROWS = 2048
_P_CAP = 1.0 - 2.0 ** -20
_TORCH_DT = {"f32": torch.float32, "f16": torch.float16}


def layer_seed(base_seed: int, layer: int) -> int:
    return int(base_seed) * 1_000_003 + int(layer)


def _mix(*parts: int) -> int:
    """SplitMix64 over the parts, folded to 31 bits.

    torch's CPU generator keeps only the low 32 bits of a seed, so seeds that
    differ only above bit 31 would replay the same stream; every generator is
    therefore seeded through this mix of (seed, purpose, stream).
    """
    h = 0x9E3779B97F4A7C15
    m = (1 << 64) - 1
    for v in parts:
        h = (h + (int(v) & m) + 0x9E3779B97F4A7C15) & m
        z = h
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
        h = z ^ (z >> 31)
    return h & 0x7FFFFFFF


_WEIGHTS, _TOKENS, _MASKS = 1, 2, 3


def zipf_profile(d_ff: int, rho: float, s: float = 1.1, seed: int = 0):
    """Zipf(s) firing probabilities with mean ``rho`` over randomly placed ranks.

    Returns ``(p [d_ff] float64, C, n_always_on)`` where ``n_always_on`` counts
    the neurons whose uncapped ``C * rank**-s`` reaches 1.
    """
    rng = np.random.default_rng(seed)
    ranks = rng.permutation(d_ff).astype(np.float64) + 1.0
    base = ranks ** (-float(s))

    def mean_p(C):
        return float(np.minimum(1.0, C * base).mean())

    lo, hi = 1e-12, 1e12
    for _ in range(300):
        mid = math.sqrt(lo * hi)
        if mean_p(mid) < rho:
            lo = mid
        else:
            hi = mid
    C = math.sqrt(lo * hi)
    p = np.minimum(1.0, C * base)
    n_on = int((p >= 1.0).sum())
    return np.minimum(p, _P_CAP), C, n_on


def _normal_rows(rows, cols, gen, device, std):
    """Yield ``(r0, r1, float32 chunk)`` of an i.i.d. N(0, std^2) matrix."""
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        chunk = torch.empty((r1 - r0, cols), dtype=torch.float32, device=device)
        chunk.normal_(mean=0.0, std=std, generator=gen)
        yield r0, r1, chunk


def q4_0_quantize(w: torch.Tensor):
    """Blockwise quantizer used only to *make* Q4_0 inputs.

    ``w`` is float32 ``[rows, cols]`` with ``cols % 32 == 0``.  Returns
    ``(scales fp16 [rows, cols/32], codes uint8 [rows, cols])``.
    """
    rows, cols = w.shape
    blk = w.reshape(rows, cols // 32, 32)
    amax = blk.abs().amax(dim=2)
    d = (amax / 7.0).to(torch.float16)
    df = d.to(torch.float32)
    safe = torch.where(df == 0, torch.ones_like(df), df)
    q = torch.round(blk / safe[:, :, None]) + 8.0
    q = torch.where(df[:, :, None] == 0, torch.full_like(q, 8.0), q)
    q = q.clamp_(0, 15).to(torch.uint8)
    return d, q.reshape(rows, cols)


def q4_0_pack(scales: torch.Tensor, codes: torch.Tensor) -> torch.Tensor:
    """Pack fp16 scales and 4-bit codes into canonical 18-byte Q4_0 blocks."""
    rows, cols = codes.shape
    nb = cols // 32
    c = codes.reshape(rows, nb, 32).to(torch.int32)
    packed = (c[:, :, :16] & 0x0F) | ((c[:, :, 16:] & 0x0F) << 4)        # [rows, nb, 16]
    bits = scales.contiguous().view(torch.int16).to(torch.int32) & 0xFFFF
    lo = (bits & 0xFF)[:, :, None]
    hi = ((bits >> 8) & 0xFF)[:, :, None]
    out = torch.cat([lo, hi, packed], dim=2).to(torch.uint8)
    return out.reshape(rows, nb * 18).contiguous()


def _stored_matrix(rows, cols, gen, device, std, wtype):
    """Draw a weight matrix; return ``(stored tensor, row L2 norms float64)``."""
    norms = torch.empty(rows, dtype=torch.float64, device=device)
    if wtype == "q4_0":
        if cols % 32:
            raise ValueError("Q4_0 needs cols % 32 == 0")
        out = torch.empty((rows, cols // 32 * 18), dtype=torch.uint8, device=device)
        for r0, r1, ch in _normal_rows(rows, cols, gen, device, std):
            d, q = q4_0_quantize(ch)
            k = q.to(torch.float64).reshape(r1 - r0, cols // 32, 32) - 8.0
            sq = d.to(torch.float64) ** 2 * (k * k).sum(dim=2)
            norms[r0:r1] = sq.sum(dim=1).sqrt()
            out[r0:r1] = q4_0_pack(d, q)
        return out, norms
    dt = _TORCH_DT[wtype]
    out = torch.empty((rows, cols), dtype=dt, device=device)
    for r0, r1, ch in _normal_rows(rows, cols, gen, device, std):
        st = ch.to(dt)
        out[r0:r1] = st
        norms[r0:r1] = st.to(torch.float64).pow(2).sum(dim=1).sqrt()
    return out, norms


def make_layer(cfg: Config, layer: int = 0, device="cpu", base_seed: int = 0):
    """All weights of one layer, on ``device``.

    Keys: ``p1`` [r, d], ``p2`` [d_ff, r], ``c`` fp32 [d_ff]; ``w_up``,
    ``w_down_t`` (and ``w_gate`` for ReGLU) as [d_ff, d] in the storage type
    (uint8 canonical Q4_0 blocks [d_ff, d/32*18] for Q4_0); ``b_up`` (ReLU,
    squared ReLU) or ``b_gate`` (ReGLU) fp32 [d_ff]; ``p`` the float64 firing
    profile (numpy); ``seed``.
    """
    seed = layer_seed(base_seed, layer)
    gen = torch.Generator(device=device)
    gen.manual_seed(_mix(seed, _WEIGHTS))
    d, f, r = cfg.d_model, cfg.d_ff, cfg.rank
    out = {"seed": seed}
    p1, _ = _stored_matrix(r, d, gen, device, cfg.w_std, cfg.pred_wtype)
    p2, _ = _stored_matrix(f, r, gen, device, cfg.w_std, cfg.pred_wtype)
    if cfg.act == "reglu":
        w_gate, gate_norm = _stored_matrix(f, d, gen, device, cfg.w_std, cfg.wtype)
    w_up, up_norm = _stored_matrix(f, d, gen, device, cfg.w_std, cfg.wtype)
    w_down_t, _ = _stored_matrix(f, d, gen, device, cfg.w_std, cfg.wtype)

    p, _, _ = zipf_profile(f, cfg.rho, cfg.zipf_s, seed)
    z = torch.from_numpy(ndtri(p)).to(device=device, dtype=torch.float64)

    # Predictor bias: logit is normal with std sigma_i around c_i; offset from
    # the logit threshold ln(tau/(1-tau)) by sigma_i * Phi^-1(p_i).
    p1d = p1.to(torch.float64)
    G = p1d @ p1d.T
    sig2 = torch.empty(f, dtype=torch.float64, device=device)
    for r0 in range(0, f, _CHUNK_ROWS):
        r1 = min(f, r0 + _CHUNK_ROWS)
        q = p2[r0:r1].to(torch.float64)
        sig2[r0:r1] = ((q @ G) * q).sum(dim=1)
    logit_tau = math.log(cfg.tau) - math.log1p(-cfg.tau)
    out["c"] = (logit_tau + sig2.clamp_min(0).sqrt() * z).to(torch.float32)

    norm = gate_norm if cfg.act == "reglu" else up_norm
    bias = (norm * z).to(torch.float32)
    out.update(p1=p1, p2=p2, w_up=w_up, w_down_t=w_down_t, p=p)
    if cfg.act == "reglu":
        out.update(w_gate=w_gate, b_gate=bias)
    else:
        out.update(b_up=bias)
    return out


def make_tokens(cfg: Config, layer: int, n_tok: int, device="cpu", base_seed: int = 0, stream: int = 0):
    """``n_tok`` decode inputs ``x ~ N(0, 1)`` for one layer, stored type."""
    gen = torch.Generator(device=device)
    gen.manual_seed(_mix(layer_seed(base_seed, layer), _TOKENS, stream))
    x = torch.empty((n_tok, cfg.d_model), dtype=torch.float32, device=device)
    x.normal_(mean=0.0, std=1.0, generator=gen)
    return x.to(_TORCH_DT[cfg.x_dtype])


def bernoulli_mask(p, n_tok: int, seed: int, device="cpu") -> torch.Tensor:
    """uint8 ``[n_tok, d_ff]`` masks with ``P[mask[t, i] = 1] = p_i``."""
    gen = torch.Generator(device=device)
    gen.manual_seed(_mix(seed, _MASKS))
    pt = torch.as_tensor(np.asarray(p), dtype=torch.float64, device=device)
    u = torch.empty((n_tok, pt.numel()), dtype=torch.float64, device=device)
    u.uniform_(0.0, 1.0, generator=gen)
    return (u < pt[None, :]).to(torch.uint8)
