"""The oracle's definitions, one function per step of the decode hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

Notation.  One token's input is ``x`` (length ``d``).  The FFN has ``d_ff``
neurons; neuron ``i`` owns row ``i`` of ``w_up`` (and of ``w_gate`` for ReGLU),
a bias, and row ``i`` of ``w_down_t`` -- the transposed down projection, so
that row ``i`` holds the weights neuron ``i`` adds into every output.  The
predictor is ``p1`` (``r x d``), ``p2`` (``d_ff x r``) and a bias ``c``.
Several tokens are stacked as rows of ``x`` (shape ``n x d``).

All arithmetic is float64.  Source tags [GN], [QB], [AB] are defined in the
package docstring.
"""

from __future__ import annotations

import math

import numpy as np

ACTIVATIONS = ("relu", "reglu", "relu2")


def to_f64(a) -> np.ndarray:
    """Exact widening of a stored array (fp16, fp32 or integer) to float64."""
    a = np.asarray(a)
    if a.dtype == np.float64:
        return a
    if a.dtype in (np.float16, np.float32) or np.issubdtype(a.dtype, np.integer):
        return a.astype(np.float64)
    raise TypeError(f"oracle: unsupported stored dtype {a.dtype}")


def _as_tokens(x) -> np.ndarray:
    x = to_f64(x)
    return x[None, :] if x.ndim == 1 else x


# --------------------------------------------------------------------------
# Q4_0 blocks
# --------------------------------------------------------------------------

Q4_0_BLOCK = 32          # weights per block
Q4_0_BYTES = 18          # fp16 scale + 16 bytes of 4-bit codes


def q4_0_dequant(blocks, cols: int) -> np.ndarray:
    """Decode rows of Q4_0 blocks into float64 weights.

    [GN] section "Lượng tử hóa và tương thích" names INT4 Q4_0 as the supported
    quantized format; the pages give no byte layout.  The layout read here:
    each row of ``cols`` weights is ``cols/32`` consecutive 18-byte blocks; a
    block starts with its scale ``d`` as a little-endian IEEE fp16, followed by
    16 bytes; byte ``j`` carries weight ``j`` of the block in its low nibble and
    weight ``j + 16`` in its high nibble; a stored code ``q`` in 0..15 means the
    weight ``d * (q - 8)``.
    """
    b = np.ascontiguousarray(np.asarray(blocks, dtype=np.uint8))
    if b.ndim == 1:
        b = b[None, :]
    if cols % Q4_0_BLOCK:
        raise ValueError("oracle: Q4_0 rows must hold a whole number of 32-weight blocks")
    nb = cols // Q4_0_BLOCK
    if b.shape[1] != nb * Q4_0_BYTES:
        raise ValueError("oracle: Q4_0 row byte length does not match cols")
    blk = b.reshape(b.shape[0], nb, Q4_0_BYTES)
    scale = blk[:, :, 0:2].copy().view("<f2")[:, :, 0].astype(np.float64)   # [rows, nb]
    codes = blk[:, :, 2:].astype(np.int64)                                   # [rows, nb, 16]
    low = codes & 0x0F          # weights 0..15 of the block
    high = codes >> 4           # weights 16..31 of the block
    q = np.concatenate([low, high], axis=2)                                  # [rows, nb, 32]
    w = scale[:, :, None] * (q.astype(np.float64) - 8.0)
    return w.reshape(b.shape[0], cols)


class Q4_0Matrix:
    """A ``rows x cols`` weight matrix held as canonical Q4_0 block bytes."""

    def __init__(self, blocks, cols: int):
        self.blocks = np.asarray(blocks, dtype=np.uint8)
        self.cols = int(cols)

    @property
    def shape(self):
        return (self.blocks.shape[0], self.cols)

    def rows(self, idx) -> np.ndarray:
        return q4_0_dequant(self.blocks[np.asarray(idx, dtype=np.int64)], self.cols)

    def dense(self) -> np.ndarray:
        return q4_0_dequant(self.blocks, self.cols)


def _rows(w, idx) -> np.ndarray:
    """Rows ``idx`` of a stored weight matrix, widened to float64."""
    if isinstance(w, Q4_0Matrix):
        return w.rows(idx)
    return to_f64(np.asarray(w)[np.asarray(idx, dtype=np.int64)])


def _all_rows(w) -> np.ndarray:
    if isinstance(w, Q4_0Matrix):
        return w.dense()
    return to_f64(w)


# --------------------------------------------------------------------------
# Activation of a set of neurons
# --------------------------------------------------------------------------

def _neurons(x, act, up_rows, b_up, gate_rows, b_gate):
    """Per-neuron output ``h`` and firing flag for the given neuron rows.

    ReLU ([GN] first section; [QB] section "Что такое «разреженная
    активация»?"): ``z = w_up_i . x + b_up_i``, ``h = max(z, 0)``, the neuron
    fires when ``z > 0``.  Squared ReLU ([GN] "Hạn chế và FAQ" lists it as
    supported): ``h = max(z, 0)**2`` with the same firing rule.  ReGLU (the
    LLaMA(ReGLU) models of [QB] "Локальность вывода..."): gate
    ``g = w_gate_i . x + b_gate_i``, ``u = w_up_i . x`` (no bias),
    ``h = max(g, 0) * u``; the neuron fires when ``g > 0``.
    Returns ``h`` and ``fired``, both ``[n_tok, n_rows]``.
    """
    if act not in ACTIVATIONS:
        raise ValueError(f"oracle: unknown activation {act!r}")
    if act in ("relu", "relu2"):
        z = x @ up_rows.T
        if b_up is not None:
            z = z + b_up[None, :]
        fired = z > 0.0
        pos = np.maximum(z, 0.0)
        h = pos if act == "relu" else pos * pos
    else:
        g = x @ gate_rows.T
        if b_gate is not None:
            g = g + b_gate[None, :]
        u = x @ up_rows.T
        fired = g > 0.0
        h = np.maximum(g, 0.0) * u
    return h, fired


# --------------------------------------------------------------------------
# O1: the dense FFN and its true firing set
# --------------------------------------------------------------------------

def dense_ffn(x, w_up, w_down_t, act="relu", b_up=None, w_gate=None, b_gate=None):
    """Dense FFN: every neuron computed.  Returns ``(y [n, d], fired [n, d_ff])``.

    ``y_j = sum_i w_down_t[i, j] * h_i`` over all ``d_ff`` neurons.  This is
    the result the sparse method must reproduce when it computes a superset of
    the neurons that fire ([QB] "Что такое «разреженная активация»?": the
    non-activated neurons add nothing material to the output).
    """
    x = _as_tokens(x)
    up = _all_rows(w_up)
    gate = _all_rows(w_gate) if act == "reglu" else None
    bu = to_f64(b_up) if b_up is not None else None
    bg = to_f64(b_gate) if b_gate is not None else None
    h, fired = _neurons(x, act, up, bu, gate, bg)
    y = h @ _all_rows(w_down_t)
    return y, fired


# --------------------------------------------------------------------------
# O2: the activation predictor and its threshold
# --------------------------------------------------------------------------

def logit_threshold(tau: float) -> float:
    """``sigmoid(l) > tau`` holds exactly when ``l > ln(tau / (1 - tau))``.

    The sigmoid is strictly increasing, so its threshold maps to one logit.
    """
    tau = float(tau)
    if not (0.0 < tau < 1.0):
        raise ValueError("oracle: tau must lie strictly between 0 and 1")
    return math.log(tau / (1.0 - tau))


def sigmoid(v):
    v = to_f64(v)
    out = np.empty_like(v)
    pos = v >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-v[pos]))
    e = np.exp(v[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def predict(x, p1, p2, c, tau, decide=np.float32):
    """Per-layer activation predictor: which neurons will this input fire?

    [QB] sections "Что такое «разреженная активация»?" and "Гибридный дизайн
    вывода CPU/GPU": a small per-layer model, trained offline, predicts the
    neurons an input activates and only those are computed; [GN] "Cách suy
    luận lai CPU/GPU" and [AB] "Aprofundamento nos Princípios Técnicos" call it
    an (adaptive, lightweight) predictor.  The pages give no architecture; the
    reading used is a low-rank linear pair with a sigmoid threshold:
    ``t = p1 x`` (no bias, no nonlinearity between the two products),
    ``l_i = p2_i . t + c_i``, neuron ``i`` predicted active when
    ``sigmoid(l_i) > tau``, i.e. ``l_i > theta`` with ``theta = ln(tau/(1-tau))``.

    The logits are float64.  The active/inactive decision is taken in the
    precision named by ``decide`` (float32 by default, the precision the GPU
    compares in): ``float32(l_i) > float32(theta)``.  A NaN logit is inactive.
    Returns ``(logits [n, d_ff] float64, mask [n, d_ff] bool)``.
    """
    x = _as_tokens(x)
    t = x @ _all_rows(p1).T                     # [n, r]
    logits = t @ to_f64(p2).T + to_f64(c)[None, :]
    theta = logit_threshold(tau)
    if decide is None or decide == np.float64:
        mask = logits > theta
    else:
        mask = logits.astype(decide) > np.asarray(theta, dtype=decide)
    return logits, mask


# --------------------------------------------------------------------------
# O3: compaction of a mask into an index list
# --------------------------------------------------------------------------

def compact(mask):
    """Ascending list of the neurons a mask marks, and its length.

    The worked example of [QB] "Гибридный дизайн вывода CPU/GPU" names the
    predicted set as the neuron numbers {3, 4, 5}; the list form keeps that
    set in ascending order.  A mask entry counts as set when it is nonzero.
    With several tokens (rows of ``mask``) the set is the union over tokens:
    neuron ``i`` is listed when any token marks it.
    """
    m = np.asarray(mask)
    if m.ndim == 1:
        m = m[None, :]
    n_tok, d_ff = m.shape
    union = np.zeros(d_ff, dtype=bool)
    for t in range(n_tok):
        union |= m[t] != 0
    idx = [i for i in range(d_ff) if union[i]]
    return np.asarray(idx, dtype=np.int32), len(idx)


# --------------------------------------------------------------------------
# O4: the sparse FFN over a list of neurons
# --------------------------------------------------------------------------

def sparse_ffn(x, idx, w_up, w_down_t, act="relu", b_up=None, w_gate=None, b_gate=None):
    """FFN restricted to the listed neurons; unlisted neurons contribute 0.

    [QB] "Что такое «разреженная активация»?" and "Гибридный дизайн вывода
    CPU/GPU": only the predicted neurons are computed; [AB] "Princípios
    Técnicos Fundamentais": hot and cold neurons each compute their share.
    For every token ``t`` and every listed neuron ``i`` the neuron output
    ``h_{t,i}`` is evaluated exactly as in the dense FFN, and
    ``y_t = sum_{i in idx} w_down_t[i] * h_{t,i}``.  With several tokens one
    list serves all of them and each token evaluates every listed neuron with
    its own input.  Returns ``y [n, d]`` (zeros when the list is empty).
    """
    x = _as_tokens(x)
    idx = np.asarray(idx, dtype=np.int64).reshape(-1)
    d = x.shape[1]
    if idx.size == 0:
        return np.zeros((x.shape[0], d), dtype=np.float64)
    up = _rows(w_up, idx)
    gate = _rows(w_gate, idx) if act == "reglu" else None
    bu = to_f64(b_up)[idx] if b_up is not None else None
    bg = to_f64(b_gate)[idx] if b_gate is not None else None
    h, _ = _neurons(x, act, up, bu, gate, bg)
    return h @ _rows(w_down_t, idx)


# --------------------------------------------------------------------------
# O6: one layer = predictor, compaction, sparse FFN
# --------------------------------------------------------------------------

def layer(x, p1, p2, c, tau, w_up, w_down_t, act="relu", b_up=None, w_gate=None, b_gate=None):
    """One decode layer of the method: predict, list the neurons, compute them.

    [QB] "Общая архитектура PowerInfer": online, the predicted neurons are
    computed and the partial results merged into the layer output.
    """
    logits, mask = predict(x, p1, p2, c, tau)
    idx, count = compact(mask)
    y = sparse_ffn(x, idx, w_up, w_down_t, act, b_up, w_gate, b_gate)
    return {"logits": logits, "mask": mask, "idx": idx, "count": count, "y": y}
