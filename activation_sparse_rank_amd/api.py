"""Thin torch-facing binding of libpi: argument marshalling only.

Each function takes device tensors, checks that their shapes, dtypes and
layouts match what the C ABI will read (the C side cannot see tensor
shapes), and forwards raw pointers plus the current HIP stream.  All
computation happens in the library's HIP kernels; a non-OK status raises
``PiError``.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib as L


class PiError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = L.load()
        msg = lib.pi_status_str(status).decode()
        detailed = status == L.PI_E_HIP or (status == L.PI_E_WORKSPACE and where == "pi_layer_noalloc")
        extra = lib.pi_last_error().decode() if detailed else ""
        super().__init__(f"{where}: {L.STATUS_NAMES.get(status, status)} ({msg}){' ' + extra if extra else ''}")
        self.status = status


_DTYPES = {torch.float32: L.PI_F32, torch.float16: L.PI_F16}
_ACTS = {"relu": L.PI_RELU, "reglu": L.PI_REGLU, "relu2": L.PI_RELU2}


def _check(status: int, where: str):
    if status != L.PI_OK:
        raise PiError(status, where)


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Predictor:
    """Predictor weights of one layer (p1 [r, d], p2 [d_ff, r], c [d_ff] fp32)."""

    def __init__(self, p1: torch.Tensor, p2: torch.Tensor, c: torch.Tensor):
        for t, n in ((p1, "p1"), (p2, "p2"), (c, "c")):
            _dev(t, n)
        if p1.dtype not in _DTYPES or p2.dtype != p1.dtype:
            raise TypeError("p1 and p2 must both be float16 or both float32")
        if c.dtype != torch.float32:
            raise TypeError("c must be float32")
        r, d = p1.shape
        f, r2 = p2.shape
        if r2 != r or c.shape != (f,):
            raise ValueError("predictor shapes disagree")
        self.p1, self.p2, self.c = p1, p2, c
        self.d_model, self.rank, self.d_ff = d, r, f
        self.wtype = _DTYPES[p1.dtype]
        self.desc = L.PiPredictor(d, r, f, self.wtype, p1.data_ptr(), p2.data_ptr(), c.data_ptr())


class FFN:
    """FFN weights of one layer.

    fp16/fp32: ``w_up``, ``w_down_t`` (and ``w_gate``) are [d_ff, d_model].
    Q4_0: they are uint8 tensors in the repacked layout (see ``q4_0_repack``)
    and ``d_model`` must be given.
    """

    def __init__(self, w_up, w_down_t, act="relu", b_up=None, w_gate=None, b_gate=None, d_model=None):
        if act not in _ACTS:
            raise ValueError(f"unknown activation {act!r}")
        if act == "reglu" and w_gate is None:
            raise ValueError("ReGLU needs w_gate")
        for t, n in ((w_up, "w_up"), (w_down_t, "w_down_t"), (w_gate, "w_gate"), (b_up, "b_up"),
                     (b_gate, "b_gate")):
            if t is not None:
                _dev(t, n)
        for b, n in ((b_up, "b_up"), (b_gate, "b_gate")):
            if b is not None and b.dtype != torch.float32:
                raise TypeError(f"{n} must be float32")
        if w_up.dtype == torch.uint8:
            if d_model is None:
                raise ValueError("Q4_0 weights need d_model")
            self.wtype = L.PI_Q4_0
            f = w_up.shape[0]
            if w_up.numel() != f * (d_model // 32) * 18:
                raise ValueError("Q4_0 buffer size does not match d_ff x d_model")
        else:
            if w_up.dtype not in _DTYPES:
                raise TypeError("weights must be float16, float32 or uint8 (Q4_0)")
            self.wtype = _DTYPES[w_up.dtype]
            f, d_model = w_up.shape
        for t, n in ((w_down_t, "w_down_t"), (w_gate, "w_gate")):
            if t is not None and (t.dtype != w_up.dtype or t.shape != w_up.shape):
                raise ValueError(f"{n} must match w_up in dtype and shape")
        for b, n in ((b_up, "b_up"), (b_gate, "b_gate")):
            if b is not None and b.shape != (f,):
                raise ValueError(f"{n} must have shape [d_ff]")
        self.w_up, self.w_down_t, self.w_gate, self.b_up, self.b_gate = w_up, w_down_t, w_gate, b_up, b_gate
        self.act = act
        self.d_model, self.d_ff = int(d_model), int(f)
        self.x_dtype = torch.float16 if self.wtype == L.PI_Q4_0 else w_up.dtype
        self.desc = L.PiFFN(self.d_model, self.d_ff, _ACTS[act], self.wtype, w_up.data_ptr(), _ptr(w_gate),
                            w_down_t.data_ptr(), _ptr(b_up), _ptr(b_gate))


def _pp(pred):
    return None if pred is None else ctypes.byref(pred.desc)


def workspace_bytes(pred: Predictor | None, ffn: FFN | None, n_tok: int) -> int:
    n = L.load().pi_workspace_bytes(_pp(pred), _pp(ffn), int(n_tok))
    if n == 0:
        raise PiError(L.PI_E_SHAPE, "pi_workspace_bytes")
    return int(n)


def alloc_workspace(pred, ffn, n_tok, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (so its fault flags start clear)."""
    return torch.zeros(workspace_bytes(pred, ffn, n_tok), dtype=torch.uint8, device=device)


def _temp_workspace(pred, ffn, n_tok, device, stream):
    """Workspace for one call that was given none.  It is allocated on the
    call's stream, so that when the tensor is freed right after the call the
    caching allocator hands its memory out again only in that stream's
    order, after the call's kernels."""
    if stream is None:
        return alloc_workspace(pred, ffn, n_tok, device)
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream), device=device)
    with torch.cuda.stream(s):
        return alloc_workspace(pred, ffn, n_tok, device)


def clear_flags(ws, stream=None):
    """Zero the workspace header: fault flags, test hooks and the count of
    down-projection rows read (pi_clear_flags)."""
    _dev(ws, "ws")
    _check(L.load().pi_clear_flags(ws.data_ptr(), _stream(stream)), "pi_clear_flags")


def read_flags(ws, stream=None) -> int:
    """The workspace's sticky fault flags (PI_FLAG_* bits) after the work
    queued on stream (pi_read_flags; synchronises that stream)."""
    _dev(ws, "ws")
    out = ctypes.c_uint32(0)
    _check(L.load().pi_read_flags(ws.data_ptr(), ctypes.byref(out), _stream(stream)), "pi_read_flags")
    return int(out.value)


def read_down_rows(ws, stream=None) -> int:
    """How many w_down_t rows the down projections of the calls on ws have
    read, summed over calls, after the work queued on stream
    (pi_read_down_rows; synchronises that stream)."""
    _dev(ws, "ws")
    out = ctypes.c_uint64(0)
    _check(L.load().pi_read_down_rows(ws.data_ptr(), ctypes.byref(out), _stream(stream)), "pi_read_down_rows")
    return int(out.value)


def read_up_rows(ws, stream=None) -> int:
    """How many w_up rows the up projections of the calls on ws have read,
    summed over calls (pi_read_up_rows; synchronises that stream)."""
    _dev(ws, "ws")
    out = ctypes.c_uint64(0)
    _check(L.load().pi_read_up_rows(ws.data_ptr(), ctypes.byref(out), _stream(stream)), "pi_read_up_rows")
    return int(out.value)


def _x(x, d, dtype, name="x"):
    _dev(x, name)
    if x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    if x.dim() != 2 or x.shape[1] != d:
        raise ValueError(f"{name} must be [n_tok, {d}]")
    return x.shape[0]


def predict(pred: Predictor, x, tau: float, mask, logits=None, ws=None, stream=None):
    n = _x(x, pred.d_model, pred.p1.dtype)
    _dev(mask, "mask")
    if mask.dtype != torch.uint8 or mask.shape != (n, pred.d_ff):
        raise ValueError("mask must be uint8 [n_tok, d_ff]")
    if logits is not None:
        _dev(logits, "logits")
        if logits.dtype != torch.float32 or logits.shape != (n, pred.d_ff):
            raise ValueError("logits must be float32 [n_tok, d_ff]")
    if ws is None:
        ws = _temp_workspace(pred, None, n, x.device, stream)
    _dev(ws, "ws")
    st = L.load().pi_predict(ctypes.byref(pred.desc), x.data_ptr(), _DTYPES[x.dtype], n, float(tau),
                             mask.data_ptr(), _ptr(logits), ws.data_ptr(), ws.numel(), _stream(stream))
    _check(st, "pi_predict")


def compact(mask, idx, count, stream=None):
    _dev(mask, "mask"), _dev(idx, "idx"), _dev(count, "count")
    if mask.dtype != torch.uint8 or mask.dim() != 2:
        raise ValueError("mask must be uint8 [n_tok, d_ff]")
    n, f = mask.shape
    if idx.dtype != torch.int32 or idx.numel() < f:
        raise ValueError("idx must be int32 with at least d_ff entries")
    if count.dtype != torch.int32 or count.numel() < 1:
        raise ValueError("count must be an int32 device scalar")
    st = L.load().pi_compact(mask.data_ptr(), n, f, idx.data_ptr(), count.data_ptr(), _stream(stream))
    _check(st, "pi_compact")


def sparse_ffn(ffn: FFN, x, idx, count, y, ws=None, max_count=None, stream=None):
    n = _x(x, ffn.d_model, ffn.x_dtype)
    _dev(idx, "idx"), _dev(count, "count"), _dev(y, "y")
    if idx.dtype != torch.int32 or count.dtype != torch.int32:
        raise TypeError("idx and count must be int32")
    if y.dtype not in _DTYPES or y.shape != (n, ffn.d_model):
        raise ValueError("y must be float32 or float16 [n_tok, d_model]")
    mc = ffn.d_ff if max_count is None else int(max_count)
    if idx.numel() < min(mc, ffn.d_ff):
        raise ValueError("idx is shorter than max_count")
    if ws is None:
        ws = _temp_workspace(None, ffn, n, x.device, stream)
    _dev(ws, "ws")
    st = L.load().pi_sparse_ffn(ctypes.byref(ffn.desc), x.data_ptr(), _DTYPES[x.dtype], n, idx.data_ptr(),
                                count.data_ptr(), mc, y.data_ptr(), _DTYPES[y.dtype], ws.data_ptr(),
                                ws.numel(), _stream(stream))
    _check(st, "pi_sparse_ffn")


def layer(pred: Predictor, ffn: FFN, x, tau: float, y, ws=None, stream=None):
    n = _x(x, ffn.d_model, ffn.x_dtype)
    _dev(y, "y")
    if y.dtype not in _DTYPES or y.shape != (n, ffn.d_model):
        raise ValueError("y must be float32 or float16 [n_tok, d_model]")
    if ws is None:
        ws = _temp_workspace(pred, ffn, n, x.device, stream)
    _dev(ws, "ws")
    st = L.load().pi_layer(ctypes.byref(pred.desc), ctypes.byref(ffn.desc), x.data_ptr(), _DTYPES[x.dtype], n,
                           float(tau), y.data_ptr(), _DTYPES[y.dtype], ws.data_ptr(), ws.numel(),
                           _stream(stream))
    _check(st, "pi_layer")


def layer_noalloc(pred: Predictor, ffn: FFN, x, tau: float, y, stream=None):
    """pi_layer with the library's static scratch (pi_layer_noalloc): the
    same result as layer(), no workspace, and nothing allocated here either.
    Calls that overlap on one GPU race on the shared scratch."""
    n = _x(x, ffn.d_model, ffn.x_dtype)
    _dev(y, "y")
    if y.dtype not in _DTYPES or y.shape != (n, ffn.d_model):
        raise ValueError("y must be float32 or float16 [n_tok, d_model]")
    st = L.load().pi_layer_noalloc(ctypes.byref(pred.desc), ctypes.byref(ffn.desc), x.data_ptr(), _DTYPES[x.dtype],
                                   n, float(tau), y.data_ptr(), _DTYPES[y.dtype], _stream(stream))
    _check(st, "pi_layer_noalloc")


def q4_0_repack(src, rows: int, cols: int, dst=None, stream=None):
    _dev(src, "src")
    if src.dtype != torch.uint8 or src.numel() != rows * (cols // 32) * 18:
        raise ValueError("src must be uint8 canonical Q4_0 blocks of rows x cols")
    if dst is None:
        dst = torch.empty_like(src)
    _dev(dst, "dst")
    if dst.dtype != torch.uint8 or dst.numel() != src.numel():
        raise ValueError("dst must be uint8 with as many bytes as src")
    st = L.load().pi_q4_0_repack(src.data_ptr(), int(rows), int(cols), dst.data_ptr(), _stream(stream))
    _check(st, "pi_q4_0_repack")
    return dst


# ---------------------------------------------------------------------------
# Neuron placement by hotness (offline, at load time)
# ---------------------------------------------------------------------------

def count_active(mask, counts, stream=None):
    """counts[i] += number of tokens whose mask row marks neuron i (pi_count_active)."""
    _dev(mask, "mask"), _dev(counts, "counts")
    if mask.dtype != torch.uint8 or mask.dim() != 2:
        raise ValueError("mask must be uint8 [n_tok, d_ff]")
    n, f = mask.shape
    if counts.dtype != torch.int32 or counts.numel() != f:
        raise ValueError("counts must be int32 [d_ff] (read as uint32)")
    st = L.load().pi_count_active(mask.data_ptr(), n, f, counts.data_ptr(), _stream(stream))
    _check(st, "pi_count_active")


def hot_order(counts) -> torch.Tensor:
    """Placement order from firing counts (pi_hot_order, host memory): perm[k]
    is the neuron placed at row k."""
    c = counts.detach().to("cpu").contiguous()
    if c.dtype != torch.int32 or c.dim() != 1:
        raise ValueError("counts must be int32 [d_ff]")
    perm = torch.empty(c.numel(), dtype=torch.int32)
    st = L.load().pi_hot_order(c.data_ptr(), c.numel(), perm.data_ptr())
    _check(st, "pi_hot_order")
    return perm


def rank_order(counts) -> torch.Tensor:
    """Placement order by rank (pi_rank_order, host memory): perm[k] is the
    neuron with the k-th highest count, ties by lower number."""
    c = counts.detach().to("cpu").contiguous()
    if c.dtype != torch.int32 or c.dim() != 1:
        raise ValueError("counts must be int32 [d_ff]")
    perm = torch.empty(c.numel(), dtype=torch.int32)
    st = L.load().pi_rank_order(c.data_ptr(), c.numel(), perm.data_ptr())
    _check(st, "pi_rank_order")
    return perm


def permute_rows(src, perm, dst=None, stream=None):
    """dst row k = src row perm[k] over the first dimension (pi_permute_rows)."""
    _dev(src, "src"), _dev(perm, "perm")
    rows = src.shape[0]
    if perm.dtype != torch.int32 or perm.numel() != rows:
        raise ValueError("perm must be int32 with one entry per row of src")
    row_bytes = src.numel() * src.element_size() // rows
    if dst is None:
        dst = torch.empty_like(src)
    _dev(dst, "dst")
    if dst.shape != src.shape or dst.dtype != src.dtype:
        raise ValueError("dst must match src in shape and dtype")
    st = L.load().pi_permute_rows(src.data_ptr(), rows, row_bytes, perm.data_ptr(), dst.data_ptr(),
                                  _stream(stream))
    _check(st, "pi_permute_rows")
    return dst


# Per-neuron arrays of a layer, by the names Predictor / FFN take.
NEURON_ARRAYS = ("p2", "c", "w_up", "w_gate", "w_down_t", "b_up", "b_gate")


def place_layer(tensors: dict, perm) -> dict:
    """Apply one neuron permutation to every per-neuron array present in
    tensors (rows of p2, w_up, w_gate, w_down_t -- canonical Q4_0 blocks for
    Q4_0 weights, before q4_0_repack -- and entries of c, b_up, b_gate);
    other entries are passed through.  Returns a new dict."""
    out = dict(tensors)
    pd = None
    for k in NEURON_ARRAYS:
        t = tensors.get(k)
        if t is None:
            continue
        if pd is None or pd.device != t.device:
            pd = perm.to(device=t.device, dtype=torch.int32).contiguous()
        out[k] = permute_rows(t, pd)
    return out


def stream_read(src, out=None, stream=None):
    """Read every byte of src once (pi_stream_read); returns out, whose XOR
    over its PI_STREAM_BLOCKS int32 entries is the XOR of src's 32-bit words."""
    _dev(src, "src")
    nbytes = src.numel() * src.element_size()
    if out is None:
        out = torch.empty(L.PI_STREAM_BLOCKS, dtype=torch.int32, device=src.device)
    _dev(out, "out")
    if out.dtype != torch.int32 or out.numel() != L.PI_STREAM_BLOCKS:
        raise ValueError("out must be int32 [PI_STREAM_BLOCKS]")
    st = L.load().pi_stream_read(src.data_ptr(), nbytes, out.data_ptr(), _stream(stream))
    _check(st, "pi_stream_read")
    return out


def gather_read(src, rows, count, row_bytes=None, max_count=None, out=None, stream=None):
    """Read the listed rows of src once (pi_gather_read): rows[0 .. count) of
    the [src.shape[0], row_bytes] matrix; returns out, whose XOR over its
    PI_STREAM_BLOCKS int32 entries is the XOR of those rows' 32-bit words."""
    _dev(src, "src"), _dev(rows, "rows"), _dev(count, "count")
    n_rows = src.shape[0]
    rb = src.numel() * src.element_size() // n_rows if row_bytes is None else int(row_bytes)
    if rows.dtype != torch.int32 or count.dtype != torch.int32:
        raise TypeError("rows and count must be int32")
    mc = rows.numel() if max_count is None else int(max_count)
    if rows.numel() < mc:
        raise ValueError("rows is shorter than max_count")
    if out is None:
        out = torch.empty(L.PI_STREAM_BLOCKS, dtype=torch.int32, device=src.device)
    _dev(out, "out")
    if out.dtype != torch.int32 or out.numel() != L.PI_STREAM_BLOCKS:
        raise ValueError("out must be int32 [PI_STREAM_BLOCKS]")
    st = L.load().pi_gather_read(src.data_ptr(), n_rows, rb, rows.data_ptr(), count.data_ptr(), mc, out.data_ptr(),
                                 _stream(stream))
    _check(st, "pi_gather_read")
    return out
