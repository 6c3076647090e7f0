"""CPU checks of the C ABI: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments before it
launches anything.  No call here reaches a kernel launch.
"""

import ctypes
import os
import re

import pytest
import torch

from activation_sparse_rank_amd import _lib as L

# The fake addresses below are never dereferenced because every call fails
# validation first; still, run these only where no GPU is visible, so that a
# validation bug can never turn into a launch with bogus pointers.
pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="fake-pointer validation tests run only on hosts without a GPU")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pi.h")

FAKE = 0x10000          # a 16-byte aligned address; never dereferenced here
FAKE_ODD = 0x10004      # not 16-byte aligned


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pi_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_exports_match_header(lib):
    declared = _header_functions()
    assert declared == sorted(L.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(8):
        assert lib.pi_status_str(s)
    assert lib.pi_last_error() == b""


def _pred(d=8192, r=1024, f=32768, wtype=L.PI_F16, p1=FAKE, p2=FAKE, c=FAKE):
    return L.PiPredictor(d, r, f, wtype, p1, p2, c)


def _ffn(d=8192, f=32768, act=L.PI_RELU, wtype=L.PI_F16, up=FAKE, gate=None, dn=FAKE, bu=FAKE, bg=None):
    return L.PiFFN(d, f, act, wtype, up, gate, dn, bu, bg)


def test_workspace_sizes(lib):
    p, f = _pred(), _ffn()
    both = lib.pi_workspace_bytes(ctypes.byref(p), ctypes.byref(f), 1)
    only_p = lib.pi_workspace_bytes(ctypes.byref(p), None, 1)
    only_f = lib.pi_workspace_bytes(None, ctypes.byref(f), 1)
    assert both >= only_p + only_f > 0
    assert only_p >= 1024 * 4
    # mask + list + count sections
    assert both >= only_p + only_f + 32768 + 32768 * 4 + 4
    assert lib.pi_workspace_bytes(ctypes.byref(p), ctypes.byref(f), 8) > both
    assert lib.pi_workspace_bytes(None, None, 1) == 0
    assert lib.pi_workspace_bytes(ctypes.byref(p), ctypes.byref(f), 0) == 0
    bad = _pred(r=1004)
    assert lib.pi_workspace_bytes(ctypes.byref(bad), None, 1) == 0


def test_predict_rejects(lib):
    p = _pred()
    ws = 1 << 30

    def call(pred=p, x=FAKE, xtype=L.PI_F16, n=1, tau=0.5, mask=FAKE, logits=None, w=FAKE, wsb=ws):
        return lib.pi_predict(ctypes.byref(pred) if pred is not None else None, x, xtype, n, tau, mask, logits,
                              w, wsb, None)

    assert call(pred=None) == L.PI_E_NULL
    assert call(x=None) == L.PI_E_NULL
    assert call(mask=None) == L.PI_E_NULL
    assert call(n=0) == L.PI_E_SHAPE
    assert call(xtype=L.PI_F32) == L.PI_E_DTYPE
    assert call(x=FAKE_ODD) == L.PI_E_ALIGN
    assert call(logits=FAKE_ODD) == L.PI_E_ALIGN
    for tau in (0.0, 1.0, -0.5, 2.0, float("nan")):
        assert call(tau=tau) == L.PI_E_RANGE
    assert call(w=None) == L.PI_E_WORKSPACE
    assert call(wsb=100) == L.PI_E_WORKSPACE
    assert call(pred=_pred(r=12)) == L.PI_E_SHAPE
    assert call(pred=_pred(d=8190)) == L.PI_E_SHAPE
    assert call(pred=_pred(wtype=L.PI_Q4_0)) == L.PI_E_DTYPE
    assert call(pred=_pred(p2=None)) == L.PI_E_NULL
    assert call(pred=_pred(c=FAKE_ODD)) == L.PI_E_ALIGN


def test_compact_rejects(lib):
    assert lib.pi_compact(None, 1, 10, FAKE, FAKE, None) == L.PI_E_NULL
    assert lib.pi_compact(FAKE, 0, 10, FAKE, FAKE, None) == L.PI_E_SHAPE
    assert lib.pi_compact(FAKE, 1, 0, FAKE, FAKE, None) == L.PI_E_SHAPE
    assert lib.pi_compact(FAKE, 1, 10, FAKE_ODD, FAKE, None) == L.PI_E_ALIGN
    assert lib.pi_compact(FAKE, 1, 10, FAKE, FAKE + 2, None) == L.PI_E_ALIGN


def test_sparse_ffn_rejects(lib):
    f = _ffn()
    ws = 1 << 30

    def call(ffn=f, x=FAKE, xtype=L.PI_F16, n=1, idx=FAKE, cnt=FAKE, mc=32768, y=FAKE, yt=L.PI_F32, w=FAKE,
             wsb=ws):
        return lib.pi_sparse_ffn(ctypes.byref(ffn) if ffn is not None else None, x, xtype, n, idx, cnt, mc, y,
                                 yt, w, wsb, None)

    assert call(ffn=None) == L.PI_E_NULL
    assert call(idx=None) == L.PI_E_NULL
    assert call(cnt=None) == L.PI_E_NULL
    assert call(y=None) == L.PI_E_NULL
    assert call(n=0) == L.PI_E_SHAPE
    assert call(xtype=L.PI_F32) == L.PI_E_DTYPE
    assert call(yt=L.PI_Q4_0) == L.PI_E_DTYPE
    assert call(mc=-1) == L.PI_E_RANGE
    assert call(mc=32769) == L.PI_E_RANGE
    assert call(y=FAKE_ODD) == L.PI_E_ALIGN
    assert call(cnt=FAKE + 1) == L.PI_E_ALIGN
    assert call(wsb=10) == L.PI_E_WORKSPACE
    assert call(ffn=_ffn(act=L.PI_REGLU)) == L.PI_E_NULL              # ReGLU needs w_gate
    assert call(ffn=_ffn(act=7)) == L.PI_E_DTYPE
    assert call(ffn=_ffn(d=8196)) == L.PI_E_SHAPE
    assert call(ffn=_ffn(up=FAKE_ODD)) == L.PI_E_ALIGN
    assert call(ffn=_ffn(f=0)) == L.PI_E_SHAPE


def test_layer_rejects(lib):
    p, f = _pred(), _ffn()

    def call(pred=p, ffn=f, xtype=L.PI_F16, n=1, tau=0.5, yt=L.PI_F32, w=FAKE, wsb=1 << 30):
        return lib.pi_layer(ctypes.byref(pred), ctypes.byref(ffn), FAKE, xtype, n, tau, FAKE, yt, w, wsb, None)

    assert call(pred=_pred(f=1000)) == L.PI_E_SHAPE
    assert call(ffn=_ffn(d=4096)) == L.PI_E_SHAPE
    assert call(pred=_pred(wtype=L.PI_F32)) == L.PI_E_DTYPE
    assert call(tau=1.0) == L.PI_E_RANGE
    assert call(wsb=1000) == L.PI_E_WORKSPACE
    assert call(n=0) == L.PI_E_SHAPE


def test_repack_rejects(lib):
    assert lib.pi_q4_0_repack(None, 1, 32, FAKE, None) == L.PI_E_NULL
    assert lib.pi_q4_0_repack(FAKE, 1, 33, 0x20000, None) == L.PI_E_SHAPE
    assert lib.pi_q4_0_repack(FAKE, 0, 32, 0x20000, None) == L.PI_E_SHAPE
    assert lib.pi_q4_0_repack(FAKE, 4, 64, FAKE + 16, None) == L.PI_E_RANGE     # overlap
    assert lib.pi_q4_0_repack(FAKE, 1, 32, 0x20004, None) == L.PI_E_ALIGN


def test_placement_rejects(lib):
    assert lib.pi_count_active(None, 1, 8, FAKE, None) == L.PI_E_NULL
    assert lib.pi_count_active(FAKE, 0, 8, 0x20000, None) == L.PI_E_SHAPE
    assert lib.pi_count_active(FAKE, 1, 0, 0x20000, None) == L.PI_E_SHAPE
    assert lib.pi_hot_order(None, 8, None) == L.PI_E_NULL
    counts = (ctypes.c_uint32 * 4)()
    perm = (ctypes.c_int32 * 4)()
    assert lib.pi_hot_order(counts, 0, perm) == L.PI_E_SHAPE
    assert lib.pi_permute_rows(None, 4, 16, FAKE, 0x20000, None) == L.PI_E_NULL
    assert lib.pi_permute_rows(FAKE, 0, 16, 0x30000, 0x20000, None) == L.PI_E_SHAPE
    assert lib.pi_permute_rows(FAKE, 4, 6, 0x30000, 0x20000, None) == L.PI_E_SHAPE
    assert lib.pi_permute_rows(FAKE, 4, 0, 0x30000, 0x20000, None) == L.PI_E_SHAPE
    assert lib.pi_permute_rows(FAKE_ODD, 4, 16, 0x30000, 0x20000, None) == L.PI_E_ALIGN
    assert lib.pi_permute_rows(FAKE, 4, 16, 0x30000, FAKE + 32, None) == L.PI_E_RANGE  # overlap


def test_stream_read_rejects(lib):
    assert lib.pi_stream_read(None, 16, FAKE, None) == L.PI_E_NULL
    assert lib.pi_stream_read(FAKE, 0, 0x20000, None) == L.PI_E_SHAPE
    assert lib.pi_stream_read(FAKE, 24, 0x20000, None) == L.PI_E_SHAPE
    assert lib.pi_stream_read(FAKE_ODD, 32, 0x20000, None) == L.PI_E_ALIGN


def test_flag_calls_reject(lib):
    assert lib.pi_clear_flags(None, None) == L.PI_E_NULL
    assert lib.pi_clear_flags(FAKE_ODD, None) == L.PI_E_ALIGN
    out = ctypes.c_uint32(0)
    assert lib.pi_read_flags(None, ctypes.byref(out), None) == L.PI_E_NULL
    assert lib.pi_read_flags(FAKE, None, None) == L.PI_E_NULL
    assert lib.pi_read_flags(FAKE_ODD, ctypes.byref(out), None) == L.PI_E_ALIGN
    rows = ctypes.c_uint64(0)
    assert lib.pi_read_down_rows(None, ctypes.byref(rows), None) == L.PI_E_NULL
    assert lib.pi_read_down_rows(FAKE, None, None) == L.PI_E_NULL
    assert lib.pi_read_down_rows(FAKE_ODD, ctypes.byref(rows), None) == L.PI_E_ALIGN
    assert lib.pi_read_up_rows(None, ctypes.byref(rows), None) == L.PI_E_NULL
    assert lib.pi_read_up_rows(FAKE, None, None) == L.PI_E_NULL
    assert lib.pi_read_up_rows(FAKE_ODD, ctypes.byref(rows), None) == L.PI_E_ALIGN


def test_workspace_has_header(lib):
    # Every workspace starts with the PI_WS_HEADER_BYTES header: a predictor-only
    # workspace is the header plus the section of t (and nothing else at 1 token).
    p = _pred(d=1024, r=64, f=512)
    assert lib.pi_workspace_bytes(ctypes.byref(p), None, 1) == L.PI_WS_HEADER_BYTES + 256


def test_gather_read_rejects(lib):
    assert lib.pi_gather_read(None, 4, 16, FAKE, FAKE, 4, FAKE, None) == L.PI_E_NULL
    assert lib.pi_gather_read(FAKE, 0, 16, FAKE, FAKE, 4, FAKE, None) == L.PI_E_SHAPE
    assert lib.pi_gather_read(FAKE, 4, 24, FAKE, FAKE, 4, FAKE, None) == L.PI_E_SHAPE
    assert lib.pi_gather_read(FAKE, 4, 16, FAKE, FAKE, -1, FAKE, None) == L.PI_E_RANGE
    assert lib.pi_gather_read(FAKE_ODD, 4, 16, FAKE, FAKE, 4, FAKE, None) == L.PI_E_ALIGN
