"""ctypes view of libpi.so (the C ABI declared in include/pi.h).

Loading fails loudly: there is no CPU fallback anywhere in this package.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpi.so")

PI_OK, PI_E_NULL, PI_E_SHAPE, PI_E_DTYPE, PI_E_ALIGN, PI_E_RANGE, PI_E_WORKSPACE, PI_E_HIP = range(8)
PI_F32, PI_F16, PI_Q4_0 = 0, 1, 2
PI_RELU, PI_REGLU, PI_RELU2 = 0, 1, 2

STATUS_NAMES = {
    PI_OK: "PI_OK", PI_E_NULL: "PI_E_NULL", PI_E_SHAPE: "PI_E_SHAPE", PI_E_DTYPE: "PI_E_DTYPE",
    PI_E_ALIGN: "PI_E_ALIGN", PI_E_RANGE: "PI_E_RANGE", PI_E_WORKSPACE: "PI_E_WORKSPACE", PI_E_HIP: "PI_E_HIP",
}

# Every symbol include/pi.h declares.
EXPORTS = ("pi_workspace_bytes", "pi_clear_flags", "pi_read_flags", "pi_read_down_rows", "pi_read_up_rows", "pi_predict", "pi_compact",
           "pi_sparse_ffn", "pi_layer", "pi_layer_noalloc", "pi_q4_0_repack", "pi_count_active", "pi_hot_order",
           "pi_rank_order", "pi_permute_rows", "pi_stream_read", "pi_gather_read", "pi_status_str", "pi_last_error")

PI_SEGMENT_ROWS = 32   # neurons per segment of pi_layer's fused kernel (pi.h)
PI_STREAM_BLOCKS = 2048  # entries of pi_stream_read's output (pi.h)

# Workspace header (pi.h): word indices and flag bits.
PI_WS_HEADER_BYTES = 256
PI_WS_FLAGS, PI_WS_WAIT_POLLS, PI_WS_SKIP_PUBLISH = 0, 1, 2
PI_WS_DOWN_ROWS = 4   # 64-bit count of down-projection rows read, words 4 and 5
PI_WS_UP_ROWS = 6     # 64-bit count of w_up rows read, words 6 and 7
PI_FLAG_WAIT_EXPIRED, PI_FLAG_FP16_RANGE = 1, 2
PI_NOALLOC_SCRATCH_BYTES = 32 << 20   # static scratch of pi_layer_noalloc (pi.h)


class PiPredictor(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("rank", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("wtype", ctypes.c_int32), ("p1", ctypes.c_void_p), ("p2", ctypes.c_void_p),
                ("c", ctypes.c_void_p)]


class PiFFN(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("act", ctypes.c_int32),
                ("wtype", ctypes.c_int32), ("w_up", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
                ("w_down_t", ctypes.c_void_p), ("b_up", ctypes.c_void_p), ("b_gate", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpi.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"libpi.so not found at {path}; build it with `python -m activation_sparse_rank_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P, PP = ctypes.c_void_p, ctypes.POINTER
    i32, f32, sz = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.pi_workspace_bytes.argtypes = [PP(PiPredictor), PP(PiFFN), i32]
    lib.pi_workspace_bytes.restype = sz
    lib.pi_clear_flags.argtypes = [P, P]
    lib.pi_clear_flags.restype = ctypes.c_int
    lib.pi_read_flags.argtypes = [P, PP(ctypes.c_uint32), P]
    lib.pi_read_flags.restype = ctypes.c_int
    lib.pi_read_down_rows.argtypes = [P, PP(ctypes.c_uint64), P]
    lib.pi_read_down_rows.restype = ctypes.c_int
    lib.pi_read_up_rows.argtypes = [P, PP(ctypes.c_uint64), P]
    lib.pi_read_up_rows.restype = ctypes.c_int
    lib.pi_predict.argtypes = [PP(PiPredictor), P, i32, i32, f32, P, P, P, sz, P]
    lib.pi_predict.restype = ctypes.c_int
    lib.pi_compact.argtypes = [P, i32, i32, P, P, P]
    lib.pi_compact.restype = ctypes.c_int
    lib.pi_sparse_ffn.argtypes = [PP(PiFFN), P, i32, i32, P, P, i32, P, i32, P, sz, P]
    lib.pi_sparse_ffn.restype = ctypes.c_int
    lib.pi_layer.argtypes = [PP(PiPredictor), PP(PiFFN), P, i32, i32, f32, P, i32, P, sz, P]
    lib.pi_layer.restype = ctypes.c_int
    lib.pi_layer_noalloc.argtypes = [PP(PiPredictor), PP(PiFFN), P, i32, i32, f32, P, i32, P]
    lib.pi_layer_noalloc.restype = ctypes.c_int
    lib.pi_q4_0_repack.argtypes = [P, i32, i32, P, P]
    lib.pi_q4_0_repack.restype = ctypes.c_int
    lib.pi_count_active.argtypes = [P, i32, i32, P, P]
    lib.pi_count_active.restype = ctypes.c_int
    lib.pi_hot_order.argtypes = [P, i32, P]
    lib.pi_hot_order.restype = ctypes.c_int
    lib.pi_rank_order.argtypes = [P, i32, P]
    lib.pi_rank_order.restype = ctypes.c_int
    lib.pi_permute_rows.argtypes = [P, i32, i32, P, P, P]
    lib.pi_permute_rows.restype = ctypes.c_int
    lib.pi_stream_read.argtypes = [P, sz, P, P]
    lib.pi_stream_read.restype = ctypes.c_int
    lib.pi_gather_read.argtypes = [P, i32, i32, P, P, i32, P, P]
    lib.pi_gather_read.restype = ctypes.c_int
    lib.pi_status_str.argtypes = [ctypes.c_int]
    lib.pi_status_str.restype = ctypes.c_char_p
    lib.pi_last_error.argtypes = []
    lib.pi_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib
