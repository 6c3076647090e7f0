"""Predictor-gated, neuron-aware sparse FFN for one AMD MI355X (gfx950).

The compute lives in libpi.so (HIP kernels behind the C ABI of include/pi.h);
this package is its thin torch binding.  Importing the package does not load
the library; the first call does, and fails loudly if it has not been built.
"""

from .api import (  # noqa: F401
    FFN,
    PiError,
    Predictor,
    alloc_workspace,
    clear_flags,
    compact,
    count_active,
    hot_order,
    rank_order,
    layer,
    layer_noalloc,
    permute_rows,
    place_layer,
    stream_read,
    gather_read,
    predict,
    q4_0_repack,
    read_down_rows,
    read_up_rows,
    read_flags,
    sparse_ffn,
    workspace_bytes,
)
from ._lib import load as load_library  # noqa: F401
