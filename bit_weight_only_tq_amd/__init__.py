"""Weight-only quantized linear layers (ternary 2-bit and W4A16) for AMD MI355X.

The compute lives in libtq.so (hand-written HIP kernels for gfx950 behind a C
ABI, include/tq.h); this package is its Python binding plus the packed
layout descriptions.  Build the library with
``python -m bit_weight_only_tq_amd.build``.
"""

from ._lib import (TQ_WORKSPACE_FLAG_BYTES, TQError, load, new_workspace, tq_abi_version,  # noqa: F401
                   tq_diag_gemv, tq_diag_stream_read, tq_gemm, tq_gemm_noalloc, tq_gemm_workspace_bytes, tq_pack,
                   tq_select_path, tq_unpack, w4a16_gemm, w4a16_gemm_asym_workspace_bytes,
                   w4a16_gemm_workspace_bytes, w4a16_pack, w4a16_pack_asym, w4a16_unpack, w4a16_unpack_asym)
from .layout import TernaryLayout, W4Layout  # noqa: F401

__all__ = [
    "TQ_WORKSPACE_FLAG_BYTES", "TQError", "load", "new_workspace", "tq_abi_version", "tq_diag_gemv", "tq_diag_stream_read", "tq_gemm", "tq_gemm_noalloc",
    "tq_gemm_workspace_bytes", "tq_pack",
    "tq_select_path",
    "tq_unpack",
    "w4a16_gemm", "w4a16_gemm_asym_workspace_bytes", "w4a16_gemm_workspace_bytes", "w4a16_pack",
    "w4a16_pack_asym", "w4a16_unpack", "w4a16_unpack_asym", "TernaryLayout", "W4Layout",
]
