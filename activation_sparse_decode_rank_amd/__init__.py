"""Activation-sparse FFN decode on MI355X (gfx950): a C-ABI HIP library
(include/sparse_ffn.h, built into libsparse_ffn.so) and a thin Python binding.

Importing the package loads the HIP library; if it is not built the import fails loudly.
"""
from . import _native  # noqa: F401  (raises ImportError when the library is missing)
from ._native import (  # noqa: F401
    EXPORTED, SFFN_ERR_HIP, SFFN_ERR_INVALID, SFFN_ERR_UNSUPPORTED, SFFN_F16, SFFN_F32,
    SFFN_MAX_BATCH, SFFN_OK, SffnDesc, SparseFFNError, sparse_ffn_compact, sparse_ffn_create,
    sparse_ffn_decode, sparse_ffn_decode_lookahead, sparse_ffn_decode_static, sparse_ffn_dense, sparse_ffn_destroy, sparse_ffn_forward,
    sparse_ffn_lookahead_begin, sparse_ffn_pack_rows,
    sparse_ffn_permutation, sparse_ffn_predict, sparse_ffn_profile_counts, sparse_ffn_read_probe,
    sparse_ffn_set_timing_events,
    sparse_ffn_status_string, sparse_ffn_workspace_bytes,
)
from .layer import (  # noqa: F401
    LookaheadBuffers, SparseFFN, decode_lookahead, decode_lookahead_fused, n_hot_for, pack_rows,
    permutation, profile_counts,
)
