"""Query-adaptive sparse decode attention for AMD MI355X (gfx950).

The compute path is the HIP library ``_lib/libsparse_decode.so`` (C ABI in
``include/sparse_decode.h`` and ``include/sparse_prefill.h``); ``native`` binds it
with ctypes under the same names, ``decoder.SparseDecoder`` marshals torch tensors
into the decode step and ``prefill.SparsePrefill`` into the Token-Sparse prefill.
"""
from . import native  # noqa: F401
from .decoder import SparseDecoder, make_config, make_tensors  # noqa: F401
from .prefill import SparsePrefill, make_prefill_tensors  # noqa: F401
