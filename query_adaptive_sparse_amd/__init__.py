"""Query-adaptive sparse decode attention for AMD MI355X (gfx950).

The compute path is the HIP library ``_lib/libsparse_decode.so`` (C ABI in
``include/sparse_decode.h``); ``native`` binds it with ctypes under the same
names and ``decoder.SparseDecoder`` marshals torch tensors into it.
"""
from . import native  # noqa: F401
from .decoder import SparseDecoder, make_config, make_tensors  # noqa: F401
