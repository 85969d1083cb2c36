"""Query-adaptive sparse decode attention for AMD MI355X (gfx950).

The compute path is the HIP library ``_lib/libsparse_decode.so`` (C ABI in
``include/sparse_decode.h``, ``include/sparse_prefill.h`` and
``include/sparse_gist_prefill.h``); ``native`` binds it with ctypes under the same
names, ``decoder.SparseDecoder`` marshals torch tensors into the decode step,
``prefill.SparsePrefill`` into the Token-Sparse prefill and
``gist_prefill.GistPrefill`` into the gist-masked (SSA) prefill.
"""
from . import native  # noqa: F401
from .decoder import SparseDecoder, make_config, make_tensors  # noqa: F401
from .prefill import SparsePrefill, make_prefill_tensors  # noqa: F401
from .gist_prefill import GistPrefill, make_gist_tensors  # noqa: F401
