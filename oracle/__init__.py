"""fp64 CPU oracle of query-adaptive sparse decode attention, of Token-Sparse prefill and of
gist-masked (SSA) prefill.

TEST INFRASTRUCTURE ONLY. Imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; the decode library and its binding never import,
call or link anything here.
"""
from . import sparse_decode_ref as ref  # noqa: F401
from . import sparse_prefill_ref as pref  # noqa: F401
from . import gist_prefill_ref as gref  # noqa: F401
from .source import GistPrefillSource, HostSource, PrefillSource  # noqa: F401
