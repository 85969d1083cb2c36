"""torch-facing wrapper of the gist-masked (SSA) prefill entry points (include/sparse_gist_prefill.h).

Marshalling only: the attention runs in the HIP library on the caller's current stream.
"""
from __future__ import annotations

import torch

from . import native as N


def make_gist_tensors(Q, K, V, Qg, Kg, Vg) -> N.gp_tensors:
    """gp_tensors from raw Q [B][Hq][N][d], K, V [B][Hkv][N][d] and gist Qg [B][Hq][M][d],
    Kg, Vg [B][Hkv][M][d] (bf16; K / V and Kg / Vg share their strides)."""
    assert K.stride() == V.stride() and Kg.stride() == Vg.stride(), "keys and values must share a layout"
    t = N.gp_tensors()
    t.q, t.q_sb, t.q_sh, t.q_st = Q.data_ptr(), Q.stride(0), Q.stride(1), Q.stride(2)
    t.k, t.v = K.data_ptr(), V.data_ptr()
    t.kv_sb, t.kv_sh, t.kv_st = K.stride(0), K.stride(1), K.stride(2)
    t.qg, t.qg_sb, t.qg_sh, t.qg_st = Qg.data_ptr(), Qg.stride(0), Qg.stride(1), Qg.stride(2)
    t.kg, t.vg = Kg.data_ptr(), Vg.data_ptr()
    t.kvg_sb, t.kvg_sh, t.kvg_st = Kg.stride(0), Kg.stride(1), Kg.stride(2)
    return t


class GistPrefill:
    """One gist-masked prefill layer's configuration and its call."""

    def __init__(self, *, batch, n_q_heads, n_kv_heads, head_dim, n_tokens, chunk_size, softmax_scale):
        cfg = N.gp_config()
        cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim = batch, n_q_heads, n_kv_heads, head_dim
        cfg.n_tokens, cfg.chunk_size, cfg.kv_dtype = n_tokens, chunk_size, N.SD_BF16
        cfg.softmax_scale = softmax_scale
        self.cfg = cfg
        self.handle, self.ws_bytes = N.sparse_gist_prefill_init(cfg)
        self._ws = None

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            try:
                N.sparse_gist_prefill_destroy(h)
            except Exception:  # interpreter shutdown: the library may already be gone
                pass
            self.handle = None

    def workspace(self, device=None) -> torch.Tensor:
        """The device workspace (allocated once, 256-byte aligned by the caching allocator)."""
        if self._ws is None:
            self._ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device or "cuda")
            assert self._ws.data_ptr() % 256 == 0
        return self._ws

    def attend(self, t: N.gp_tensors, out: torch.Tensor, out_gist: torch.Tensor):
        """out fp32 [B][Hq][N][d], out_gist fp32 [B][Hq][M][d], both contiguous."""
        for o in (out, out_gist):
            assert o.dtype == torch.float32 and o.is_contiguous()
        N.sparse_gist_prefill_attend(self.handle, t, self.workspace(out.device).data_ptr(), out.data_ptr(),
                                     out_gist.data_ptr(), torch.cuda.current_stream().cuda_stream)
