"""torch-facing wrapper of the Token-Sparse prefill entry points (include/sparse_prefill.h).

Marshalling only: every step runs in the HIP library on the caller's current stream.
"""
from __future__ import annotations

import torch

from . import native as N


def make_prefill_tensors(Q, K, V, head_mode=None) -> N.sp_tensors:
    """sp_tensors from Q [B][Hq][L][d] and K, V [B][Hkv][L][d] (bf16, shared K / V strides), and an
    optional device int8 head_mode [Hq] (1 = full-attention head, 0 = sparse head)."""
    assert K.stride() == V.stride(), "K and V must share a layout"
    t = N.sp_tensors()
    t.q, t.q_sb, t.q_sh, t.q_st = Q.data_ptr(), Q.stride(0), Q.stride(1), Q.stride(2)
    t.k, t.v = K.data_ptr(), V.data_ptr()
    t.kv_sb, t.kv_sh, t.kv_st = K.stride(0), K.stride(1), K.stride(2)
    if head_mode is not None:
        assert head_mode.dtype == torch.int8 and head_mode.numel() == Q.shape[1] and head_mode.is_contiguous()
        t.head_mode = head_mode.data_ptr()
    return t


class SparsePrefill:
    """One prefill layer's configuration, its workspace, and the two calls."""

    def __init__(self, *, batch, n_q_heads, n_kv_heads, head_dim, seq_len, window, tau, softmax_scale,
                 device="cuda"):
        cfg = N.sp_config()
        cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim = batch, n_q_heads, n_kv_heads, head_dim
        cfg.seq_len, cfg.window, cfg.kv_dtype = seq_len, window, N.SD_BF16
        cfg.tau, cfg.softmax_scale = tau, softmax_scale
        self.cfg = cfg
        self.handle, self.ws_bytes = N.sparse_prefill_init(cfg)
        self.device = torch.device(device)
        self.ws = None

    def alloc_workspace(self):
        if self.ws is None:
            self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
            assert self.ws.data_ptr() % 256 == 0
        return self.ws

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            try:
                N.sparse_prefill_destroy(h)
            except Exception:  # interpreter shutdown: the library may already be gone
                pass
            self.handle = None

    @staticmethod
    def _stream():
        return torch.cuda.current_stream().cuda_stream

    def select(self, t: N.sp_tensors):
        N.sparse_prefill_select(self.handle, t, self.alloc_workspace().data_ptr(), self._stream())

    def attend(self, t: N.sp_tensors, out: torch.Tensor):
        assert out.dtype == torch.float32 and out.is_contiguous()
        N.sparse_prefill_attend(self.handle, t, self.alloc_workspace().data_ptr(), out.data_ptr(), self._stream())

    def step(self, t: N.sp_tensors, out: torch.Tensor):
        self.select(t)
        self.attend(t, out)

    def status(self) -> int:
        """The device status word after the enqueued work (synchronises the current stream): an
        internal-invariant flag, 0 on any input; nonzero means a library defect."""
        torch.cuda.current_stream().synchronize()
        return int(self.selection()["status"][0].item())

    def selection(self) -> dict:
        ws = self.alloc_workspace()
        v = N.sparse_prefill_view(self.handle, ws.data_ptr())
        base = ws.data_ptr()
        c = self.cfg
        B, Hq, L = c.batch, c.n_q_heads, c.seq_len

        def view(ptr, dtype, shape):
            n = 1
            for s in shape:
                n *= s
            es = torch.tensor([], dtype=dtype).element_size()
            return ws[ptr - base:ptr - base + n * es].view(dtype).view(*shape)

        return {"importance": view(v.importance, torch.float64, (B, Hq, L)),
                "budget": view(v.budget, torch.int32, (B,)),
                "head_bits": view(v.head_bits, torch.int32, (B, Hq, v.words)),
                "list": view(v.list, torch.int32, (B, Hq, L)),
                "status": view(v.status, torch.int32, (4,))}
