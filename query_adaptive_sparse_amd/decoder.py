"""torch-facing wrapper over the C ABI: tensors in, device pointers and strides out.

Marshalling only. Every step runs in the HIP library on the caller's current
stream; nothing here computes any part of the decode step.
"""
from __future__ import annotations

import ctypes

import torch

from . import native as N

_DTYPES = {torch.float32: N.SD_F32, torch.bfloat16: N.SD_BF16}
_MODES = {"topk": N.SD_TOPK, "topp": N.SD_TOPP, "hier": N.SD_HIER_TOPK, "coverage": N.SD_COVERAGE}


def make_config(*, batch, kv_batch, n_q_heads, n_kv_heads, head_dim, n_ctx, chunk_size, dtype, mode, n_queries=1,
                route="summary", route_dim=0, top_k=0, top_k_seg=0, seg_size=0, top_p=1.0, select_scale=1.0, tau=0.0,
                softmax_scale=1.0, keep_first=0, keep_last=0, sink=0, window=0, attend_summary=1,
                attend_blocks=0, head_masks=False, head_mode=None):
    """An sd_config plus the host array it points to (keep both alive)."""
    cfg = N.sd_config()
    cfg.batch, cfg.n_queries, cfg.kv_batch = batch, n_queries, kv_batch
    cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim = n_q_heads, n_kv_heads, head_dim
    cfg.n_ctx, cfg.chunk_size, cfg.seg_size = n_ctx, chunk_size, seg_size
    cfg.route = N.SD_ROUTE_PROXY if route == "proxy" else N.SD_ROUTE_SUMMARY
    cfg.route_dim = route_dim
    cfg.kv_dtype = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else {"f32": N.SD_F32, "bf16": N.SD_BF16}[dtype]
    cfg.mode = _MODES[mode]
    cfg.top_k, cfg.top_k_seg = top_k, top_k_seg
    cfg.top_p, cfg.select_scale, cfg.tau, cfg.softmax_scale = top_p, select_scale, tau, softmax_scale
    cfg.keep_first, cfg.keep_last, cfg.sink, cfg.window = keep_first, keep_last, sink, window
    cfg.attend_summary = int(attend_summary)  # 0 none, 1 selected chunks', 2 every chunk's
    cfg.attend_blocks = attend_blocks
    cfg.head_masks = int(bool(head_masks))
    hm = None
    if head_mode is not None:
        hm = (ctypes.c_int8 * len(head_mode))(*[int(x) for x in head_mode])
        cfg.head_mode = ctypes.cast(hm, ctypes.POINTER(ctypes.c_int8))
    return cfg, hm


def _ptr(t):
    return None if t is None else t.data_ptr()


def make_tensors(q, K, V, Kg=None, Vg=None, Kmg=None, Kp=None, P=None, ctx_len=None) -> N.sd_tensors:
    """sd_tensors from torch tensors (q [B][Hq][d] or [B][T][Hq][d]; K, V [Bkv][Hkv][N][d]; ...);
    ``ctx_len``: an optional device int32 [B] of the tokens each sequence's cache holds this step."""
    t = N.sd_tensors()
    if ctx_len is not None:
        assert ctx_len.dtype == torch.int32 and ctx_len.is_contiguous() and ctx_len.numel() == q.shape[0]
        t.ctx_len = ctx_len.data_ptr()
    t.q = _ptr(q)
    if q.dim() == 4:
        t.q_sb, t.q_st, t.q_sh = q.stride(0), q.stride(1), q.stride(2)
    else:
        t.q_sb, t.q_st, t.q_sh = q.stride(0), 0, q.stride(1)

    def sb(x):
        return 0 if x.shape[0] == 1 else x.stride(0)

    t.k, t.v = _ptr(K), _ptr(V)
    assert K.stride() == V.stride(), "K and V must share a layout"
    t.kv_sb, t.kv_sh, t.kv_st = sb(K), K.stride(1), K.stride(2)
    if Kg is not None:
        t.kg, t.vg = _ptr(Kg), _ptr(Vg)
        t.g_sb, t.g_sh, t.g_st = sb(Kg), Kg.stride(1), Kg.stride(2)
    if Kmg is not None:
        t.kmg = _ptr(Kmg)
        t.mg_sb, t.mg_sh, t.mg_st = sb(Kmg), Kmg.stride(1), Kmg.stride(2)
    if Kp is not None:
        t.kp = _ptr(Kp)
        t.kp_sb, t.kp_sh, t.kp_st = sb(Kp), Kp.stride(1), Kp.stride(2)
    if P is not None:
        assert P.is_contiguous()
        t.proj = _ptr(P)
    return t


class SparseDecoder:
    """One decode layer's configuration, its workspace, and the four calls."""

    def __init__(self, device="cuda", **params):
        self.params = params
        self.cfg, self._hm = make_config(**params)
        self.handle, self.ws_bytes = N.sparse_decode_init(self.cfg)
        self.levels = N.sparse_decode_num_levels(self.handle)
        self.attend_blocks = N.sparse_decode_attend_blocks(self.handle)
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
                N.sparse_decode_destroy(h)
            except Exception:  # interpreter shutdown: the library may already be gone
                pass
            self.handle = None

    @staticmethod
    def _stream():
        return torch.cuda.current_stream().cuda_stream

    def score_chunks(self, t: N.sd_tensors, level: int):
        N.sparse_decode_score_chunks(self.handle, t, level, self.alloc_workspace().data_ptr(), self._stream())

    def select(self, level: int):
        N.sparse_decode_select(self.handle, level, self.alloc_workspace().data_ptr(), self._stream())

    def attend(self, t: N.sd_tensors):
        N.sparse_decode_attend(self.handle, t, self.alloc_workspace().data_ptr(), self._stream())

    def combine(self, out: torch.Tensor, lse: torch.Tensor):
        assert out.dtype == torch.float32 and lse.dtype == torch.float32 and out.is_contiguous() and lse.is_contiguous()
        N.sparse_decode_combine(self.handle, self.alloc_workspace().data_ptr(), out.data_ptr(), lse.data_ptr(),
                                self._stream())

    def step(self, t: N.sd_tensors, out: torch.Tensor, lse: torch.Tensor):
        """score -> select (per level) -> attend -> combine, enqueued on the current stream by one
        library call (sparse_decode_step)."""
        assert out.dtype == torch.float32 and lse.dtype == torch.float32 and out.is_contiguous() and lse.is_contiguous()
        N.sparse_decode_step(self.handle, t, self.alloc_workspace().data_ptr(), out.data_ptr(), lse.data_ptr(),
                             self._stream())

    def status(self) -> int:
        """The device status word after the enqueued work (synchronises the current stream). It is
        an internal-invariant flag: 0 after every step on any input; nonzero means a library defect."""
        torch.cuda.current_stream().synchronize()
        return int(self.selection()["status"][0].item())

    # ---- inspection (device views into the workspace)
    def selection(self) -> dict:
        ws = self.alloc_workspace()
        v = N.sparse_decode_selection_view(self.handle, ws.data_ptr())
        base = ws.data_ptr()
        p = self.params
        B, Hq, Hk = p["batch"], p["n_q_heads"], p["n_kv_heads"]
        T = p.get("n_queries", 1) or 1
        G = Hq // Hk
        # the library orders a sequence's T x Hq query rows by KV group, then token, then head;
        # rows here come token-major (row t * Hq + h), like the outputs
        perm = torch.tensor([(h // G) * T * G + t * G + h % G for t in range(T) for h in range(Hq)],
                            device=ws.device)

        def view(ptr, dtype, shape):
            n = 1
            for s in shape:
                n *= s
            off = ptr - base
            es = torch.tensor([], dtype=dtype).element_size()
            return ws[off:off + n * es].view(dtype).view(*shape)

        def rows(x):
            return x if T == 1 else x.index_select(1, perm)

        out = {
            "scores0": rows(view(v.scores0, torch.float64, (B, T * Hq, v.len0))),
            "head_bits": rows(view(v.head_bits, torch.int32, (B, T * Hq, v.words))),
            "list": view(v.list, torch.int32, (B, Hk, v.n_entries)),
            "count": view(v.count, torch.int32, (B, Hk)),
            "status": view(v.status, torch.int32, (4,)),
        }
        if v.len1:
            out["scores1"] = rows(view(v.scores1, torch.float64, (B, T * Hq, v.len1)))
            out["cand1"] = rows(view(v.cand1, torch.int32, (B, T * Hq, v.len1)))
        return out
