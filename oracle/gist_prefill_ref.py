"""Plain fp64 CPU oracle of gist-masked (SSA) block-sparse prefill attention.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module; the library never does.

Source: [SSA] review of "Simplified Sparse Attention" (aitrends.kr, article
69798): "핵심 기여" (contributions) -- the prefill kernel recovers a block-sparse
pattern by permuting the key columns and skips the empty blocks; "방법론"
(method) and "기술 상세" (technical details) -- the input is split into chunks of
C raw tokens, a gist token follows every chunk, and the gist causal mask keeps a
chunk's tokens from reaching the raw tokens of earlier chunks directly: what
came before reaches them only through the gists.

Readings where the page is silent (fixed choices of this oracle):

* Sequence: N = M C raw tokens in M whole chunks; gist m follows chunk m, so in
  the interleaved order raw token i of chunk m sits at m (C + 1) + i and gist m
  at m (C + 1) + C.
* Mask: causal in the interleaved order, and a raw key is visible only to the
  queries of its own chunk (raw tokens after it and the chunk's gist). Hence raw
  token t (chunk m = t // C) sees gists 0 .. m - 1 and raw tokens m C .. t;
  gist m sees gists 0 .. m and the C raw tokens of chunk m.
* Key-column permutation: the keys are taken as [gists 0 .. M - 1 | raw tokens
  0 .. N - 1]; every query's visible keys are then a prefix of the gists plus a
  run of its own chunk's raw tokens, the block-sparse layout the kernel tiles.
* Attention: softmax of ``softmax_scale * q . k`` over the visible keys of the
  query head's KV group (h // G), in fp64 with max subtraction; outputs for the
  N raw and the M gist queries.

Arithmetic: inputs arrive as fp64 (their bf16 values are exact in fp64).
"""
from __future__ import annotations

import numpy as np

from .sparse_decode_ref import attend


def visible_keys(w, kind: str, i: int):
    """[SSA] gist causal mask after the key-column permutation: (gist key indices, raw key indices)
    visible to query i of ``kind`` "raw" (token i) or "gist" (gist i)."""
    C = w.chunk_size
    if kind == "raw":
        m = i // C
        return np.arange(m), np.arange(m * C, i + 1)
    return np.arange(i + 1), np.arange(i * C, (i + 1) * C)


def gp_attend_rows(w, src, b: int, h: int, kind: str, rows) -> tuple:
    """Attention of the queries ``rows`` of ``kind`` of head h over their visible keys.
    Returns (o [n, d], lse [n])."""
    g = h // (w.n_q_heads // w.n_kv_heads)
    o = np.zeros((len(rows), w.head_dim))
    lse = np.zeros(len(rows))
    for n, i in enumerate(rows):
        gj, rj = visible_keys(w, kind, i)
        Kg, Vg = src.gist_kv_rows(b, g, gj)
        Kr, Vr = src.raw_kv_rows(b, g, rj)
        Kc = np.concatenate([Kg, Kr], axis=0)
        Vc = np.concatenate([Vg, Vr], axis=0)
        oi, li = attend(src.q_row(b, h, kind, i)[None, :], Kc, Vc, w.softmax_scale)
        o[n], lse[n] = oi[0], li[0]
    return o, lse


def gist_prefill(w, src, raw_rows=None, gist_rows=None) -> dict:
    """Outputs O [B][Hq][N][d] for the raw queries and Og [B][Hq][M][d] for the gist queries; with
    ``raw_rows`` / ``gist_rows`` only those query indices are computed (the rest stays NaN)."""
    B, Hq, d, C = w.batch, w.n_q_heads, w.head_dim, w.chunk_size
    N = w.n_tokens
    M = N // C
    O = np.full((B, Hq, N, d), np.nan)
    Og = np.full((B, Hq, M, d), np.nan)
    rr = list(range(N)) if raw_rows is None else list(raw_rows)
    gr = list(range(M)) if gist_rows is None else list(gist_rows)
    for b in range(B):
        for h in range(Hq):
            if rr:
                O[b, h, rr] = gp_attend_rows(w, src, b, h, "raw", rr)[0]
            if gr:
                Og[b, h, gr] = gp_attend_rows(w, src, b, h, "gist", gr)[0]
    return {"out": O, "out_gist": Og}
