"""Plain fp64 CPU oracle of Token-Sparse prefill attention.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module; the library never does.

Source: [TSA] Technical summary of "Token Sparse Attention" (gist.science,
paper 2602.03216), section 2 "방법론" (method): per attention head a subset S_h
of token positions is chosen, Q, K and V are gathered at S_h into compact dense
tensors, attention runs on them, and the compact output is scattered back into
a zero-initialised sequence-length output at the head's positions (the residual
stream keeps the skipped tokens). "동적 토큰 커버리지" (dynamic token coverage):
a light proxy attention map of the most recent queries against every key gives
token importance as column sums; the tokens are taken in ascending importance
and the low tail is cut until its mass exceeds tau; that global budget k is then
applied by every head to its own scores (top-k per head).

Readings where the page is silent (fixed choices of this oracle):

* Proxy map: per query head h, the last W query positions of the sequence
  (W = ``window``) attend causally (key position <= query position) to the
  head's KV group; logits ``softmax_scale * q . k`` with the dot product summed
  in index order in fp64; each row is softmax-normalised; head h's importance of
  key j is the sum over the W rows, in row order.
* Budget: the heads' importances summed per position in head order; the
  coverage cut of the decode oracle (``coverage_budget``): ascending order, the
  shortest prefix whose mass exceeds ``tau`` times the total is removed,
  ``k = max(1, L - removed)``.
* Per-head selection: head h keeps the k positions of highest importance_h
  (equal importance: lower position first), ascending.
* Compressed attention: the head's queries, keys and values at S_h, causal in
  position order (compact row i attends compact rows 0..i), softmax scale
  ``softmax_scale``; output rows scattered back to positions S_h, every other
  row of the head is zero. Keys and values come from the head's KV group
  (h // G).
* Mixed heads ([EA] technical summary of "Elastic Attention" (gist.science,
  paper 2601.17367), sections 2.1 and 2.3: a router assigns every attention head full attention (FA) or sparse
  attention (SA), and one fused kernel runs all heads): ``head_mode[h] = 1``
  marks a full-attention query head, 0 a sparse one (the router's decision is an
  input; the page does not define SA's pattern, read here as the Token-Sparse
  selection above). Full heads keep every position (plain causal attention);
  the budget is the coverage cut of the sparse heads' importances only.

Arithmetic: inputs arrive as fp64 (their bf16 values are exact in fp64).
"""
from __future__ import annotations

import math

import numpy as np

from .sparse_decode_ref import attend, coverage_budget, order_desc, select_top_k


def window_scores(Qw: np.ndarray, K: np.ndarray) -> np.ndarray:
    """``s[i, j] = q_i . k_j`` for the window queries Qw [W, d] and keys K [L, d], summed over the
    dimensions in index order (one rounding per multiply and per add)."""
    acc = np.zeros((Qw.shape[0], K.shape[0]), dtype=np.float64)
    for i in range(Qw.shape[1]):
        acc = acc + Qw[:, i][:, None] * K[:, i][None, :]
    return acc


def proxy_importance(Qw: np.ndarray, K: np.ndarray, scale: float, pos0: int) -> np.ndarray:
    """[TSA] dynamic token coverage, scoring: the causal softmax map of the window queries (at
    positions pos0, pos0 + 1, ...) over the keys, summed over the window rows per key."""
    s = window_scores(Qw, K)
    L = K.shape[0]
    imp = np.zeros(L, dtype=np.float64)
    for i in range(Qw.shape[0]):
        vis = pos0 + i + 1                         # keys 0 .. pos0 + i are visible
        ell = scale * s[i, :vis]
        e = np.exp(ell - ell.max())
        imp[:vis] = imp[:vis] + e / math.fsum(e.tolist())
    return imp


def head_modes(w) -> list:
    """[EA] head-wise routing: 1 = full-attention head, 0 = sparse head (all sparse by default)."""
    m = getattr(w, "head_mode", None)
    return [0] * w.n_q_heads if m is None else [int(x) for x in m]


def head_importances(w, src, b: int, pool_map=map) -> list:
    """[TSA] dynamic token coverage, scoring: every query head's proxy-map importance for
    sequence b, head by head (``pool_map`` may evaluate the heads concurrently; each head's
    arithmetic is ``proxy_importance`` alone)."""
    L, W, Hq = w.seq_len, w.window, w.n_q_heads
    G = Hq // w.n_kv_heads

    def one(h):
        Qw = src.q_rows(b, h, np.arange(L - W, L))
        return proxy_importance(Qw, src.k_all(b, h // G), w.softmax_scale, L - W)

    return list(pool_map(one, range(Hq)))


def select_from_importances(w, imps: list) -> dict:
    """The global budget and every head's positions from the heads' importances ([TSA] dynamic
    token coverage: budget from the summed importance of the sparse heads, then top-k per head)."""
    L, Hq = w.seq_len, w.n_q_heads
    modes = head_modes(w)
    total = np.zeros(L, dtype=np.float64)
    for h in range(Hq):
        if not modes[h]:
            total = total + imps[h]
    k, margin = coverage_budget(total, w.tau)
    sets, gaps = {}, {}
    for h in range(Hq):
        if modes[h]:
            sets[h], gaps[h] = np.arange(L), math.inf
            continue
        sets[h] = select_top_k(imps[h], k)
        o = order_desc(imps[h])
        gaps[h] = abs(imps[h][o[k - 1]] - imps[h][o[k]]) if k < L else math.inf
    return {"importance": imps, "budget": k, "margin": margin, "sets": sets, "gaps": gaps}


def tsa_select(w, src, b: int, pool_map=map) -> dict:
    """Per-head importances, the global budget and every head's positions for sequence b."""
    return select_from_importances(w, head_importances(w, src, b, pool_map=pool_map))


def tsa_attend_rows(w, src, b: int, h: int, S: np.ndarray, rows) -> tuple:
    """[TSA] compression and attention: compact rows ``rows`` (indices into S) of head h attend
    the head's compact keys 0..i. Returns (o [n, d], lse [n]) for those rows."""
    G = w.n_q_heads // w.n_kv_heads
    g = h // G
    o = np.zeros((len(rows), w.head_dim))
    lse = np.zeros(len(rows))
    for n, i in enumerate(rows):
        keys = S[:i + 1]
        Kc, Vc = src.kv_rows(b, g, keys)
        oi, li = attend(src.q_rows(b, h, S[i:i + 1]), Kc, Vc, w.softmax_scale)
        o[n], lse[n] = oi[0], li[0]
    return o, lse


def tsa_prefill(w, src, heads=None, rows_per_head=None, seed=0) -> dict:
    """Selection of every sequence, and the scattered output O [B][Hq][L][d] for ``heads``
    (default all); with ``rows_per_head`` only that many sampled compact rows per head are
    computed (the rest of O stays NaN, the unselected positions stay 0)."""
    B, Hq, L, d = w.batch, w.n_q_heads, w.seq_len, w.head_dim
    rng = np.random.default_rng(seed)
    sel = [tsa_select(w, src, b) for b in range(B)]
    O = np.full((B, Hq, L, d), np.nan)
    for b in range(B):
        for h in (range(Hq) if heads is None else heads):
            S = sel[b]["sets"][h]
            O[b, h] = 0.0
            O[b, h, S] = np.nan
            rows = range(len(S)) if rows_per_head is None else sorted(
                set(rng.choice(len(S), min(rows_per_head, len(S)), replace=False).tolist()) | {0, len(S) - 1})
            o, _ = tsa_attend_rows(w, src, b, h, S, list(rows))
            O[b, h, S[list(rows)]] = o
    return {"sel": sel, "out": O}
