"""Plain fp64 CPU oracle of query-adaptive sparse decode attention.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module; the decode library never does.

Sources (cited by page title and section):

* [SSA] AI Trends summary of "SSA / H-SSA" (aitrends.kr/articles/69798), sections
  "방법론" (method) and "기술 상세" (technical detail): relevance of chunk m to
  query q_t is ``s_{t,m} = q_t^T k_{g_m}``; the top-k chunks form I_t; K/V_hybrid
  is the union of the gist KV and raw KV of the chunks in I_t; standard attention
  runs over it. Section "핵심 기여" (contributions): H-SSA scores meta-gists
  first, keeps candidate segments, re-scores the gists inside them; decode
  builds a compact list of selected key indices, runs split-K partial attention
  and combines. Glossary "Grouped-Query Attention": per-head top-k, then the
  union over the group so every KV block is loaded once.
* [RTP] Review of "Full Attention Strikes Back" (blog.secrett2633.cloud),
  section "1. Key Terms & Definitions": retrieval heads keep the full KV cache; a
  16-dim low-dimensional projection scores token importance; dynamic top-p picks
  a per-query variable budget that secures attention mass instead of a fixed k.
* [TSA] Technical summary of "Token Sparse Attention", section 2 "Dynamic Token
  Coverage": token importance is the column sum of a proxy attention map; the
  budget comes from cutting the ascending-importance tail until the cut mass
  exceeds a coverage threshold tau; each head then keeps its own top-k.
* [HiLS] Review of "Hierarchical Sparse Attention Done Right", section 1: a
  landmark token's key summarises its chunk; GQA extended to group-wise chunk
  selection. Section 3 and the kernel figure: adjacent query tokens are grouped
  and their chunks' union is processed together.

Readings where the pages are silent (each is a fixed choice of this oracle):

* Order: scores sorted descending, equal scores by lower index first, so every
  selection is unique.
* Top-p: the minimal prefix of that order whose softmax mass (logits
  ``select_scale * s`` over ALL entries) reaches ``p * Z``; p >= 1 selects all.
* Forced chunks (sink / most recent) and the local-head window are added to the
  group union; they are not part of a head's own top-p set.
* Two-level: the top ``k_seg`` segments by meta score give candidate chunks in
  ascending order; the top ``k`` candidates by chunk score are kept in total.
* Hybrid context: the raw tokens of the selected chunks plus, when enabled, the
  summary K/V of those same chunks. Every head of a GQA group attends to the
  group union.
* Proxy scoring: the same d x r projection maps the query and the keys;
  ``q_p = q P`` in fp64, score ``q_p . k_p``.
* Coverage budget (decode form of [TSA]): the proxy attention map is the
  current query's per-head softmax over the chunk scores (``select_scale``);
  importance = the sum of the sequence's scored heads' probabilities; the
  ascending order breaks equal importance by the higher index first; the cut
  removes the shortest ascending prefix whose mass exceeds ``tau`` times the
  total; the budget ``k = max(1, entries - removed)`` is shared by every head of
  the sequence, each of which then keeps its own top-k.
* Variant "all summaries": the summary K/V of every chunk join the context,
  not only the selected chunks' ([SSA] 기술 상세 has the query interact with
  all summaries first); they are attended by every head of the group.
* Multi-query decode ([HiLS] section 3, kernel figure): a sequence may carry T
  adjacent query tokens; each (token, head) selects on its own, the group union
  runs over all T x G of them, and every one attends that union. The T tokens
  read the same cache (their past); their own keys are not in it.
* Variant "per-head masks": the group still loads the union once, but head h
  attends only to the raw (and selected-summary) rows of its own selection plus
  the forced sink / recent chunks; local groups are unmasked.
* Growing cache ([HiLS] section 3: decode advances by steps of adjacent tokens
  whose keys join the cache; [SSA] "주요 결과" / "관련 Figure": the per-step cost
  is followed as the context grows): at a step sequence b's cache holds n_b
  tokens (``ctx_len[b]``) of a larger capacity. Its complete chunks,
  ``n_b // chunk_size`` of them, are the ones with a summary key, so they are
  what is scored and selected; forced chunks count from 0 and from the last
  complete chunk; the raw tokens of the incomplete last chunk have no summary
  yet and are attended by every head of the group without being selected
  (within a chunk tokens see their own chunk's earlier tokens directly); local
  heads take the sink and the window of the n_b tokens.

Arithmetic: inputs arrive as fp64 (their bf16 / fp16 / fp32 values are exact in
fp64). Scores are summed in index order, one rounding per multiply and per
add. Attention uses fp64 matmuls and max-subtracted exponentials.
"""
from __future__ import annotations

import math

import numpy as np

TOPK, TOPP, HIER, PROXY_TOPP, COVERAGE = "topk", "topp", "hier", "proxy", "coverage"


# --------------------------------------------------------------------------- scores
def chunk_scores(q: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """[SSA] method: ``s_m = q^T k_{g_m}`` for every summary key row of ``keys``.

    ``q`` is [d], ``keys`` is [M, d]; the sum runs over i = 0..d-1 in order.
    """
    acc = np.zeros(keys.shape[0], dtype=np.float64)
    for i in range(q.shape[0]):
        acc = acc + q[i] * keys[:, i]
    return acc


def proxy_query(q: np.ndarray, P: np.ndarray) -> np.ndarray:
    """[RTP] key terms: the query's low-dimensional projection ``q_p = q P`` ([d] x [d, r])."""
    acc = np.zeros(P.shape[1], dtype=np.float64)
    for i in range(q.shape[0]):
        acc = acc + q[i] * P[i, :]
    return acc


def proxy_scores(qp: np.ndarray, Kp: np.ndarray) -> np.ndarray:
    """[RTP] key terms: token importance ``s_t = q_p . k_p[t]`` over the r proxy dims, in order."""
    acc = np.zeros(Kp.shape[0], dtype=np.float64)
    for j in range(qp.shape[0]):
        acc = acc + qp[j] * Kp[:, j]
    return acc


# ------------------------------------------------------------------------ selection
def order_desc(s: np.ndarray) -> np.ndarray:
    """Positions sorted by score descending; equal scores by lower position first."""
    return np.lexsort((np.arange(s.shape[0]), -s))


def select_top_k(s: np.ndarray, k: int) -> np.ndarray:
    """[SSA] method: the k highest-scoring entries (all of them when k >= len), ascending."""
    if k <= 0:
        raise ValueError("top-k needs k >= 1")
    return np.sort(order_desc(s)[: min(k, s.shape[0])])


def select_top_p(s: np.ndarray, p: float, scale: float):
    """[RTP] dynamic top-p: minimal descending prefix whose softmax mass reaches ``p``.

    Returns (ascending selection, margin). ``margin`` is the distance of the
    decision from the threshold, ``min(|c_n - pZ|, |c_{n-1} - pZ|) / Z``, where
    ``c_j`` is the mass of the first j entries of the order.
    """
    n = s.shape[0]
    if not p > 0:
        raise ValueError("top-p needs p > 0")
    if p >= 1.0:
        return np.arange(n), math.inf
    ell = scale * s
    mass = np.exp(ell - ell.max())
    Z = math.fsum(mass.tolist())
    target = p * Z
    o = order_desc(s)
    c = np.cumsum(mass[o])
    hit = np.nonzero(c >= target)[0]
    n_sel = int(hit[0]) + 1 if hit.size else n
    above = abs(c[n_sel - 1] - target)
    below = abs(c[n_sel - 2] - target) if n_sel >= 2 else abs(target)
    return np.sort(o[:n_sel]), min(above, below) / Z


def coverage_importance(score_rows, scale: float) -> np.ndarray:
    """[TSA] dynamic token coverage, scoring: every head's attention distribution over the
    entries (softmax of ``scale * s``), summed over the heads in order."""
    imp = np.zeros(score_rows[0].shape[0], dtype=np.float64)
    for s in score_rows:
        ell = scale * s
        mass = np.exp(ell - ell.max())
        imp = imp + mass / math.fsum(mass.tolist())
    return imp


def coverage_budget(imp: np.ndarray, tau: float):
    """[TSA] dynamic token coverage, budget: entries in ascending importance (equal importance:
    higher index first; the cumulative masses, hence the budget, do not depend on how ties are
    ordered); cut the tail until the cut mass exceeds ``tau`` times the total; the budget is what
    remains, at least 1. Returns (budget, margin of the cut decision / total)."""
    n = imp.shape[0]
    order = np.lexsort((-np.arange(n), imp))
    c = np.cumsum(imp[order])
    T = math.fsum(imp.tolist())
    thr = tau * T
    hit = np.nonzero(c > thr)[0]
    removed = int(hit[0]) + 1 if hit.size else n
    above = abs(c[removed - 1] - thr)
    below = abs(c[removed - 2] - thr) if removed >= 2 else abs(thr)
    return max(1, n - removed), (min(above, below) / T if T > 0 else math.inf)


def candidates(segments: np.ndarray, seg_size: int) -> np.ndarray:
    """[SSA] H-SSA: the chunks under the kept segments, ascending."""
    return (np.sort(segments)[:, None] * seg_size + np.arange(seg_size)[None, :]).ravel()


def select_two_level(s_seg: np.ndarray, score_chunks, k_seg: int, k: int, seg_size: int):
    """[SSA] H-SSA coarse-to-fine: top-k_seg segments, then top-k of their chunks.

    ``score_chunks(chunk_ids)`` returns the chunk scores of the candidates.
    Returns (selected chunk ids ascending, kept segments, candidates, candidate scores).
    """
    segs = select_top_k(s_seg, k_seg)
    cand = candidates(segs, seg_size)
    s2 = score_chunks(cand)
    pick = select_top_k(s2, k)
    return cand[pick], segs, cand, s2


def edge_entries(n: int, first: int, last: int) -> np.ndarray:
    """Entries [0, first) and [n - last, n): forced sink / recent chunks, or a local
    head's sink tokens plus sliding window."""
    a = np.arange(min(first, n))
    b = np.arange(max(0, n - last), n)
    return np.union1d(a, b)


def group_union(sets) -> np.ndarray:
    """[SSA] glossary GQA / [HiLS] section 1: union of the group's per-head selections."""
    u = np.zeros(0, dtype=np.int64)
    for s in sets:
        u = np.union1d(u, s)
    return u.astype(np.int64)


# ------------------------------------------------------------------------ attention
def attend(qh: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, scale: float):
    """Exact softmax attention of queries ``qh`` [G, d] over rows ``Kc, Vc`` [T, d].

    Returns (o [G, d], lse [G]) with ``lse = log sum_j exp(scale * q . k_j)``.
    """
    logits = scale * (Kc @ qh.T)                  # [T, G]
    mx = logits.max(axis=0)
    e = np.exp(logits - mx[None, :])
    L = e.sum(axis=0)
    o = (e.T @ Vc) / L[:, None]
    return o, mx + np.log(L)


def lse_combine(o_parts: np.ndarray, lse_parts: np.ndarray):
    """[SSA] decode kernel, combine stage: merge split partials (o_s, lse_s).

    ``LSE = log sum_s exp(lse_s)``, ``o = sum_s exp(lse_s - LSE) o_s``.
    """
    mx = lse_parts.max(axis=0)
    w = np.exp(lse_parts - mx[None, ...])
    L = w.sum(axis=0)
    o = (w[..., None] * o_parts).sum(axis=0) / L[..., None]
    return o, mx + np.log(L)


def hybrid_rows(U: np.ndarray, chunk_size: int) -> np.ndarray:
    """[SSA] technical detail: raw token positions of the selected chunks, ascending."""
    U = np.asarray(U, dtype=np.int64)
    return (U[:, None] * chunk_size + np.arange(chunk_size)[None, :]).ravel()


# ------------------------------------------------------------------------ the step
def group_queries(w, g: int) -> list:
    """Query rows of KV group g: every query token t of the sequence (T adjacent
    tokens, usually one) and every head g*G + j of the group, as indices
    ``t * Hq + h`` into the sequence's [T * Hq] query rows ([HiLS] section 3:
    adjacent query tokens share one union of chunks)."""
    G = w.n_q_heads // w.n_kv_heads
    T = getattr(w, "n_queries", 1)
    return [t * w.n_q_heads + g * G + j for t in range(T) for j in range(G)]


def cache_tokens(w, b: int, ctx_len=None) -> int:
    """Tokens sequence b's cache holds at this step: ctx_len[b] for a growing cache, else the
    whole cache."""
    return w.n_ctx if ctx_len is None else int(ctx_len[b])


def sequence_budget(w, src, b: int, n_ent=None):
    """Coverage budget of sequence b from all its scored query rows' chunk scores (over its first
    ``n_ent`` chunks, default all)."""
    bk = b if w.kv_batch > 1 else 0
    n_ent = w.n_ctx // w.chunk_size if n_ent is None else n_ent
    rows = [chunk_scores(src.q[b, qi], src.Kg[bk, g][:n_ent])
            for g in range(w.n_kv_heads) if g not in tuple(w.local_kv_heads) for qi in group_queries(w, g)]
    return coverage_budget(coverage_importance(rows, w.select_scale), w.tau)


def select_group(w, src, b: int, g: int, n_tok=None) -> dict:
    """Per-query-row selections (keyed by row ``t * Hq + h``) and the group union
    for sequence b, KV group g, over a cache of ``n_tok`` tokens (default: all of it)."""
    bk = b if w.kv_batch > 1 else 0
    n_tok = w.n_ctx if n_tok is None else n_tok
    n_ent = n_tok // w.chunk_size  # complete chunks: the ones with a summary key
    if n_tok != w.n_ctx and w.mode == HIER:
        raise ValueError("two-level selection reads whole caches")
    res = {"heads": {}, "scores": {}, "margin": math.inf, "segments": {}, "cand": {}}
    if g in tuple(w.local_kv_heads):
        res["union"] = edge_entries(n_ent, w.sink, w.window)
        return res
    per_head = []
    for h in group_queries(w, g):
        q = src.q[b, h]
        if n_ent == 0:  # nothing complete to score
            s, sel = np.zeros(0), np.zeros(0, dtype=np.int64)
        elif w.mode == TOPK:
            s = chunk_scores(q, src.Kg[bk, g][:n_ent])
            sel = select_top_k(s, w.top_k)
        elif w.mode == TOPP:
            s = chunk_scores(q, src.Kg[bk, g][:n_ent])
            sel, mg = select_top_p(s, w.top_p, w.select_scale)
            res["margin"] = min(res["margin"], mg)
        elif w.mode == HIER:
            s = chunk_scores(q, src.Kmg[bk, g])
            sel, segs, cand, s2 = select_two_level(
                s, lambda c: chunk_scores(q, src.Kg[bk, g][c]), w.top_k_seg, w.top_k, w.seg_size)
            res["segments"][h] = segs
            res["cand"][h] = (cand, s2)
        elif w.mode == COVERAGE:
            s = chunk_scores(q, src.Kg[bk, g][:n_ent])
            k_b, mg = sequence_budget(w, src, b, n_ent)
            sel = select_top_k(s, k_b)
            res["margin"] = min(res["margin"], mg)
            res["budget"] = k_b
        elif w.mode == PROXY_TOPP:
            qp = proxy_query(q, src.P[g])
            s = proxy_scores(qp, src.Kp[bk, g][:n_tok])
            sel, mg = select_top_p(s, w.top_p, w.select_scale)
            res["margin"] = min(res["margin"], mg)
        else:
            raise ValueError(w.mode)
        res["heads"][h] = sel
        res["scores"][h] = s
        per_head.append(sel)
    U = group_union(per_head)
    if w.keep_first or w.keep_last:
        U = group_union([U, edge_entries(n_ent, w.keep_first, w.keep_last)])
    res["union"] = U
    return res


def attend_group(w, src, b: int, g: int, U: np.ndarray, heads=None, n_tok=None):
    """The query heads of group g attend to the hybrid context of union U: raw
    rows of U's chunks and of the incomplete last chunk, then (``attend_summary``)
    the summary rows of U, or of every complete chunk with ``all_summaries``. With
    ``head_masks`` and a scored group, head h attends only to its own selection
    ``heads[h]`` plus the forced chunks and the incomplete chunk (summary rows of
    every chunk stay visible to all heads). ``n_tok``: tokens in the cache
    (default all); an empty context gives o = 0 and lse = -inf."""
    rows_q = group_queries(w, g)
    bk = b if w.kv_batch > 1 else 0
    n_tok = w.n_ctx if n_tok is None else n_tok
    n_ent = n_tok // w.chunk_size
    tail = np.arange(n_ent * w.chunk_size, n_tok)  # the incomplete last chunk's raw tokens
    summaries = w.attend_summary and w.mode != PROXY_TOPP
    all_sum = summaries and getattr(w, "all_summaries", False)
    masked = getattr(w, "head_masks", False) and g not in tuple(w.local_kv_heads)
    qh = src.q[b, rows_q]

    def context(S):
        rows = np.concatenate([hybrid_rows(S, w.chunk_size), tail]).astype(np.int64)
        Kc, Vc = src.kv_rows(bk, g, rows)
        if summaries:
            srows = np.arange(n_ent) if all_sum else np.asarray(S, dtype=np.int64)
            Kc = np.concatenate([Kc, src.Kg[bk, g][srows]], axis=0)
            Vc = np.concatenate([Vc, src.Vg[bk, g][srows]], axis=0)
        return Kc, Vc

    def attend_or_empty(q, Kc, Vc):
        if Kc.shape[0] == 0:
            return np.zeros((q.shape[0], w.head_dim)), np.full(q.shape[0], -np.inf)
        return attend(q, Kc, Vc, w.softmax_scale)

    if not masked:
        Kc, Vc = context(U)
        return attend_or_empty(qh, Kc, Vc)
    forced = edge_entries(n_ent, w.keep_first, w.keep_last)
    o = np.zeros((len(rows_q), w.head_dim))
    lse = np.zeros(len(rows_q))
    for j, qi in enumerate(rows_q):
        S = group_union([heads[qi], forced])
        Kc, Vc = context(S)
        oj, lj = attend_or_empty(qh[j:j + 1], Kc, Vc)
        o[j], lse[j] = oj[0], lj[0]
    return o, lse


def decode_step(w, src, groups=None, attend_groups=None, ctx_len=None) -> dict:
    """One decode step: selections for ``groups`` (default all (b, g)), attention
    for ``attend_groups`` (default the same), over caches of ``ctx_len[b]`` tokens
    (default whole). Returns per-(b, g) results and output / lse arrays [B][T * Hq]
    (NaN where not computed)."""
    B, Hq, Hk, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    T = getattr(w, "n_queries", 1)
    if groups is None:
        groups = [(b, g) for b in range(B) for g in range(Hk)]
    if attend_groups is None:
        attend_groups = groups
    out = np.full((B, T * Hq, d), np.nan)
    lse = np.full((B, T * Hq), np.nan)
    sel = {}
    for b, g in groups:
        sel[(b, g)] = select_group(w, src, b, g, cache_tokens(w, b, ctx_len))
    for b, g in attend_groups:
        n_tok = cache_tokens(w, b, ctx_len)
        if (b, g) not in sel:
            sel[(b, g)] = select_group(w, src, b, g, n_tok)
        o, l = attend_group(w, src, b, g, sel[(b, g)]["union"], sel[(b, g)]["heads"], n_tok)
        out[b, group_queries(w, g)] = o
        lse[b, group_queries(w, g)] = l
    return {"sel": sel, "out": out, "lse": lse}
