"""Checks that pin the oracle to things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle module ``ref``
disagrees with a hand-derived closed form, a library routine it does not use, a
brute-force search or an invariant. ``tests/test_oracle_pins.py`` runs them on
the real oracle; ``tests/test_oracle_mutations.py`` runs them on copies of the
oracle with planted mistakes and expects each mistake to be caught.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- golden fixtures
def pin_golden_scores(ref):
    fx = _load("scores_dot.json")
    s = ref.chunk_scores(np.array(fx["q"], float), np.array(fx["keys"], float))
    assert np.array_equal(s, np.array(fx["expected"], float)), s


def pin_golden_proxy(ref):
    fx = _load("proxy_scores.json")
    qp = ref.proxy_query(np.array(fx["q"], float), np.array(fx["P"], float))
    assert np.array_equal(qp, np.array(fx["expected_qp"], float)), qp
    s = ref.proxy_scores(qp, np.array(fx["Kp"], float))
    assert np.array_equal(s, np.array(fx["expected"], float)), s


def pin_golden_topk(ref):
    fx = _load("topk_ties.json")
    s = np.array(fx["scores"], float)
    for k, exp in fx["cases"]:
        got = ref.select_top_k(s, k)
        assert got.tolist() == exp, (k, got)


def pin_golden_topp(ref):
    fx = _load("topp_masses.json")
    s = np.array(fx["scores"], float)
    for p, exp, margin in fx["cases"]:
        got, mg = ref.select_top_p(s, p, fx["select_scale"])
        assert got.tolist() == exp, (p, got)
        if margin is not None:
            assert abs(mg - margin) < 1e-12, (p, mg)


def pin_golden_two_level(ref):
    fx = _load("two_level.json")
    s1 = np.array(fx["segment_scores"], float)
    cs = np.array(fx["chunk_scores"], float)
    for k, exp in fx["cases"]:
        sel, segs, cand, _ = ref.select_two_level(s1, lambda c: cs[c], fx["k_seg"], k, fx["seg_size"])
        assert segs.tolist() == fx["expected_segments"], segs
        assert cand.tolist() == fx["expected_candidates"], cand
        assert sel.tolist() == exp, (k, sel)


def pin_golden_union(ref):
    fx = _load("union_forced.json")
    U = ref.group_union([np.array(h) for h in fx["heads"]]
                        + [ref.edge_entries(fx["n"], fx["keep_first"], fx["keep_last"])])
    assert U.tolist() == fx["expected_union"], U
    for n, sink, window, exp in fx["local_cases"]:
        assert ref.edge_entries(n, sink, window).tolist() == exp


def pin_golden_attention(ref):
    fx = _load("attention_closed_form.json")
    q, K, V = (np.array(fx[k], float) for k in ("q", "K", "V"))
    o, lse = ref.attend(q, K, V, fx["scale"])
    assert np.allclose(o, fx["expected_o"], rtol=0, atol=1e-12), o
    assert np.allclose(lse, fx["expected_lse"], rtol=0, atol=1e-12), lse
    oc, lc = ref.lse_combine(np.array(fx["split_o"], float), np.array(fx["split_lse"], float))
    assert np.allclose(oc, fx["expected_o"], rtol=0, atol=1e-12), oc
    assert np.allclose(lc, fx["expected_lse"], rtol=0, atol=1e-12), lc


# ---------------------------------------------------------------- exact arithmetic
def pin_scores_exact(ref, seed=0):
    """Dyadic inputs: every product and partial sum is exact, so the fp64 score
    equals the rational dot product; random floats agree with math.fsum."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-64, 64, 96) / 8.0
    K = rng.integers(-64, 64, (40, 96)) / 16.0
    s = ref.chunk_scores(q, K)
    exact = [float(sum(Fraction(a) * Fraction(b) for a, b in zip(q, row))) for row in K]
    assert np.array_equal(s, np.array(exact)), "score is not q.k"
    qf = rng.standard_normal(128)
    Kf = rng.standard_normal((30, 128))
    s = ref.chunk_scores(qf, Kf)
    ref_s = np.array([math.fsum((qf * row).tolist()) for row in Kf])
    assert np.allclose(s, ref_s, rtol=1e-12, atol=1e-12)
    P = rng.integers(-8, 8, (96, 16)) / 4.0
    qp = ref.proxy_query(q, P)
    exact_qp = [float(sum(Fraction(q[i]) * Fraction(P[i, j]) for i in range(96))) for j in range(16)]
    assert np.array_equal(qp, np.array(exact_qp))
    Kp = rng.integers(-32, 32, (50, 16)) / 2.0
    sp = ref.proxy_scores(qp, Kp)
    exact_sp = [float(sum(Fraction(qp[j]) * Fraction(row[j]) for j in range(16))) for row in Kp]
    assert np.array_equal(sp, np.array(exact_sp))


# ---------------------------------------------------------------- brute force
def _brute_topk(s, k):
    n = len(s)
    k = min(k, n)
    best = None
    for comb in itertools.combinations(range(n), k):
        key = (-sum(Fraction(float(s[i])) for i in comb), comb)
        if best is None or key < best:
            best = key
    return list(best[1])


def _brute_topp(s, p, scale):
    n = len(s)
    if p >= 1:
        return list(range(n))
    mx = max(scale * float(x) for x in s)
    mass = [Fraction(math.exp(scale * float(x) - mx)) for x in s]
    Z = sum(mass)
    for size in range(1, n + 1):
        best = None
        for comb in itertools.combinations(range(n), size):
            m = sum(mass[i] for i in comb)
            if m >= Fraction(p) * Z:
                key = (-m, comb)
                if best is None or key < best:
                    best = key
        if best is not None:
            return list(best[1])
    return list(range(n))


def pin_bruteforce(ref, trials=60, seed=1):
    """Top-k and top-p sets equal an exhaustive subset search on tiny rows with
    small-integer scores (exact, with deliberate ties)."""
    rng = np.random.default_rng(seed)
    for t in range(trials):
        n = int(rng.integers(1, 11))
        s = rng.integers(-3, 4, n).astype(float)
        k = int(rng.integers(1, n + 2))
        assert ref.select_top_k(s, k).tolist() == _brute_topk(s, k), ("topk", s, k)
        p = float(rng.choice([0.1, 0.33, 0.5, 0.77, 0.9, 0.99, 1.0]))
        scale = float(rng.choice([0.5, 1.0, 1.7]))
        got, mg = ref.select_top_p(s, p, scale)
        if mg > 1e-9:
            assert got.tolist() == _brute_topp(s, p, scale), ("topp", s, p, scale)


# ---------------------------------------------------------------- invariants
def pin_topp_minimal(ref, trials=40, seed=2):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        n = int(rng.integers(2, 3000))
        s = rng.standard_normal(n) * float(rng.choice([0.3, 3.0, 30.0]))
        p = float(rng.uniform(0.05, 0.999))
        scale = float(rng.choice([0.1, 1.0]))
        S, mg = ref.select_top_p(s, p, scale)
        mass = np.exp(scale * s - np.max(scale * s))
        Z = math.fsum(mass.tolist())
        order = np.lexsort((np.arange(n), -s))
        assert sorted(order[:len(S)].tolist()) == S.tolist(), "not a prefix of the order"
        if mg > 1e-12:
            inc = math.fsum(mass[S].tolist())
            last = order[len(S) - 1]
            exc = inc - mass[last]
            assert inc >= p * Z, "mass below p"
            assert exc < p * Z, "not minimal"


def pin_reductions(ref, seed=3):
    rng = np.random.default_rng(seed)
    for t in range(30):
        n = int(rng.integers(1, 200))
        s = rng.integers(-5, 5, n).astype(float)
        assert ref.select_top_k(s, 1).tolist() == [int(np.argmax(s))]
    # two-level with every segment kept equals flat top-k
    for t in range(20):
        S, sg = int(rng.integers(1, 12)), int(rng.integers(1, 9))
        cs = rng.integers(-4, 4, S * sg).astype(float)
        s1 = rng.standard_normal(S)
        k = int(rng.integers(1, S * sg + 2))
        sel, _, _, _ = ref.select_two_level(s1, lambda c: cs[c], S, k, sg)
        assert sel.tolist() == ref.select_top_k(cs, k).tolist()


def pin_union(ref, seed=4):
    rng = np.random.default_rng(seed)
    for t in range(20):
        sets = [np.sort(rng.choice(100, int(rng.integers(0, 30)), replace=False)) for _ in range(5)]
        U = ref.group_union(sets)
        assert np.all(np.diff(U) > 0)
        assert set(U.tolist()) == set().union(*[set(x.tolist()) for x in sets])


def _sdpa(qh, Kc, Vc, scale, mask=None):
    q = torch.from_numpy(qh)[None, :, None, :]          # [1, G, 1, d]
    k = torch.from_numpy(Kc)[None, None].expand(1, qh.shape[0], -1, -1)
    v = torch.from_numpy(Vc)[None, None].expand(1, qh.shape[0], -1, -1)
    am = None
    if mask is not None:
        am = torch.full((Kc.shape[0],), -math.inf, dtype=torch.float64)
        am[torch.from_numpy(mask)] = 0.0
        am = am[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=am, scale=scale)
    logits = scale * (torch.from_numpy(Kc) @ torch.from_numpy(qh).T)   # [T, G]
    if mask is not None:
        logits = logits + am[0, 0, 0][:, None]
    lse = torch.logsumexp(logits, dim=0)
    return o[0, :, 0, :].numpy(), lse.numpy()


def pin_masked_dense(ref, seed=5):
    """Attention over any index set equals dense attention with -inf outside it
    (torch SDPA in fp64), and the split-K combine of any partition equals it too."""
    rng = np.random.default_rng(seed)
    for t in range(10):
        T, d, G = int(rng.integers(2, 300)), int(rng.choice([8, 64])), int(rng.integers(1, 8))
        K, V = rng.standard_normal((T, d)), rng.standard_normal((T, d))
        qh = rng.standard_normal((G, d)) * 2
        scale = 1 / math.sqrt(d)
        U = np.sort(rng.choice(T, int(rng.integers(1, T + 1)), replace=False))
        o, lse = ref.attend(qh, K[U], V[U], scale)
        o2, lse2 = _sdpa(qh, K, V, scale, mask=U)
        assert np.allclose(o, o2, rtol=1e-12, atol=1e-12), "masked attention"
        assert np.allclose(lse, lse2, rtol=1e-12, atol=1e-12), "masked lse"
        cuts = np.sort(rng.choice(np.arange(1, len(U)), min(len(U) - 1, int(rng.integers(0, 6))), replace=False)) if len(U) > 1 else []
        parts = np.split(U, cuts)
        po, pl = zip(*[ref.attend(qh, K[p], V[p], scale) for p in parts])
        oc, lc = ref.lse_combine(np.stack(po), np.stack(pl))
        assert np.allclose(oc, o2, rtol=1e-12, atol=1e-12), "combine"
        assert np.allclose(lc, lse2, rtol=1e-12, atol=1e-12), "combine lse"


def _tiny_workload(mode, **kw):
    base = dict(name="pin", batch=2, kv_batch=2, n_q_heads=6, n_kv_heads=2, head_dim=16, n_ctx=96,
                chunk_size=8, mode=mode, top_k=3, top_k_seg=2, seg_size=4, top_p=0.9,
                select_scale=0.25, softmax_scale=0.25, keep_first=0, keep_last=0, route_dim=4,
                local_kv_heads=(), sink=0, window=0, attend_summary=True, all_summaries=False,
                head_masks=False, tau=0.0)
    base.update(kw)
    return SimpleNamespace(**base)


class _Src:
    def __init__(self, w, rng):
        B, Hq, Hk, d, N = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx
        M = N // w.chunk_size
        self.q = rng.standard_normal((B, getattr(w, "n_queries", 1) * Hq, d))  # rows t * Hq + h
        self.K = rng.standard_normal((w.kv_batch, Hk, N, d))
        self.V = rng.standard_normal((w.kv_batch, Hk, N, d))
        self.Kg = rng.standard_normal((w.kv_batch, Hk, M, d))
        self.Vg = rng.standard_normal((w.kv_batch, Hk, M, d))
        self.Kmg = rng.standard_normal((w.kv_batch, Hk, max(1, M // max(1, w.seg_size)), d))
        self.P = rng.standard_normal((Hk, d, w.route_dim))
        self.Kp = rng.standard_normal((w.kv_batch, Hk, N, w.route_dim))

    def kv_rows(self, bk, g, rows):
        return self.K[bk, g][rows], self.V[bk, g][rows]


def pin_dense_limits(ref, seed=6):
    """k = all chunks, p = 1, and two-level keeping everything all reduce the
    step to dense attention over [raw K; summary K] (torch SDPA, fp64); local
    heads reduce to dense attention over their sink + window slice."""
    rng = np.random.default_rng(seed)
    cases = [
        _tiny_workload("topk", top_k=12),
        _tiny_workload("topk", top_k=50),
        _tiny_workload("topp", top_p=1.0),
        _tiny_workload("hier", top_k_seg=3, top_k=12, seg_size=4),
        _tiny_workload("proxy", chunk_size=1, top_p=1.0, attend_summary=False),
        _tiny_workload("proxy", chunk_size=1, top_p=1.0, attend_summary=False, local_kv_heads=(1,),
                       sink=5, window=17),
    ]
    for w in cases:
        src = _Src(w, rng)
        res = ref.decode_step(w, src)
        G = w.n_q_heads // w.n_kv_heads
        for b in range(w.batch):
            for g in range(w.n_kv_heads):
                qh = src.q[b, g * G:(g + 1) * G]
                if g in w.local_kv_heads:
                    rows = np.r_[0:w.sink, w.n_ctx - w.window:w.n_ctx]
                    Kc, Vc = src.K[b, g][rows], src.V[b, g][rows]
                elif w.attend_summary and w.mode != "proxy":
                    Kc = np.concatenate([src.K[b, g], src.Kg[b, g]])
                    Vc = np.concatenate([src.V[b, g], src.Vg[b, g]])
                else:
                    Kc, Vc = src.K[b, g], src.V[b, g]
                o2, l2 = _sdpa(qh, Kc, Vc, w.softmax_scale)
                assert np.allclose(res["out"][b, g * G:(g + 1) * G], o2, rtol=1e-11, atol=1e-11), (w.mode, b, g)
                assert np.allclose(res["lse"][b, g * G:(g + 1) * G], l2, rtol=1e-11, atol=1e-11), (w.mode, b, g)


def pin_step_masked(ref, seed=7):
    """A sparse step equals dense attention masked to its own union, and each
    head's set is inside the union; top-k sets have exactly k entries."""
    rng = np.random.default_rng(seed)
    for w in (_tiny_workload("topk", keep_first=1, keep_last=2), _tiny_workload("topp", top_p=0.7),
              _tiny_workload("hier"), _tiny_workload("proxy", chunk_size=1, top_p=0.6, attend_summary=False)):
        src = _Src(w, rng)
        res = ref.decode_step(w, src)
        G = w.n_q_heads // w.n_kv_heads
        M = w.n_ctx // w.chunk_size
        for (b, g), r in res["sel"].items():
            U = r["union"]
            forced = set(range(min(w.keep_first, M))) | set(range(max(0, M - w.keep_last), M))
            heads_u = set().union(*[set(S.tolist()) for S in r["heads"].values()])
            assert set(U.tolist()) == heads_u | forced, "union is not heads + forced entries"
            for h, S in r["heads"].items():
                assert set(S.tolist()) <= set(U.tolist())
                if w.mode in ("topk", "hier"):
                    assert len(S) == min(w.top_k, M if w.mode == "topk" else w.top_k_seg * w.seg_size)
            rows = (U[:, None] * w.chunk_size + np.arange(w.chunk_size)).ravel()
            mask = rows
            Kc, Vc = src.K[b, g], src.V[b, g]
            if w.attend_summary and w.mode != "proxy":
                Kc = np.concatenate([Kc, src.Kg[b, g]])
                Vc = np.concatenate([Vc, src.Vg[b, g]])
                mask = np.concatenate([rows, w.n_ctx + U])
            qh = src.q[b, g * G:(g + 1) * G]
            o2, l2 = _sdpa(qh, Kc, Vc, w.softmax_scale, mask=mask)
            assert np.allclose(res["out"][b, g * G:(g + 1) * G], o2, rtol=1e-11, atol=1e-11), w.mode
            assert np.allclose(res["lse"][b, g * G:(g + 1) * G], l2, rtol=1e-11, atol=1e-11), w.mode


def pin_step_selection(ref, seed=8):
    """Per-head sets of a whole step equal the brute-force sets of that head's
    scores (scores re-derived here with math.fsum)."""
    rng = np.random.default_rng(seed)
    w = _tiny_workload("topp", n_ctx=64, chunk_size=8, top_p=0.8, keep_first=1)
    src = _Src(w, rng)
    res = ref.decode_step(w, src)
    G = w.n_q_heads // w.n_kv_heads
    for (b, g), r in res["sel"].items():
        for h, S in r["heads"].items():
            s = np.array([math.fsum((src.q[b, h] * k).tolist()) for k in src.Kg[b, g]])
            assert S.tolist() == _brute_topp(s, w.top_p, w.select_scale), (b, h)
        assert 0 in r["union"].tolist()
    w = _tiny_workload("topk", n_ctx=80, chunk_size=8, top_k=4)
    src = _Src(w, rng)
    res = ref.decode_step(w, src)
    for (b, g), r in res["sel"].items():
        for h, S in r["heads"].items():
            s = np.array([math.fsum((src.q[b, h] * k).tolist()) for k in src.Kg[b, g]])
            assert S.tolist() == _brute_topk(s, w.top_k), (b, h)


def pin_variants(ref, seed=9):
    """The two context variants against dense attention with masks built here from their
    definitions (torch SDPA, fp64): with per-head masks head h sees the raw and summary rows of its
    own set plus the forced chunks (local groups: the sink + window); with all summaries every head
    sees the union's raw rows plus every chunk's summary. With one head per group and no forced
    chunks the per-head masks change nothing."""
    rng = np.random.default_rng(seed)
    cases = [
        _tiny_workload("topk", keep_first=1, keep_last=2, head_masks=True, all_summaries=False),
        _tiny_workload("topp", top_p=0.7, head_masks=True, all_summaries=False),
        _tiny_workload("hier", head_masks=True, all_summaries=False),
        _tiny_workload("proxy", chunk_size=1, top_p=0.6, attend_summary=False, head_masks=True,
                       all_summaries=False, local_kv_heads=(1,), sink=3, window=9),
        _tiny_workload("topp", top_p=0.7, keep_last=1, head_masks=False, all_summaries=True),
        _tiny_workload("topk", keep_first=2, head_masks=True, all_summaries=True),
    ]
    for w in cases:
        src = _Src(w, rng)
        res = ref.decode_step(w, src)
        G = w.n_q_heads // w.n_kv_heads
        M = w.n_ctx // w.chunk_size
        forced = [e for e in range(M) if e < w.keep_first or e >= M - w.keep_last]
        summ = w.attend_summary and w.mode != "proxy"
        for (b, g), r in res["sel"].items():
            Kc, Vc = src.K[b, g], src.V[b, g]
            if summ:
                Kc = np.concatenate([Kc, src.Kg[b, g]])
                Vc = np.concatenate([Vc, src.Vg[b, g]])
            for j in range(G):
                h = g * G + j
                if g in w.local_kv_heads:
                    chunks = [e for e in range(M) if e < w.sink or e >= M - w.window]
                elif w.head_masks:
                    chunks = sorted(set(r["heads"][h].tolist()) | set(forced))
                else:
                    chunks = r["union"].tolist()
                mask = [c * w.chunk_size + t for c in chunks for t in range(w.chunk_size)]
                if summ:
                    mask += [w.n_ctx + e for e in (range(M) if w.all_summaries else chunks)]
                o2, l2 = _sdpa(src.q[b, h][None], Kc, Vc, w.softmax_scale, mask=np.array(mask))
                assert np.allclose(res["out"][b, h], o2[0], rtol=1e-11, atol=1e-11), (w.mode, b, h)
                assert np.allclose(res["lse"][b, h], l2[0], rtol=1e-11, atol=1e-11), (w.mode, b, h)
    w1 = _tiny_workload("topp", n_q_heads=2, n_kv_heads=2, top_p=0.8, head_masks=True, all_summaries=False)
    w0 = _tiny_workload("topp", n_q_heads=2, n_kv_heads=2, top_p=0.8, head_masks=False, all_summaries=False)
    src = _Src(w1, np.random.default_rng(seed + 1))
    a, c = ref.decode_step(w1, src), ref.decode_step(w0, src)
    assert np.array_equal(a["out"], c["out"]) and np.array_equal(a["lse"], c["lse"]), "G = 1 masks"


def _brute_coverage(score_rows, scale, tau):
    """Budget by the definition, every quantity re-derived: probabilities with math.exp and
    math.fsum, importance summed per entry over the heads, the cut walked one entry at a time."""
    n = len(score_rows[0])
    imp = [0.0] * n
    for s in score_rows:
        mx = max(scale * x for x in s)
        e = [math.exp(scale * x - mx) for x in s]
        Z = math.fsum(e)
        for m in range(n):
            imp[m] += e[m] / Z
    T = math.fsum(imp)
    order = sorted(range(n), key=lambda m: (imp[m], -m))
    cut, removed = 0.0, 0
    for m in order:
        cut += imp[m]
        removed += 1
        if cut > tau * T:
            break
    return max(1, n - removed)


def pin_coverage(ref, seed=10):
    """Coverage budget: equals the definition walked entry by entry; tau = 0 removes exactly one
    entry; the budget never grows with tau; in a step every scored head keeps exactly its own
    top-budget entries (brute force over its scores)."""
    rng = np.random.default_rng(seed)
    for t in range(30):
        n, H = int(rng.integers(2, 40)), int(rng.integers(1, 6))
        rows = [rng.standard_normal(n) * rng.choice([0.3, 3.0]) for _ in range(H)]
        scale, tau = float(rng.choice([0.5, 1.0, 2.0])), float(rng.uniform(0, 0.95))
        k, _ = ref.coverage_budget(ref.coverage_importance(rows, scale), tau)
        assert k == _brute_coverage(rows, scale, tau), (t, k)
        k0, _ = ref.coverage_budget(ref.coverage_importance(rows, scale), 0.0)
        assert k0 == n - 1, "tau = 0"
        ks = [ref.coverage_budget(ref.coverage_importance(rows, scale), x)[0] for x in (0.1, 0.3, 0.6, 0.9)]
        assert ks == sorted(ks, reverse=True), "budget grows with tau"
    w = _tiny_workload("coverage", n_ctx=96, chunk_size=8, tau=0.2, keep_last=1)
    src = _Src(w, rng)
    res = ref.decode_step(w, src)
    G = w.n_q_heads // w.n_kv_heads
    for b in range(w.batch):
        rows = [np.array([math.fsum((src.q[b, h] * k).tolist()) for k in src.Kg[b, h // G]]) for h in range(w.n_q_heads)]
        k = _brute_coverage(rows, w.select_scale, w.tau)
        for g in range(w.n_kv_heads):
            r = res["sel"][(b, g)]
            for j in range(G):
                h = g * G + j
                assert r["heads"][h].tolist() == _brute_topk(rows[h], k), (b, h)


class _TokenView:
    """The same caches, with query token t's rows of every sequence as a one-token step."""

    def __init__(self, src, t, Hq):
        self.__dict__.update({k: v for k, v in src.__dict__.items() if k != "q"})
        self.q = src.q[:, t * Hq:(t + 1) * Hq]
        self._src = src

    def kv_rows(self, bk, g, rows):
        return self._src.kv_rows(bk, g, rows)


def pin_multi_query(ref, seed=11):
    """T adjacent query tokens per sequence: each token's rows select exactly what the same
    queries select in a one-token step; the group union is the union over the tokens'
    one-token unions; every (token, head) output is dense attention masked to that union
    (torch SDPA, fp64)."""
    rng = np.random.default_rng(seed)
    for w in (_tiny_workload("topk", n_queries=3, keep_last=1), _tiny_workload("topp", n_queries=2, top_p=0.7),
              _tiny_workload("hier", n_queries=2),
              _tiny_workload("proxy", n_queries=3, chunk_size=1, top_p=0.6, attend_summary=False)):
        T, Hq, G = w.n_queries, w.n_q_heads, w.n_q_heads // w.n_kv_heads
        w1 = SimpleNamespace(**{**vars(w), "n_queries": 1})
        src = _Src(w, rng)
        res = ref.decode_step(w, src)
        views = [_TokenView(src, t, Hq) for t in range(T)]
        for (b, g), r in res["sel"].items():
            singles = [ref.select_group(w1, views[t], b, g) for t in range(T)]
            assert r["union"].tolist() == ref.group_union([x["union"] for x in singles]).tolist(), (w.mode, b, g)
            for t in range(T):
                for j in range(G):
                    h = g * G + j
                    assert r["heads"][t * Hq + h].tolist() == singles[t]["heads"][h].tolist(), (w.mode, b, t, h)
            U = r["union"]
            rows = (U[:, None] * w.chunk_size + np.arange(w.chunk_size)).ravel()
            mask, Kc, Vc = rows, src.K[b, g], src.V[b, g]
            if w.attend_summary and w.mode != "proxy":
                Kc, Vc = np.concatenate([Kc, src.Kg[b, g]]), np.concatenate([Vc, src.Vg[b, g]])
                mask = np.concatenate([rows, w.n_ctx + U])
            qi = [t * Hq + g * G + j for t in range(T) for j in range(G)]
            o2, l2 = _sdpa(src.q[b, qi], Kc, Vc, w.softmax_scale, mask=mask)
            assert np.allclose(res["out"][b, qi], o2, rtol=1e-11, atol=1e-11), w.mode
            assert np.allclose(res["lse"][b, qi], l2, rtol=1e-11, atol=1e-11), w.mode


class _CutSrc:
    """The same caches cut to their first n tokens (n // chunk_size summary rows)."""

    def __init__(self, src, n, chunk):
        m = n // chunk
        self.q, self.P = src.q, src.P
        self.K, self.V, self.Kp = src.K[:, :, :n], src.V[:, :, :n], src.Kp[:, :, :n]
        self.Kg, self.Vg = src.Kg[:, :, :m], src.Vg[:, :, :m]
        self.Kmg = src.Kmg

    def kv_rows(self, bk, g, rows):
        return self.K[bk, g][rows], self.V[bk, g][rows]


def pin_growing_cache(ref, seed=12):
    """Caches holding n_b tokens of a larger capacity (a growing cache): (1) when n_b is whole
    chunks, every selection and output equals the oracle on the caches cut to n_b tokens (forced
    chunks and local windows follow n_b; nothing past it is read); (2) with everything selected
    (k = all, p = 1) a step is dense attention (torch SDPA, fp64) over the n_b raw tokens plus the
    complete chunks' summaries, the incomplete last chunk's tokens included without a summary; a
    cache with no complete chunk attends its tokens alone, and an empty one gives o = 0, lse = -inf;
    (3) a sparse step is dense attention masked to the union's chunk rows, the incomplete chunk's
    tokens and the union's summaries (per-head masks: the head's own set, the forced chunks and the
    incomplete chunk's tokens)."""
    rng = np.random.default_rng(seed)
    # (1) whole chunks: the oracle on the cut caches
    for w in (_tiny_workload("topk", keep_first=1, keep_last=2), _tiny_workload("topp", top_p=0.7, keep_last=1),
              _tiny_workload("coverage", tau=0.3),
              _tiny_workload("proxy", chunk_size=1, top_p=0.6, attend_summary=False, local_kv_heads=(1,),
                             sink=3, window=9)):
        src = _Src(w, rng)
        ctx = [64, 80] if w.chunk_size > 1 else [41, 77]
        res = ref.decode_step(w, src, ctx_len=ctx)
        for b in range(w.batch):
            wc = SimpleNamespace(**{**vars(w), "n_ctx": ctx[b]})
            cut = ref.decode_step(wc, _CutSrc(src, ctx[b], w.chunk_size), groups=[(b, g) for g in range(w.n_kv_heads)])
            for g in range(w.n_kv_heads):
                r, rc = res["sel"][(b, g)], cut["sel"][(b, g)]
                assert r["union"].tolist() == rc["union"].tolist(), (w.mode, b, g)
                for h in r["heads"]:
                    assert r["heads"][h].tolist() == rc["heads"][h].tolist(), (w.mode, b, h)
            assert np.array_equal(res["out"][b], cut["out"][b]) and np.array_equal(res["lse"][b], cut["lse"][b]), w.mode
    # (2) everything selected: dense attention over the valid tokens and complete summaries
    for w, ctx in ((_tiny_workload("topk", top_k=50), [83, 61]), (_tiny_workload("topp", top_p=1.0), [5, 8]),
                   (_tiny_workload("topk", top_k=50), [0, 17]),
                   (_tiny_workload("proxy", chunk_size=1, top_p=1.0, attend_summary=False, local_kv_heads=(1,),
                                   sink=4, window=11), [50, 93])):
        src = _Src(w, rng)
        res = ref.decode_step(w, src, ctx_len=ctx)
        G = w.n_q_heads // w.n_kv_heads
        for b in range(w.batch):
            n, m = ctx[b], ctx[b] // w.chunk_size
            for g in range(w.n_kv_heads):
                qs = slice(g * G, (g + 1) * G)
                if n == 0:
                    assert np.all(res["out"][b, qs] == 0.0) and np.all(res["lse"][b, qs] == -np.inf)
                    continue
                if g in w.local_kv_heads:
                    rows = np.union1d(np.arange(min(w.sink, n)), np.arange(max(0, n - w.window), n))
                    Kc, Vc = src.K[b, g][rows], src.V[b, g][rows]
                elif w.attend_summary and w.mode != "proxy":
                    Kc = np.concatenate([src.K[b, g][:n], src.Kg[b, g][:m]])
                    Vc = np.concatenate([src.V[b, g][:n], src.Vg[b, g][:m]])
                else:
                    Kc, Vc = src.K[b, g][:n], src.V[b, g][:n]
                o2, l2 = _sdpa(src.q[b, qs], Kc, Vc, w.softmax_scale)
                assert np.allclose(res["out"][b, qs], o2, rtol=1e-11, atol=1e-11), (w.mode, b, g)
                assert np.allclose(res["lse"][b, qs], l2, rtol=1e-11, atol=1e-11), (w.mode, b, g)
    # (3) sparse steps with an incomplete last chunk: masked dense attention
    for w, ctx in ((_tiny_workload("topp", top_p=0.7, keep_last=1), [83, 45]),
                   (_tiny_workload("topk", top_k=2, keep_first=1, head_masks=True), [70, 91])):
        src = _Src(w, rng)
        res = ref.decode_step(w, src, ctx_len=ctx)
        G = w.n_q_heads // w.n_kv_heads
        for (b, g), r in res["sel"].items():
            n, m = ctx[b], ctx[b] // w.chunk_size
            assert all(int(e) < m for e in r["union"]), "selected past the complete chunks"
            forced = [e for e in range(m) if e < w.keep_first or e >= m - w.keep_last]
            Kc = np.concatenate([src.K[b, g], src.Kg[b, g]])
            Vc = np.concatenate([src.V[b, g], src.Vg[b, g]])
            for j in range(G):
                h = g * G + j
                chunks = sorted(set(r["heads"][h].tolist()) | set(forced)) if w.head_masks else r["union"].tolist()
                mask = [c * w.chunk_size + t for c in chunks for t in range(w.chunk_size)]
                mask += list(range(m * w.chunk_size, n)) + [w.n_ctx + c for c in chunks]
                o2, l2 = _sdpa(src.q[b, h][None], Kc, Vc, w.softmax_scale, mask=np.array(mask))
                assert np.allclose(res["out"][b, h], o2[0], rtol=1e-11, atol=1e-11), (w.mode, b, h)
                assert np.allclose(res["lse"][b, h], l2[0], rtol=1e-11, atol=1e-11), (w.mode, b, h)


ALL_PINS = [pin_golden_scores, pin_golden_proxy, pin_golden_topk, pin_golden_topp, pin_golden_two_level,
            pin_golden_union, pin_golden_attention, pin_scores_exact, pin_bruteforce, pin_topp_minimal,
            pin_reductions, pin_union, pin_masked_dense, pin_dense_limits, pin_step_masked,
            pin_step_selection, pin_variants, pin_coverage, pin_multi_query, pin_growing_cache]
