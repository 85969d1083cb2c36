"""Pins of the Token-Sparse prefill oracle against what the page and the mathematics fix.

Each pin takes the oracle module as an argument, so a mutated copy can be checked too.
References are library routines in fp64 (torch softmax / SDPA), exact rational arithmetic, or
brute force over all subsets, never a retyping of the oracle's own loops.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import torch


def _workload(**kw):
    base = dict(name="pin", batch=2, n_q_heads=4, n_kv_heads=2, head_dim=16, seq_len=40, window=6, tau=0.3,
                softmax_scale=0.25)
    base.update(kw)
    return SimpleNamespace(**base)


class _Src:
    def __init__(self, w, rng, scale=1.0):
        B, Hq, Hk, d, L = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.seq_len
        self.Q = rng.standard_normal((B, Hq, L, d)) * scale
        self.K = rng.standard_normal((B, Hk, L, d)) * scale
        self.V = rng.standard_normal((B, Hk, L, d))

    def q_rows(self, b, h, rows):
        return self.Q[b, h][np.asarray(rows, dtype=np.int64)]

    def k_all(self, b, g):
        return self.K[b, g]

    def kv_rows(self, b, g, rows):
        rows = np.asarray(rows, dtype=np.int64)
        return self.K[b, g][rows], self.V[b, g][rows]


def _torch_importance(Qw, K, scale, pos0):
    q, k = torch.from_numpy(Qw), torch.from_numpy(K)
    logits = scale * (q @ k.T)
    W, L = logits.shape
    mask = torch.arange(L)[None, :] > (pos0 + torch.arange(W))[:, None]
    a = torch.softmax(logits.masked_fill(mask, -math.inf), dim=1)
    return a.sum(dim=0).numpy()


def pin_importance_library(pref, seed=20):
    """Importance equals the column sums of torch's fp64 causal softmax map."""
    rng = np.random.default_rng(seed)
    for t in range(10):
        L, W, d = int(rng.integers(8, 200)), int(rng.integers(1, 9)), int(rng.choice([4, 16]))
        W = min(W, L)
        Qw, K = rng.standard_normal((W, d)) * 2, rng.standard_normal((L, d))
        scale = float(rng.choice([0.1, 0.5, 1.0]))
        imp = pref.proxy_importance(Qw, K, scale, L - W)
        ref = _torch_importance(Qw, K, scale, L - W)
        assert np.allclose(imp, ref, rtol=1e-12, atol=1e-14), t


def pin_importance_invariants(pref, seed=21):
    """Every window row is a distribution: the importance sums to W; key j >= L - W is seen only by
    rows i >= j - (L - W); a single-row window is the textbook softmax of the last query."""
    rng = np.random.default_rng(seed)
    for t in range(10):
        L, W, d = int(rng.integers(10, 100)), int(rng.integers(1, 8)), 8
        Qw, K = rng.standard_normal((W, d)), rng.standard_normal((L, d))
        imp = pref.proxy_importance(Qw, K, 0.5, L - W)
        assert abs(imp.sum() - W) < 1e-12 and np.all(imp >= 0)
        # the last key is seen by the last row only
        q, k = torch.from_numpy(Qw[-1]), torch.from_numpy(K)
        p_last = torch.softmax(0.5 * (k @ q), dim=0).numpy()
        assert abs(imp[-1] - p_last[-1]) < 1e-14
        one = pref.proxy_importance(Qw[-1:], K, 0.5, L - 1)
        assert np.allclose(one, p_last, rtol=1e-12, atol=1e-15)


def _brute_budget(total, tau):
    """Shortest ascending prefix whose exact mass exceeds tau x total (all orders of equal values
    give the same masses); budget = max(1, L - removed)."""
    vals = [Fraction(float(x)) for x in total]
    T = sum(vals)
    thr = Fraction(tau) * T
    asc = sorted(vals)
    c = Fraction(0)
    removed = len(vals)
    for r, v in enumerate(asc, start=1):
        c += v
        if c > thr:
            removed = r
            break
    return max(1, len(vals) - removed)


def _brute_topk(s, k):
    """Among all k-subsets, the one of maximum exact sum; ties: lexicographically smallest."""
    best, best_key = None, None
    for comb in itertools.combinations(range(len(s)), k):
        key = (sum(Fraction(float(s[i])) for i in comb), [-i for i in comb])
        if best_key is None or key > best_key:
            best, best_key = comb, key
    return list(best)


def pin_select_bruteforce(pref, seed=22):
    """On tiny prompts the global budget equals the exact-arithmetic coverage cut of the heads'
    summed importance, and every head's set is its brute-force top-budget subset."""
    rng = np.random.default_rng(seed)
    for t in range(6):
        w = _workload(seq_len=int(rng.integers(6, 12)), window=3, tau=float(rng.uniform(0.05, 0.7)),
                      n_q_heads=4, n_kv_heads=2, head_dim=4)
        src = _Src(w, rng, scale=1.5)
        for b in range(w.batch):
            r = pref.tsa_select(w, src, b)
            total = sum(_torch_importance(src.Q[b, h, w.seq_len - w.window:], src.K[b, h // 2], w.softmax_scale,
                                          w.seq_len - w.window) for h in range(w.n_q_heads))
            k = _brute_budget(total, w.tau)
            assert r["budget"] == k, (t, b, r["budget"], k)
            for h in range(w.n_q_heads):
                assert r["sets"][h].tolist() == _brute_topk(r["importance"][h], k), (t, b, h)


def _sdpa_masked(q, K, V, scale, allowed):
    qt = torch.from_numpy(q)[None, None]                 # [1, 1, n, d]
    kt = torch.from_numpy(K)[None, None]
    vt = torch.from_numpy(V)[None, None]
    am = torch.where(torch.from_numpy(allowed), 0.0, -math.inf).to(torch.float64)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=scale)[0, 0].numpy()


def pin_attention_masked_dense(pref, seed=23):
    """The scattered output equals dense attention over the whole prompt with a mask keeping, for
    query position p in S_h, the keys in S_h at positions <= p (torch SDPA, fp64); every other
    position of the head is zero."""
    rng = np.random.default_rng(seed)
    w = _workload(seq_len=48, window=5, tau=0.4)
    src = _Src(w, rng)
    res = pref.tsa_prefill(w, src)
    G = w.n_q_heads // w.n_kv_heads
    for b in range(w.batch):
        for h in range(w.n_q_heads):
            S = res["sel"][b]["sets"][h]
            O = res["out"][b, h]
            keep = np.zeros(w.seq_len, dtype=bool)
            keep[S] = True
            assert np.all(O[~keep] == 0.0)
            allowed = keep[None, :] & (np.arange(w.seq_len)[None, :] <= S[:, None])
            ref = _sdpa_masked(src.Q[b, h][S], src.K[b, h // G], src.V[b, h // G], w.softmax_scale, allowed)
            assert np.allclose(O[S], ref, rtol=1e-11, atol=1e-12), (b, h)


def pin_attention_dense_limit(pref, seed=24):
    """Keeping every position reduces the compressed attention to textbook causal attention."""
    rng = np.random.default_rng(seed)
    w = _workload(seq_len=30)
    src = _Src(w, rng)
    S = np.arange(w.seq_len)
    for h in range(w.n_q_heads):
        o, _ = pref.tsa_attend_rows(w, src, 0, h, S, list(range(w.seq_len)))
        g = h // (w.n_q_heads // w.n_kv_heads)
        q = torch.from_numpy(src.Q[0, h])[None, None]
        k = torch.from_numpy(src.K[0, g])[None, None]
        v = torch.from_numpy(src.V[0, g])[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.softmax_scale)[0, 0]
        assert np.allclose(o, ref.numpy(), rtol=1e-11, atol=1e-12), h


def pin_mixed_heads(pref, seed=25):
    """Head-wise full / sparse routing: the budget is the exact coverage cut of the sparse heads'
    summed importance only, every sparse head keeps its brute-force top-budget subset, and a full
    head keeps every position."""
    rng = np.random.default_rng(seed)
    for t, modes in enumerate([(1, 0, 0, 1), (0, 1, 1, 1), (1, 1, 0, 0)]):
        w = _workload(seq_len=int(rng.integers(6, 12)), window=3, tau=float(rng.uniform(0.05, 0.7)),
                      n_q_heads=4, n_kv_heads=2, head_dim=4, head_mode=modes)
        src = _Src(w, rng, scale=1.5)
        for b in range(w.batch):
            r = pref.tsa_select(w, src, b)
            total = sum(_torch_importance(src.Q[b, h, w.seq_len - w.window:], src.K[b, h // 2], w.softmax_scale,
                                          w.seq_len - w.window) for h in range(w.n_q_heads) if not modes[h])
            k = _brute_budget(total, w.tau)
            assert r["budget"] == k, (t, b, r["budget"], k)
            for h in range(w.n_q_heads):
                want = list(range(w.seq_len)) if modes[h] else _brute_topk(r["importance"][h], k)
                assert r["sets"][h].tolist() == want, (t, b, h)


def pin_full_heads_textbook(pref, seed=26):
    """Every head routed to full attention: the layer is textbook causal attention (torch SDPA,
    fp64) for every head."""
    rng = np.random.default_rng(seed)
    w = _workload(seq_len=33, window=4, head_mode=(1, 1, 1, 1))
    src = _Src(w, rng)
    res = pref.tsa_prefill(w, src)
    G = w.n_q_heads // w.n_kv_heads
    for b in range(w.batch):
        for h in range(w.n_q_heads):
            q = torch.from_numpy(src.Q[b, h])[None, None]
            k = torch.from_numpy(src.K[b, h // G])[None, None]
            v = torch.from_numpy(src.V[b, h // G])[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.softmax_scale)
            assert np.allclose(res["out"][b, h], ref[0, 0].numpy(), rtol=1e-11, atol=1e-12), (b, h)


PREFILL_PINS = [pin_importance_library, pin_importance_invariants, pin_select_bruteforce,
                pin_attention_masked_dense, pin_attention_dense_limit, pin_mixed_heads, pin_full_heads_textbook]
