"""Pins of the gist-masked (SSA) prefill oracle against what the page and the mathematics fix.

Each pin takes the oracle module as an argument, so a mutated copy can be checked too. References
are torch's fp64 scaled-dot-product attention on the interleaved sequence with the mask written in
interleaved positions (a formulation independent of the oracle's permuted key segments), the
textbook causal attention it reduces to, and a hand-derived fixture of visible key sets.
"""
from __future__ import annotations

import json
import math
import os
from types import SimpleNamespace

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _workload(**kw):
    base = dict(name="pin", batch=2, n_q_heads=4, n_kv_heads=2, head_dim=16, n_tokens=20, chunk_size=4,
                softmax_scale=0.3)
    base.update(kw)
    return SimpleNamespace(**base)


class _Src:
    def __init__(self, w, rng, zero_keys=False, onehot_values=False):
        B, Hq, Hk, d, N, C = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_tokens, w.chunk_size
        M = N // C
        self.Q = rng.standard_normal((B, Hq, N, d))
        self.Qg = rng.standard_normal((B, Hq, M, d))
        self.K = np.zeros((B, Hk, N, d)) if zero_keys else rng.standard_normal((B, Hk, N, d))
        self.Kg = np.zeros((B, Hk, M, d)) if zero_keys else rng.standard_normal((B, Hk, M, d))
        if onehot_values:  # gist key j -> e_j, raw key t -> e_(M + t)
            eye = np.eye(d)
            self.Vg = np.broadcast_to(eye[:M], (B, Hk, M, d)).copy()
            self.V = np.broadcast_to(eye[M:M + N], (B, Hk, N, d)).copy()
        else:
            self.V = rng.standard_normal((B, Hk, N, d))
            self.Vg = rng.standard_normal((B, Hk, M, d))

    def q_row(self, b, h, kind, i):
        return (self.Q if kind == "raw" else self.Qg)[b, h, i]

    def raw_kv_rows(self, b, g, rows):
        rows = np.asarray(rows, dtype=np.int64)
        return self.K[b, g][rows], self.V[b, g][rows]

    def gist_kv_rows(self, b, g, rows):
        rows = np.asarray(rows, dtype=np.int64)
        return self.Kg[b, g][rows], self.Vg[b, g][rows]


def _interleaved_sdpa(w, src, b, h):
    """Dense attention over the interleaved sequence (gist m after chunk m) with the mask: causal,
    and a raw key visible only inside its own chunk. Returns (O raw [N][d], O gist [M][d])."""
    N, C = w.n_tokens, w.chunk_size
    M = N // C
    g = h // (w.n_q_heads // w.n_kv_heads)
    P = N + M
    pos = np.arange(P)
    chunk = pos // (C + 1)
    is_gist = pos % (C + 1) == C
    idx = np.where(is_gist, chunk, chunk * C + pos % (C + 1))
    Q = np.where(is_gist[:, None], src.Qg[b, h][np.minimum(idx, M - 1)], src.Q[b, h][np.minimum(idx, N - 1)])
    K = np.where(is_gist[:, None], src.Kg[b, g][np.minimum(idx, M - 1)], src.K[b, g][np.minimum(idx, N - 1)])
    V = np.where(is_gist[:, None], src.Vg[b, g][np.minimum(idx, M - 1)], src.V[b, g][np.minimum(idx, N - 1)])
    allowed = (pos[None, :] <= pos[:, None]) & (is_gist[None, :] | (chunk[None, :] == chunk[:, None]))
    am = torch.where(torch.from_numpy(allowed), 0.0, -math.inf).to(torch.float64)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q)[None, None], torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None],
        attn_mask=am, scale=w.softmax_scale)[0, 0].numpy()
    return out[~is_gist][np.argsort(idx[~is_gist])], out[is_gist][np.argsort(idx[is_gist])]


def pin_interleaved_sdpa(gref, seed=40):
    """Raw and gist outputs equal dense fp64 attention over the interleaved sequence with the gist
    causal mask, for several chunk sizes (1 included) and chunk counts."""
    rng = np.random.default_rng(seed)
    for C, M in [(4, 5), (1, 6), (3, 4), (5, 1)]:
        w = _workload(chunk_size=C, n_tokens=C * M)
        src = _Src(w, rng)
        r = gref.gist_prefill(w, src)
        for b in range(w.batch):
            for h in range(w.n_q_heads):
                o_raw, o_gist = _interleaved_sdpa(w, src, b, h)
                assert np.allclose(r["out"][b, h], o_raw, rtol=1e-11, atol=1e-12), (C, M, b, h)
                assert np.allclose(r["out_gist"][b, h], o_gist, rtol=1e-11, atol=1e-12), (C, M, b, h)


def pin_single_chunk_textbook(gref, seed=41):
    """One chunk: the raw tokens run textbook causal attention among themselves, and the gist
    attends to every raw token and itself without a mask."""
    rng = np.random.default_rng(seed)
    w = _workload(chunk_size=12, n_tokens=12)
    src = _Src(w, rng)
    r = gref.gist_prefill(w, src)
    G = w.n_q_heads // w.n_kv_heads
    for b in range(w.batch):
        for h in range(w.n_q_heads):
            g = h // G
            q, k, v = (torch.from_numpy(x)[None, None] for x in (src.Q[b, h], src.K[b, g], src.V[b, g]))
            ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.softmax_scale)
            assert np.allclose(r["out"][b, h], ref[0, 0].numpy(), rtol=1e-11, atol=1e-12)
            kk = torch.from_numpy(np.concatenate([src.K[b, g], src.Kg[b, g]]))[None, None]
            vv = torch.from_numpy(np.concatenate([src.V[b, g], src.Vg[b, g]]))[None, None]
            qg = torch.from_numpy(src.Qg[b, h])[None, None]
            refg = torch.nn.functional.scaled_dot_product_attention(qg, kk, vv, scale=w.softmax_scale)
            assert np.allclose(r["out_gist"][b, h], refg[0, 0].numpy(), rtol=1e-11, atol=1e-12)


def pin_visible_sets_fixture(gref, seed=42):
    """With all keys zero every visible key gets the same weight; with one-hot values the output
    row is the indicator of the visible set over its size. The sets must match the hand-derived
    fixture (C = 2, M = 3)."""
    fx = json.load(open(os.path.join(GOLDEN, "gist_mask_c2_m3.json")))
    C, M = fx["chunk_size"], fx["n_chunks"]
    w = _workload(chunk_size=C, n_tokens=C * M, head_dim=16, batch=1, n_q_heads=2, n_kv_heads=1)
    src = _Src(w, np.random.default_rng(seed), zero_keys=True, onehot_values=True)
    r = gref.gist_prefill(w, src)
    for kind, key in (("raw", "out"), ("gist", "out_gist")):
        for e in fx[kind]:
            want = np.zeros(w.head_dim)
            cols = list(e["gists"]) + [M + t for t in e["raws"]]
            want[cols] = 1.0 / len(cols)
            for h in range(w.n_q_heads):
                got = r[key][0, h, e["query"]]
                assert np.allclose(got, want, atol=1e-14), (kind, e, got)


GIST_PINS = [pin_interleaved_sdpa, pin_single_chunk_textbook, pin_visible_sets_fixture]
