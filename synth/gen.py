"""Seeded synthetic decode inputs, identical on CPU and GPU.

Every random value comes from a counter-based generator: element ``i`` of the
array tagged ``tag`` under seed ``seed`` takes the 16-bit code
``lowbias32(lowbias32((i mod 2^32) ^ k1) ^ (i >> 32) ^ k2) >> 16`` (two rounds of
the lowbias32 integer finaliser published by C. Wellons in the hash-prospector
project, keys derived from seed and tag) and becomes
``table[code]``, where ``table[c]`` is the standard normal quantile at
``(c + 0.5) / 65536`` rounded once (round-to-nearest-even) to the array's dtype.
The draws are therefore i.i.d. N(0,1) at 16-bit resolution (|x| <= 4.33).
All integer work is done in int64 with products kept below 2^49, so CPU and GPU
produce the same bits, and any subset of rows can be drawn on its own.

Structured workloads add deterministic plants on the summary keys (arithmetic of
the generator, not of the method):

* ``gist_align``: per (sequence, KV group) ``plants_per_head`` distinct seeded
  chunks per query head get summary key ``3 * q_h / |q_h|``.
* ``zipf``: per (sequence, KV group) a seeded permutation ``pi`` gives target
  logits ``l_m = -s * ln(pi_m + 1)`` (centred); summary key
  ``z_perp + sqrt(d) * l_m * w`` with ``w = Q^T (Q Q^T)^-1 1`` over the group's
  queries ``Q`` and ``z_perp`` a normal vector with span(Q) projected out, so every
  head of the group sees a Zipf(s) chunk-mass profile.
* ``needles``: per KV group, 4 query heads x ``plants_per_head`` distinct seeded
  segments, one seeded chunk inside each; that chunk's summary key and its
  segment's meta-summary key are set to ``3 * q_h / |q_h|``.
* proxy keys: ``Kp = fp16(K @ P)`` with ``P`` an N(0,1) d x r matrix per KV head,
  summed in fp64 in index order with separate multiply and add.

Prefill inputs (``make_prefill_inputs``): Q [B][Hq][L][d], K and V [B][Hkv][L][d],
N(0,1) as above; per (sequence, KV group) a unit direction ``u_g`` (normal draw,
normalised) is added as ``beta * u_g`` to every query of the group and as
``gamma_j * u_g`` to key j, with ``gamma_j = sqrt(d) * l_j / beta`` and ``l_j`` the
centred Zipf(s) logit profile of a seeded permutation, so each head's attention
mass over the keys is Zipf-like. The plant is added in fp64 and rounded once to
bf16 on the device that generates the inputs; the oracle reads those tensors.

No function here computes anything the decode or prefill path computes.
"""
from __future__ import annotations

import math
from functools import lru_cache

import numpy as np
import torch

from .configs import HIER, PROXY_TOPP, PrefillWorkload, Workload

_M32 = 0xFFFFFFFF

# array tags
T_Q, T_K, T_V, T_KG, T_VG, T_KMG, T_P = 1, 2, 3, 4, 5, 6, 7
T_PERM, T_OFF, T_Z = 8, 9, 10
T_PQ, T_PK, T_PV, T_PU, T_PPERM = 11, 12, 13, 14, 15  # prefill
T_GQ, T_GK, T_GV, T_GQG, T_GKG, T_GVG = 16, 17, 18, 19, 20, 21  # gist-masked prefill

_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "f64": torch.float64}


def _lowbias32_int(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & _M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & _M32
    x ^= x >> 16
    return x


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for int64 x in [0, 2^32) without leaving int64 range."""
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & _M32


def _lowbias32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _keys(seed: int, tag: int) -> tuple[int, int]:
    k1 = _lowbias32_int(seed * 0x9E3779B1 + tag * 0x85EBCA77 + 0x27D4EB2F)
    k2 = _lowbias32_int(k1 ^ 0x68E31DA4)
    return k1, k2


def hash32(seed: int, tag: int, idx: torch.Tensor) -> torch.Tensor:
    """32-bit hash of int64 counters ``idx`` (int64 result in [0, 2^32))."""
    k1, k2 = _keys(seed, tag)
    x = _lowbias32((idx & _M32) ^ k1)
    x = _lowbias32(x ^ ((idx >> 32) ^ k2))
    return x


def codes(seed: int, tag: int, idx: torch.Tensor) -> torch.Tensor:
    return hash32(seed, tag, idx) >> 16


@lru_cache(maxsize=None)
def _table_cpu(dtype: str) -> torch.Tensor:
    from scipy.special import ndtri
    u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return torch.from_numpy(ndtri(u)).to(_DT[dtype])


def table(dtype: str, device) -> torch.Tensor:
    return _table_cpu(dtype).to(device)


def normal_at(seed: int, tag: int, flat_idx: torch.Tensor, dtype: str) -> torch.Tensor:
    """Values at the given flat element indices (any shape, any device)."""
    tab = table(dtype, flat_idx.device)
    return tab[codes(seed, tag, flat_idx)]


def normal(shape, seed: int, tag: int, dtype: str, device="cpu", block: int = 1 << 25) -> torch.Tensor:
    n = math.prod(shape)
    out = torch.empty(n, dtype=_DT[dtype], device=device)
    tab = table(dtype, device)
    for s in range(0, n, block):
        e = min(n, s + block)
        idx = torch.arange(s, e, dtype=torch.int64, device=device)
        out[s:e] = tab[codes(seed, tag, idx)]
    return out.view(*shape)


def rows_at(shape, seed: int, tag: int, dtype: str, b: int, h: int, rows: torch.Tensor) -> torch.Tensor:
    """Rows ``[b, h, rows, :]`` of a 4-D [B][H][N][d] array drawn by :func:`normal`."""
    _, H, N, d = shape
    rows = rows.to(torch.int64)
    flat = ((b * H + h) * N + rows)[:, None] * d + torch.arange(d, dtype=torch.int64, device=rows.device)[None, :]
    return normal_at(seed, tag, flat, dtype)


def permutation(seed: int, tag: int, salt: int, n: int) -> torch.Tensor:
    """Seeded permutation of range(n): indices sorted by a per-index hash (stable)."""
    idx = torch.arange(n, dtype=torch.int64) + (salt << 32)
    h = hash32(seed, tag, idx)
    return torch.sort(h, stable=True).indices


def _unit3(qh: torch.Tensor) -> torch.Tensor:
    q64 = qh.double()
    return 3.0 * q64 / torch.sqrt(torch.sum(q64 * q64))


def proxy_keys(K: torch.Tensor, P: torch.Tensor, block: int = 1 << 20) -> torch.Tensor:
    """fp16(K @ P) per KV head, fp64 sums in index order, separate mul and add."""
    Bk, H, N, d = K.shape
    r = P.shape[-1]
    out = torch.empty(Bk, H, N, r, dtype=torch.float16, device=K.device)
    P64 = P.double()
    for b in range(Bk):
        for h in range(H):
            for s in range(0, N, block):
                e = min(N, s + block)
                Kb = K[b, h, s:e].double()
                acc = torch.zeros(e - s, r, dtype=torch.float64, device=K.device)
                for i in range(d):
                    prod = Kb[:, i:i + 1] * P64[h, i][None, :]
                    acc = acc + prod
                out[b, h, s:e] = acc.to(torch.float16)
    return out


def make_inputs(w: Workload, device="cpu", seed: int | None = None) -> dict:
    """All inputs of one decode step of workload ``w`` as tensors on ``device``."""
    seed = w.seed if seed is None else seed
    dt = w.dtype
    B, Bk, Hq, Hk, d, N = w.batch, w.kv_batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx
    G, M = w.group, w.n_chunks
    out = {"workload": w, "seed": seed}
    T = w.n_queries
    # q [B][Hq][d], or [B][T][Hq][d] for T adjacent query tokens per sequence
    out["q"] = normal((B, Hq, d) if T == 1 else (B, T, Hq, d), seed, T_Q, dt, device)
    out["K"] = normal((Bk, Hk, N, d), seed, T_K, dt, device)
    out["V"] = normal((Bk, Hk, N, d), seed, T_V, dt, device)
    mode = torch.zeros(Hk, dtype=torch.int8)
    for g in w.local_kv_heads:
        mode[g] = 1
    out["head_mode"] = mode.to(device)

    if w.mode == PROXY_TOPP:
        r = w.route_dim
        P = normal((Hk, d, r), seed, T_P, "f32", "cpu")
        out["P"] = P.to(device)
        out["Kp"] = proxy_keys(out["K"], out["P"])
        return out

    # summary (gist / landmark) keys and values: built on the host, small
    Kg = normal((Bk, Hk, M, d), seed, T_KG, dt, "cpu")
    Vg = normal((Bk, Hk, M, d), seed, T_VG, dt, "cpu")
    # per sequence, every query row [T * Hq][d], row t * Hq + h; head plants use token 0
    qc = out["q"].to("cpu").reshape(B, T * Hq, d)
    if w.plant == "gist_align":
        n_p = w.plants_per_head
        for b in range(Bk):
            for g in range(Hk):
                perm = permutation(seed, T_PERM, b * Hk + g, M)
                for j in range(G):
                    vec = _unit3(qc[b, g * G + j]).to(Kg.dtype)
                    for m in perm[j * n_p:(j + 1) * n_p].tolist():
                        Kg[b, g, m] = vec
    elif w.plant == "zipf":
        z = normal((Bk, Hk, M, d), seed, T_Z, "f64", "cpu")
        for b in range(Bk):
            for g in range(Hk):
                pi = torch.empty(M, dtype=torch.float64)
                pi[permutation(seed, T_PERM, b * Hk + g, M)] = torch.arange(M, dtype=torch.float64)
                ell = -w.zipf_s * torch.log(pi + 1.0)
                ell = ell - ell.mean()
                # the group's T x G query rows
                Q = torch.stack([qc[b, t * Hq + g * G + j] for t in range(T) for j in range(G)]).double()
                gram = Q @ Q.T
                wv = Q.T @ torch.linalg.solve(gram, torch.ones(Q.shape[0], dtype=torch.float64))
                zg = z[b, g]
                zperp = zg - (Q.T @ torch.linalg.solve(gram, Q @ zg.T)).T
                Kg[b, g] = (zperp + math.sqrt(d) * ell[:, None] * wv[None, :]).to(Kg.dtype)
    if w.mode == HIER:
        S, sg = w.n_segments, w.seg_size
        Kmg = normal((Bk, Hk, S, d), seed, T_KMG, dt, "cpu")
        n_p = w.plants_per_head
        for b in range(Bk):
            for g in range(Hk):
                segs = permutation(seed, T_PERM, b * Hk + g, S)[:G * n_p].tolist()
                offs = (codes(seed, T_OFF, torch.arange(G * n_p, dtype=torch.int64)
                              + ((b * Hk + g) << 32)) % sg).tolist()
                for j in range(G):
                    vec = _unit3(qc[b, g * G + j]).to(Kg.dtype)
                    for t in range(j * n_p, (j + 1) * n_p):
                        Kmg[b, g, segs[t]] = vec
                        Kg[b, g, segs[t] * sg + offs[t]] = vec
        out["Kmg"] = Kmg.to(device)
    out["Kg"] = Kg.to(device)
    out["Vg"] = Vg.to(device)
    return out


def make_prefill_inputs(w: PrefillWorkload, device="cpu", seed: int | None = None) -> dict:
    """Q, K, V of one prefill step of workload ``w`` as tensors on ``device``."""
    seed = w.seed if seed is None else seed
    B, Hq, Hk, d, L, G = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.seq_len, w.group
    dt = _DT[w.dtype]
    U = normal((B, Hk, d), seed, T_PU, "f64", "cpu")
    U = U / torch.sqrt((U * U).sum(dim=-1, keepdim=True))
    Q = torch.empty((B, Hq, L, d), dtype=dt, device=device)
    K = torch.empty((B, Hk, L, d), dtype=dt, device=device)
    V = normal((B, Hk, L, d), seed, T_PV, w.dtype, device)
    for b in range(B):
        for g in range(Hk):
            u = U[b, g].to(device)
            for j in range(G):
                h = g * G + j
                flat = torch.arange((b * Hq + h) * L * d, (b * Hq + h + 1) * L * d, dtype=torch.int64, device=device)
                z = normal_at(seed, T_PQ, flat, "f64").view(L, d)
                Q[b, h] = (z + w.beta * u[None, :]).to(dt)
            pi = torch.empty(L, dtype=torch.float64)
            pi[permutation(seed, T_PPERM, b * Hk + g, L)] = torch.arange(L, dtype=torch.float64)
            ell = -w.zipf_s * torch.log(pi + 1.0)
            gamma = ((ell - ell.mean()) * math.sqrt(d) / w.beta).to(device)
            flat = torch.arange((b * Hk + g) * L * d, (b * Hk + g + 1) * L * d, dtype=torch.int64, device=device)
            z = normal_at(seed, T_PK, flat, "f64").view(L, d)
            K[b, g] = (z + gamma[:, None] * u[None, :]).to(dt)
    return {"workload": w, "seed": seed, "Q": Q, "K": K, "V": V}


def make_gist_inputs(w, device="cpu", seed: int | None = None) -> dict:
    """Raw Q [B][Hq][N][d], K, V [B][Hkv][N][d] and gist Qg [B][Hq][M][d], Kg, Vg [B][Hkv][M][d] of one
    gist-masked prefill step of workload ``w``: independent N(0, 1) entries rounded to the dtype (the
    attention's cost does not depend on the values; the parity tests check every visible key)."""
    seed = w.seed if seed is None else seed
    B, Hq, Hk, d, N, C = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_tokens, w.chunk_size
    M = N // C
    out = {"workload": w, "seed": seed}
    for name, tag, shape in (("Q", T_GQ, (B, Hq, N, d)), ("K", T_GK, (B, Hk, N, d)), ("V", T_GV, (B, Hk, N, d)),
                             ("Qg", T_GQG, (B, Hq, M, d)), ("Kg", T_GKG, (B, Hk, M, d)),
                             ("Vg", T_GVG, (B, Hk, M, d))):
        out[name] = normal(shape, seed, tag, w.dtype, device)
    return out
