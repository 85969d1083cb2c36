"""Named decode workloads: shapes and selection parameters.

Five full-size workloads follow the shapes of the models the pages evaluate on
(Qwen2-7B-style SSA decode, a Llama-3.1-8B-style 128K top-p decode, H-SSA
two-level routing at 512K, and RTPurbo-style mixed heads at 1M tokens), plus a
tiny fp32 case. Each has a reduced twin with the same structure that the fp64
oracle finishes in seconds; the twins span several attention tiles and end on
ragged tails.

This module holds parameters only -- no arithmetic of the method.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

TOPK = "topk"          # per-head top-k over chunk summary scores
TOPP = "topp"          # per-head dynamic top-p over the softmax of chunk scores
HIER = "hier"          # two-level: top-k segments (meta summaries) -> top-k chunks
PROXY_TOPP = "proxy"   # per-token top-p on rank-r proxy-key scores; local heads
COVERAGE = "coverage"  # per-sequence coverage budget (tau), then per-head top-k


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int                 # sequences
    kv_batch: int              # distinct KV caches; 1 = every query reads one cache
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_ctx: int                 # tokens in the cache
    chunk_size: int            # tokens per chunk; 1 = token-level selection
    dtype: str                 # "f32" | "bf16" (q, K, V, summary K/V)
    mode: str
    top_k: int = 0
    top_k_seg: int = 0
    seg_size: int = 0          # summaries per meta-summary (HIER)
    top_p: float = 1.0
    tau: float = 0.0           # coverage threshold (COVERAGE): tail mass cut from the importance
    select_scale: float = 1.0  # logit scale of the top-p softmax
    softmax_scale: float = 1.0
    keep_first: int = 0        # forced leading chunks (attention sink)
    keep_last: int = 0         # forced trailing chunks (most recent)
    route_dim: int = 0         # proxy-key rank (PROXY_TOPP)
    local_kv_heads: tuple = () # KV heads that run sink + sliding window
    sink: int = 0
    window: int = 0
    attend_summary: bool = True
    all_summaries: bool = False  # variant: every chunk's summary K/V joins the context
    head_masks: bool = False     # variant: each head attends to its own selection + forced chunks
    plant: str = ""            # synthetic structure recipe, see synth.gen
    plants_per_head: int = 0
    zipf_s: float = 0.0
    attend_blocks: int = 0     # persistent attention workgroups (0 = library default)
    n_queries: int = 1         # adjacent query tokens per sequence (multi-query decode)
    seed: int = 0

    # derived -------------------------------------------------------------
    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_chunks(self) -> int:
        return self.n_ctx // self.chunk_size

    @property
    def n_segments(self) -> int:
        return self.n_chunks // self.seg_size if self.seg_size else 0

    @property
    def n_entries(self) -> int:
        """Length of the per-group selection domain: chunks, or tokens at chunk_size 1."""
        return self.n_chunks

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _inv_sqrt(d: int) -> float:
    return 1.0 / math.sqrt(d)


C1 = Workload(
    name="c1_tiny_f32", batch=16, kv_batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64,
    n_ctx=2048, chunk_size=64, dtype="f32", mode=TOPK, top_k=4,
    softmax_scale=_inv_sqrt(64), select_scale=_inv_sqrt(64), seed=1)

C2 = Workload(
    name="c2_ssa_qwen2_7b_32k", batch=8, kv_batch=8, n_q_heads=28, n_kv_heads=4, head_dim=128,
    n_ctx=32768, chunk_size=16, dtype="bf16", mode=TOPK, top_k=128,
    softmax_scale=_inv_sqrt(128), select_scale=_inv_sqrt(128),
    plant="gist_align", plants_per_head=8, seed=2)

C3 = Workload(
    name="c3_topp_llama31_8b_128k", batch=4, kv_batch=4, n_q_heads=32, n_kv_heads=8,
    head_dim=128, n_ctx=131072, chunk_size=64, dtype="bf16", mode=TOPP, top_p=0.95,
    softmax_scale=_inv_sqrt(128), select_scale=_inv_sqrt(128), keep_first=1, keep_last=1,
    plant="zipf", zipf_s=1.1, seed=3)

C4 = Workload(
    name="c4_hssa_512k", batch=1, kv_batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
    n_ctx=524288, chunk_size=32, dtype="bf16", mode=HIER, top_k_seg=16, top_k=64, seg_size=32,
    softmax_scale=_inv_sqrt(128), select_scale=_inv_sqrt(128),
    plant="needles", plants_per_head=4, seed=4)

C5 = Workload(
    name="c5_rtpurbo_1m", batch=1, kv_batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
    n_ctx=1048576, chunk_size=1, dtype="bf16", mode=PROXY_TOPP, top_p=0.9, route_dim=16,
    softmax_scale=_inv_sqrt(128), select_scale=1.0 / (16 * math.sqrt(128)),
    local_kv_heads=(4, 5, 6, 7), sink=64, window=4096, attend_summary=False, seed=5)

FULL = {w.name: w for w in (C1, C2, C3, C4, C5)}

# Reduced twins: same structure, sizes the oracle finishes in seconds.
C2S = replace(C2, name="c2s", batch=2, kv_batch=2, n_ctx=4096, top_k=32, seed=12)
C3S = replace(C3, name="c3s", batch=2, kv_batch=2, n_ctx=16384, seed=13)
C4S = replace(C4, name="c4s", n_ctx=32768, top_k_seg=4, top_k=16, seed=14)
C5S = replace(C5, name="c5s", n_ctx=65536, window=1000, seed=15)
C1S = replace(C1, name="c1s", seed=11)

SMALL = {w.name: w for w in (C1S, C2S, C3S, C4S, C5S)}

# Context variants of the 128K workload (the same selection; what the heads attend to differs).
C3_HEADMASK = replace(C3, name="c3_topp_llama31_8b_128k_headmask", head_masks=True)
# The coverage budget rule on the 128K workload: cut 20% of the head-summed importance mass.
C3_COVERAGE = replace(C3, name="c3_coverage_llama31_8b_128k", mode=COVERAGE, tau=0.2, top_p=1.0)
C3_ALLSUM = replace(C3, name="c3_topp_llama31_8b_128k_allsum", all_summaries=True)
C3S_COVERAGE = replace(C3_COVERAGE, name="c3s_coverage", batch=2, kv_batch=2, n_ctx=16384, seed=16)
# Multi-query decode: 4 adjacent query tokens per sequence share each KV group's union (4 tokens x
# 4 heads = 16 query rows per group).
C3_MQ4 = replace(C3, name="c3_mq4_llama31_8b_128k", n_queries=4)
C3S_MQ4 = replace(C3_MQ4, name="c3s_mq4", batch=2, kv_batch=2, n_ctx=16384, seed=17)
VARIANTS = {w.name: w for w in (C3_HEADMASK, C3_ALLSUM, C3_COVERAGE, C3S_COVERAGE, C3_MQ4, C3S_MQ4)}

ALL = {**FULL, **SMALL, **VARIANTS}

# The workload the throughput metric is quoted on: 128K context, top-p decode.
BENCH = C3


# ---------------------------------------------------------------------------------------------
# Token-Sparse prefill (compress -> attend -> scatter) workloads.
@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int               # L tokens of the prompt
    window: int                # W most recent queries of the proxy attention map
    tau: float                 # coverage threshold of the global budget
    softmax_scale: float
    dtype: str = "bf16"
    beta: float = 4.0          # plant: every query of a KV group gets beta * u_g ...
    zipf_s: float = 1.1        # ... and key j gets gamma_j * u_g, a Zipf(s) logit profile
    seed: int = 0
    head_mode: tuple | None = None  # per query head: 1 = full attention, 0 = sparse (None: all sparse)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


# The 128K prompt of the Llama-3.1-8B shape (the page's 128K setting); 20% of the importance mass
# of the proxy map is cut.
P1 = PrefillWorkload(name="p1_tsa_llama31_8b_128k", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     seq_len=131072, window=64, tau=0.2, softmax_scale=_inv_sqrt(128), seed=31)
P1S = replace(P1, name="p1s", seq_len=4096, window=64, seed=32)
P1T = replace(P1, name="p1t", batch=2, n_q_heads=8, n_kv_heads=2, seq_len=1024, window=32, tau=0.3, seed=33)
# Head-wise routing over the same prompt: the first query head of every KV group runs full attention
# (8 of 32 heads), the others the Token-Sparse selection, all in the same launches.
P1M = replace(P1, name="p1m_elastic_llama31_8b_128k", head_mode=tuple(int(h % 4 == 0) for h in range(32)))
PREFILL = {w.name: w for w in (P1, P1S, P1T, P1M)}


@dataclass(frozen=True)
class GistWorkload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_tokens: int              # N raw tokens, M = N / chunk_size gists
    chunk_size: int
    softmax_scale: float
    dtype: str = "bf16"
    seed: int = 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_chunks(self) -> int:
        return self.n_tokens // self.chunk_size


# Gist-masked prefill of the Qwen2-7B shape with the SSA decode workload's chunking (16 raw tokens per
# gist) over a 32K prompt; small cases for parity: a 2K prompt, and odd shapes (one-token chunks,
# chunks that do not divide the 128-query block, a sequence that ends mid-block).
G1 = GistWorkload(name="p2_ssa_qwen2_7b_32k", batch=1, n_q_heads=28, n_kv_heads=4, head_dim=128, n_tokens=32768,
                  chunk_size=16, softmax_scale=_inv_sqrt(128), seed=41)
G1S = replace(G1, name="p2s", n_tokens=2048, seed=42)
G1T = replace(G1, name="p2t", batch=2, n_q_heads=4, n_kv_heads=2, n_tokens=1000, chunk_size=20, seed=43)
GIST = {w.name: w for w in (G1, G1S, G1T)}


def get(name: str):
    if name in ALL:
        return ALL[name]
    return PREFILL[name] if name in PREFILL else GIST[name]


def library_params(w: Workload) -> dict:
    """Keyword arguments of query_adaptive_sparse_amd.SparseDecoder for workload ``w``."""
    mode = {TOPK: "topk", TOPP: "topp", HIER: "hier", PROXY_TOPP: "topp", COVERAGE: "coverage"}[w.mode]
    return dict(
        batch=w.batch, n_queries=w.n_queries, kv_batch=w.kv_batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
        head_dim=w.head_dim, n_ctx=w.n_ctx, chunk_size=w.chunk_size, dtype=w.dtype, mode=mode,
        route="proxy" if w.mode == PROXY_TOPP else "summary", route_dim=w.route_dim,
        top_k=w.top_k, top_k_seg=w.top_k_seg, seg_size=w.seg_size, top_p=w.top_p, tau=w.tau,
        select_scale=w.select_scale, softmax_scale=w.softmax_scale,
        keep_first=w.keep_first, keep_last=w.keep_last, sink=w.sink, window=w.window,
        attend_summary=(2 if w.all_summaries else 1) if (w.attend_summary and w.mode != PROXY_TOPP) else 0,
        head_masks=w.head_masks, attend_blocks=w.attend_blocks,
        head_mode=[1 if g in w.local_kv_heads else 0 for g in range(w.n_kv_heads)])
