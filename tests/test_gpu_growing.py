"""A cache that grows between decode steps, one handle and one workspace for every step (needs an
MI355X).

Each step the caches hold ctx_len[b] tokens of a larger capacity; the step's T query tokens are
new, and afterwards their T keys and values are appended (and, when a chunk becomes complete, its
summary row), then ctx_len grows by T. Memory past each sequence's valid tokens and summary rows
holds NaN, so any read of it would poison the outputs. Every step is compared with the oracle run
on that step's cache: selections, union lists and scores bit-exact, outputs within max-abs 2e-3
and relative-L2 1e-3.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from synth import configs, gen
from tests import parity

pytestmark = pytest.mark.gpu

# (workload, query tokens per step, initial tokens per sequence, steps)
CASES = [
    ("c3s", 4, [16384 - 3 * 64 - 6, 12345], 4),   # top-p, chunks of 64: both sequences complete a chunk
    ("c2s", 2, [4096 - 16 - 3, 1000], 4),         # top-k, chunks of 16
    ("c3s_coverage", 1, [16384 - 64 - 2, 7000], 3),  # coverage budget
    ("c5s", 2, [65536 - 7], 3),                   # token-level proxy top-p with local heads
]


def _nan_like(x):
    return torch.full_like(x, float("nan"))


@pytest.mark.parametrize("name,T,n0,steps", CASES, ids=[c[0] for c in CASES])
def test_growing_cache_steps(name, T, n0, steps):
    from oracle import HostSource
    from query_adaptive_sparse_amd import SparseDecoder, make_tensors

    w = replace(configs.get(name), name=f"{name}_grow", n_queries=T)
    full = gen.make_inputs(w, device="cuda")
    B, C = w.batch, w.chunk_size
    assert all(n + T * steps <= w.n_ctx for n in n0)
    # device caches holding only each sequence's valid prefix; NaN elsewhere
    live = {k: _nan_like(full[k]) for k in ("K", "V", "Kg", "Vg", "Kp") if k in full}
    for b in range(B):
        bk = b if w.kv_batch > 1 else 0
        live["K"][bk, :, :n0[b]] = full["K"][bk, :, :n0[b]]
        live["V"][bk, :, :n0[b]] = full["V"][bk, :, :n0[b]]
        if "Kp" in live:
            live["Kp"][bk, :, :n0[b]] = full["Kp"][bk, :, :n0[b]]
        if "Kg" in live:
            live["Kg"][bk, :, :n0[b] // C] = full["Kg"][bk, :, :n0[b] // C]
            live["Vg"][bk, :, :n0[b] // C] = full["Vg"][bk, :, :n0[b] // C]
    dec = SparseDecoder(device="cuda", **configs.library_params(w))
    ctx = torch.tensor(n0, dtype=torch.int32, device="cuda")
    n = list(n0)
    completed = 0
    for step in range(steps):
        q = gen.normal((B, T, w.n_q_heads, w.head_dim), w.seed + 1000 + step, gen.T_Q, w.dtype, "cuda")
        inp = {"q": q, "K": live["K"], "V": live["V"], "Kg": live.get("Kg"), "Vg": live.get("Vg"),
               "Kp": live.get("Kp"), "P": full.get("P")}
        t = make_tensors(q, live["K"], live["V"], Kg=live.get("Kg"), Vg=live.get("Vg"), Kp=live.get("Kp"),
                         P=full.get("P"), ctx_len=ctx)
        out = torch.full((B, T, w.n_q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, T, w.n_q_heads), float("nan"), dtype=torch.float32, device="cuda")
        dec.step(t, out, lse)
        torch.cuda.synchronize()
        g_res = {"out": out.cpu().numpy().reshape(B, T * w.n_q_heads, w.head_dim),
                 "lse": lse.cpu().numpy().reshape(B, T * w.n_q_heads),
                 "sel": {k: v.cpu() for k, v in dec.selection().items()}}
        assert dec.status() == 0
        o_res = parity.ref.decode_step(w, HostSource({k: v for k, v in inp.items() if v is not None}), ctx_len=n)
        rep = parity.compare(w, g_res, o_res)
        print(f"[grow] {name} step {step} tokens {n}: {rep}", flush=True)
        # append the step's T tokens (and any completed chunk's summary row)
        for b in range(B):
            bk = b if w.kv_batch > 1 else 0
            a, e = n[b], n[b] + T
            live["K"][bk, :, a:e] = full["K"][bk, :, a:e]
            live["V"][bk, :, a:e] = full["V"][bk, :, a:e]
            if "Kp" in live:
                live["Kp"][bk, :, a:e] = full["Kp"][bk, :, a:e]
            if "Kg" in live and e // C > a // C:
                live["Kg"][bk, :, a // C:e // C] = full["Kg"][bk, :, a // C:e // C]
                live["Vg"][bk, :, a // C:e // C] = full["Vg"][bk, :, a // C:e // C]
                completed += e // C - a // C
            n[b] = e
        ctx.copy_(torch.tensor(n, dtype=torch.int32))
    if C > 1:
        assert completed >= 1, "no step completed a chunk"
