"""The variants through the HIP path against the oracle (needs an MI355X): per-head masks
inside the loaded union, every chunk's summary K/V in the context, the coverage budget, and
multi-query decode (several adjacent query tokens per sequence)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from synth import configs, gen
from tests import parity

pytestmark = pytest.mark.gpu

REDUCED = [("c1s", dict(head_masks=True)), ("c2s", dict(head_masks=True)), ("c3s", dict(head_masks=True)),
           ("c4s", dict(head_masks=True)), ("c5s", dict(head_masks=True)),
           ("c1s", dict(all_summaries=True)), ("c2s", dict(all_summaries=True)), ("c3s", dict(all_summaries=True)),
           ("c4s", dict(all_summaries=True)), ("c3s", dict(head_masks=True, all_summaries=True)),
           ("c2s", dict(head_masks=True, chunk_size=1, n_ctx=8192, top_k=700)),
           # coverage budget: tau 0 keeps all but one entry, tau near 1 clamps the budget to 1
           ("c1s", dict(mode="coverage", tau=0.3)), ("c2s", dict(mode="coverage", tau=0.1)),
           ("c3s", dict(mode="coverage", tau=0.0)), ("c3s", dict(mode="coverage", tau=0.999)),
           ("c3s", dict(mode="coverage", tau=0.5, head_masks=True, all_summaries=True)),
           ("c2s", dict(mode="coverage", tau=0.15, chunk_size=1, n_ctx=2048, local_kv_heads=(1, 3), sink=16,
                        window=100)),
           # multi-query decode: T adjacent tokens per sequence; T x G rows per group up to 16
           # (8 rows: hi / lo halves of P in one MFMA; more: two MFMAs)
           ("c1s", dict(n_queries=2)), ("c1s", dict(n_queries=4)), ("c2s", dict(n_queries=2)),
           ("c3s", dict(n_queries=3)), ("c4s", dict(n_queries=2)), ("c5s", dict(n_queries=2)),
           ("c3s", dict(n_queries=4, head_masks=True)), ("c3s", dict(n_queries=2, mode="coverage", tau=0.3)),
           ("c1s", dict(n_queries=16, n_q_heads=1))]


@pytest.mark.parametrize("name,kw", REDUCED, ids=[f"{n}-" + "-".join(k for k in kw) for n, kw in REDUCED])
def test_variant_reduced(name, kw):
    w = replace(configs.get(name), name=f"{name}_variant", **kw)
    print(f"[variant] {w.name} {kw}", flush=True)
    inp = gen.make_inputs(w, device="cuda")
    g = parity.run_gpu(w, inp)
    o = parity.oracle_step(w, inp)
    rep = parity.compare(w, g, o)
    if w.mode == "coverage":
        rep["budgets"] = sorted({r["budget"] for r in o["sel"].values() if "budget" in r})
    print(f"[variant] {w.name}: {rep}", flush=True)


@pytest.mark.parametrize("name", sorted(configs.VARIANTS))
def test_variant_full(name):
    """Full 128K workload with a variant: every selection compared, attention for sampled groups."""
    w = configs.get(name)
    print(f"[variant-full] {name}: generating inputs", flush=True)
    inp = parity.gpu_inputs(w)
    g = parity.run_gpu(w, inp)
    assert int(g["sel"]["status"][0]) == 0
    groups = [(b, gg) for b in range(w.batch) for gg in range(w.n_kv_heads)]
    rng = np.random.default_rng(w.seed + 100)
    pick = [groups[i] for i in rng.choice(len(groups), size=3, replace=False)]
    o = parity.oracle_step(w, inp, groups=groups, attend_groups=pick)
    rep = parity.compare(w, g, o)
    print(f"[variant-full] {name}: {rep}", flush=True)
    del inp
    torch.cuda.empty_cache()
