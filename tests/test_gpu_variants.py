"""The two context variants through the HIP path against the oracle (needs an MI355X):
per-head masks inside the loaded union, and every chunk's summary K/V in the context."""
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
           ("c2s", dict(head_masks=True, chunk_size=1, n_ctx=8192, top_k=700))]


@pytest.mark.parametrize("name,kw", REDUCED, ids=[f"{n}-" + "-".join(k for k in kw) for n, kw in REDUCED])
def test_variant_reduced(name, kw):
    w = replace(configs.get(name), name=f"{name}_variant", **kw)
    print(f"[variant] {w.name} {kw}", flush=True)
    inp = gen.make_inputs(w, device="cuda")
    g = parity.run_gpu(w, inp)
    o = parity.oracle_step(w, inp)
    rep = parity.compare(w, g, o)
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
