"""Full-size workloads, in the launch configuration bench.py uses (needs an MI355X).

Selections, lists and fp64 scores are compared for every head and group;
attention outputs for a seeded sample of (sequence, KV group) units that the
oracle evaluates one by one.
"""
import numpy as np
import pytest
import torch

from synth import configs
from tests import parity

pytestmark = pytest.mark.gpu

# (workload, number of (sequence, KV group) units whose outputs the oracle checks)
CASES = [("c1_tiny_f32", 16), ("c2_ssa_qwen2_7b_32k", 4), ("c3_topp_llama31_8b_128k", 3),
         ("c4_hssa_512k", 8), ("c5_rtpurbo_1m", 2)]


@pytest.mark.parametrize("name,n_attend", CASES, ids=[c[0] for c in CASES])
def test_parity_full(name, n_attend):
    w = configs.get(name)
    print(f"[full] {name}: generating inputs", flush=True)
    inp = parity.gpu_inputs(w)
    g = parity.run_gpu(w, inp)
    status = int(g["sel"]["status"][0])
    assert status == 0, f"device status flags {status}"
    groups = [(b, gg) for b in range(w.batch) for gg in range(w.n_kv_heads)]
    rng = np.random.default_rng(w.seed)
    pick = [groups[i] for i in rng.choice(len(groups), size=min(n_attend, len(groups)), replace=False)]
    if w.local_kv_heads:  # one scored and one local group at least
        pick = [(0, 0), (0, w.local_kv_heads[0])]
    print(f"[full] {name}: oracle on {len(groups)} selections, {len(pick)} attention units", flush=True)
    o = parity.oracle_step(w, inp, groups=groups, attend_groups=pick)
    rep = parity.compare(w, g, o)
    print(f"[full] {name}: {rep}", flush=True)
    del inp
    torch.cuda.empty_cache()
