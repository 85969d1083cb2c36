"""The seeded generator: deterministic, subset-consistent, and the planted structure holds."""
import hashlib

import numpy as np
import torch

from oracle import HostSource, ref
from synth import configs, gen


def test_codes_are_stable():
    idx = torch.arange(0, 1 << 16, dtype=torch.int64)
    c = gen.codes(3, gen.T_K, idx).to(torch.int32).numpy()
    assert c.min() >= 0 and c.max() < 65536
    # equidistribution: every 1/16 bucket within 5% of its share
    hist = np.bincount(c >> 12, minlength=16)
    assert np.all(np.abs(hist - 4096) < 205), hist
    again = gen.codes(3, gen.T_K, idx).to(torch.int32).numpy()
    assert np.array_equal(c, again)
    assert not np.array_equal(c, gen.codes(4, gen.T_K, idx).to(torch.int32).numpy())
    # the hash is pure integer arithmetic: pin it against a plain-int evaluation
    for i in (0, 1, 77, 65535, (1 << 33) + 5):
        k1, k2 = gen._keys(3, gen.T_K)
        x = gen._lowbias32_int((i & 0xFFFFFFFF) ^ k1)
        x = gen._lowbias32_int(x ^ ((i >> 32) ^ k2))
        assert int(gen.codes(3, gen.T_K, torch.tensor([i]))[0]) == x >> 16


def test_table_is_normal_quantiles():
    tab = gen.table("f64", "cpu").numpy()
    assert np.all(np.diff(tab) > 0)
    assert abs(tab.mean()) < 1e-12 and abs(tab.std() - 1) < 1e-3
    bf = gen.table("bf16", "cpu").float().numpy()
    assert np.all(np.abs(bf - tab) <= np.abs(tab) * 2.0 ** -8 + 1e-30)


def test_rows_match_whole_array():
    shape = (2, 3, 50, 16)
    full = gen.normal(shape, 9, gen.T_V, "bf16")
    rows = torch.tensor([0, 7, 49, 3])
    got = gen.rows_at(shape, 9, gen.T_V, "bf16", 1, 2, rows)
    assert torch.equal(got, full[1, 2, rows])
    sha = hashlib.sha256(full.view(torch.int16).numpy().tobytes()).hexdigest()
    assert sha == hashlib.sha256(gen.normal(shape, 9, gen.T_V, "bf16", block=97).view(torch.int16).numpy().tobytes()).hexdigest()


def test_plants_c2s_in_top_k():
    w = configs.get("c2s")
    x = gen.make_inputs(w)
    src = HostSource(x)
    G = w.group
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            perm = gen.permutation(w.seed, gen.T_PERM, b * w.n_kv_heads + g, w.n_chunks)
            for j in range(G):
                h = g * G + j
                s = ref.chunk_scores(src.q[b, h], src.Kg[b, g])
                top = set(ref.select_top_k(s, w.top_k).tolist())
                planted = perm[j * w.plants_per_head:(j + 1) * w.plants_per_head].tolist()
                assert set(planted) <= top


def test_plants_c4s_needles_selected():
    w = configs.get("c4s")
    x = gen.make_inputs(w)
    r = ref.decode_step(w, HostSource(x), attend_groups=[])
    for (b, g), res in r["sel"].items():
        # each head picks its own needles: 4 disjoint sets of 16 chunks
        assert len(res["union"]) == w.group * w.top_k


def test_zipf_profile_c3s():
    w = configs.get("c3s")
    x = gen.make_inputs(w)
    src = HostSource(x)
    s = ref.chunk_scores(src.q[0, 0], src.Kg[0, 0]) * w.select_scale
    # logits follow -1.1 ln(rank) up to bf16 rounding of the keys
    srt = np.sort(s)[::-1]
    ranks = np.arange(1, len(srt) + 1)
    slope = np.polyfit(np.log(ranks[:100]), srt[:100], 1)[0]
    assert abs(slope + w.zipf_s) < 0.05, slope
