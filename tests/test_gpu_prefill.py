"""Token-Sparse prefill through the HIP path against the fp64 oracle (needs an MI355X).

Selections bit-exact: the budget, every head's position bitmap and list. Importance within
1e-12 relative (both sides fp64; the softmax normalisers are summed in different orders).
Outputs (fp32 from bf16 MFMA with fp32 accumulation) within max-abs 2e-3 and relative-L2 1e-3 of
the oracle's fp64 attention; positions a head did not keep are exactly zero.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import PrefillSource, pref
from synth import configs, gen
from tests.parity import ATOL, RTOL_L2

pytestmark = pytest.mark.gpu


def run_gpu(w, inp):
    from query_adaptive_sparse_amd import SparsePrefill, make_prefill_tensors
    sp = SparsePrefill(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                       seq_len=w.seq_len, window=w.window, tau=w.tau, softmax_scale=w.softmax_scale, device="cuda")
    hm = None if w.head_mode is None else torch.tensor(w.head_mode, dtype=torch.int8, device="cuda")
    t = make_prefill_tensors(inp["Q"], inp["K"], inp["V"], head_mode=hm)
    out = torch.full((w.batch, w.n_q_heads, w.seq_len, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    sp.step(t, out)
    torch.cuda.synchronize()
    sel = {k: v.cpu() for k, v in sp.selection().items()}
    return sel, out


def compare(w, inp, sel, out, heads=None, rows_per_head=None):
    src = PrefillSource(inp)
    o = pref.tsa_prefill(w, src, heads=heads, rows_per_head=rows_per_head)
    assert int(sel["status"][0]) == 0
    rep = {"budgets": [], "min_gap": np.inf, "min_margin": np.inf, "imp_rel": 0.0}
    for b in range(w.batch):
        r = o["sel"][b]
        k = int(sel["budget"][b])
        rep["budgets"].append(k)
        rep["min_margin"] = min(rep["min_margin"], r["margin"])
        all_full = w.head_mode is not None and all(w.head_mode)
        assert all_full or k == r["budget"], f"budget differs at b={b}: {k} vs {r['budget']}"
        for h in range(w.n_q_heads):
            imp = sel["importance"][b, h].numpy()
            rep["imp_rel"] = max(rep["imp_rel"], float(np.max(np.abs(imp - r["importance"][h]) / np.abs(r["importance"][h]))))
            bits = np.unpackbits(sel["head_bits"][b, h].numpy().view(np.uint8), bitorder="little")[:w.seq_len]
            S = r["sets"][h]
            assert np.array_equal(np.nonzero(bits)[0], S), f"head set differs at b={b} h={h}"
            assert np.array_equal(sel["list"][b, h, :len(S)].numpy(), S), f"list differs at b={b} h={h}"
            rep["min_gap"] = min(rep["min_gap"], r["gaps"][h])
    assert rep["imp_rel"] <= 1e-12, rep
    ref = o["out"]
    got = out.cpu().numpy()
    mask = ~np.isnan(ref)
    assert np.all(np.isfinite(got[mask]))
    d = got[mask] - ref[mask]
    rep["max_abs"] = float(np.max(np.abs(d)))
    rep["rel_l2"] = float(np.linalg.norm(d) / max(np.linalg.norm(ref[mask]), 1e-30))
    zero = ref == 0.0
    assert np.all(got[zero] == 0.0), "an unkept position is not zero"
    assert rep["max_abs"] <= ATOL and rep["rel_l2"] <= RTOL_L2, rep
    return rep


CASES = [("p1t", {}), ("p1t", dict(tau=0.0)), ("p1t", dict(tau=0.995)), ("p1t", dict(window=1)),
         ("p1t", dict(seq_len=1000, window=17)), ("p1t", dict(seq_len=64, window=64, tau=0.2)),
         ("p1t", dict(n_q_heads=8, n_kv_heads=8, tau=0.1)),
         ("p1t", dict(head_mode=(1, 0, 0, 0, 0, 1, 1, 0))), ("p1t", dict(head_mode=(1,) * 8)),
         ("p1t", dict(seq_len=200, window=8, head_mode=(0, 0, 0, 0, 0, 0, 0, 1)))]


@pytest.mark.parametrize("name,kw", CASES, ids=[f"{n}-" + "-".join(f"{k}{v}" for k, v in kw.items()) for n, kw in CASES])
def test_prefill_reduced(name, kw):
    w = replace(configs.get(name), **kw)
    print(f"[prefill] {w.name} {kw}", flush=True)
    inp = gen.make_prefill_inputs(w, device="cuda")
    sel, out = run_gpu(w, inp)
    rep = compare(w, inp, sel, out)
    print(f"[prefill] {w.name}: {rep}", flush=True)


def test_prefill_4k_sampled():
    """32 heads, 4K prompt, 64-query window: every selection, sampled output rows of 4 heads."""
    w = configs.get("p1s")
    inp = gen.make_prefill_inputs(w, device="cuda")
    sel, out = run_gpu(w, inp)
    rep = compare(w, inp, sel, out, heads=[0, 9, 22, 31], rows_per_head=48)
    print(f"[prefill] {w.name}: {rep}", flush=True)


def test_prefill_deterministic():
    w = configs.get("p1t")
    inp = gen.make_prefill_inputs(w, device="cuda")
    s1, o1 = run_gpu(w, inp)
    s2, o2 = run_gpu(w, inp)
    assert torch.equal(o1, o2)
    for k in ("importance", "budget", "head_bits"):
        assert torch.equal(s1[k], s2[k]), k


def test_prefill_128k_sampled():
    """The 128K prompt (32 heads): importance of two sampled heads against the oracle; every head's
    set equals its top-budget by the GPU's own importance (verified on the sampled heads); the
    budget equals the coverage cut of the GPU importances summed over heads; sampled output rows."""
    from oracle import ref
    w = configs.get("p1_tsa_llama31_8b_128k")
    print(f"[prefill-128k] generating inputs", flush=True)
    inp = gen.make_prefill_inputs(w, device="cuda")
    sel, out = run_gpu(w, inp)
    assert int(sel["status"][0]) == 0
    src = PrefillSource(inp)
    L, W = w.seq_len, w.window
    imp_gpu = sel["importance"][0].numpy()
    for h in (3, 26):
        print(f"[prefill-128k] oracle importance of head {h}", flush=True)
        imp = pref.proxy_importance(src.q_rows(0, h, np.arange(L - W, L)), src.k_all(0, h // w.group),
                                    w.softmax_scale, L - W)
        assert np.max(np.abs(imp_gpu[h] - imp) / imp) <= 1e-12
    total = np.zeros(L)
    for h in range(w.n_q_heads):
        total = total + imp_gpu[h]
    k, margin = ref.coverage_budget(total, w.tau)
    assert int(sel["budget"][0]) == k, (int(sel["budget"][0]), k, margin)
    for h in range(w.n_q_heads):
        S = ref.select_top_k(imp_gpu[h], k)
        assert np.array_equal(sel["list"][0, h, :k].numpy(), S), h
    rng = np.random.default_rng(5)
    got = out.cpu().numpy()
    worst = 0.0
    for h in (3, 26):
        S = sel["list"][0, h, :k].numpy().astype(np.int64)
        rows = sorted(set(rng.choice(k, 24, replace=False).tolist()) | {0, k - 1})
        o, _ = pref.tsa_attend_rows(w, src, 0, h, S, rows)
        d = got[0, h, S[rows]] - o
        worst = max(worst, float(np.max(np.abs(d))))
        assert np.max(np.abs(d)) <= ATOL and np.linalg.norm(d) / np.linalg.norm(o) <= RTOL_L2, h
        keep = np.zeros(L, dtype=bool)
        keep[S] = True
        assert np.all(got[0, h, ~keep] == 0.0)
    print(f"[prefill-128k] budget {k} margin {margin:.2e} max_abs {worst:.2e}", flush=True)


def test_prefill_mixed_128k_sampled():
    """Head-wise routing at 128K (8 full-attention heads of 32): the budget equals the coverage cut of
    the GPU importances summed over the sparse heads only; full heads keep every position; sampled
    output rows of a full and a sparse head against the oracle."""
    from oracle import ref
    w = configs.get("p1m_elastic_llama31_8b_128k")
    print(f"[prefill-mixed] generating inputs", flush=True)
    inp = gen.make_prefill_inputs(w, device="cuda")
    sel, out = run_gpu(w, inp)
    assert int(sel["status"][0]) == 0
    src = PrefillSource(inp)
    L = w.seq_len
    imp_gpu = sel["importance"][0].numpy()
    total = np.zeros(L)
    for h in range(w.n_q_heads):
        if not w.head_mode[h]:
            total = total + imp_gpu[h]
    k, margin = ref.coverage_budget(total, w.tau)
    assert int(sel["budget"][0]) == k, (int(sel["budget"][0]), k, margin)
    rng = np.random.default_rng(6)
    got = out.cpu().numpy()
    worst = 0.0
    for h in (4, 5):
        full = bool(w.head_mode[h])
        S = np.arange(L) if full else ref.select_top_k(imp_gpu[h], k)
        assert np.array_equal(sel["list"][0, h, :len(S)].numpy(), S), h
        rows = sorted(set(rng.choice(len(S), 16, replace=False).tolist()) | {0, len(S) - 1})
        print(f"[prefill-mixed] head {h} ({'full' if full else 'sparse'}): oracle rows", flush=True)
        o, _ = pref.tsa_attend_rows(w, src, 0, h, S, rows)
        d = got[0, h, S[rows]] - o
        worst = max(worst, float(np.max(np.abs(d))))
        assert np.max(np.abs(d)) <= ATOL and np.linalg.norm(d) / np.linalg.norm(o) <= RTOL_L2, h
    print(f"[prefill-mixed] budget {k} margin {margin:.2e} max_abs {worst:.2e}", flush=True)


def test_prefill_token_major_layout():
    """Token-major storage ([B][L][H][d] viewed as [B][H][L][d]): the kernels take the strides."""
    w = replace(configs.get("p1t"), seq_len=300, window=16)
    inp = gen.make_prefill_inputs(w, device="cuda")
    tm = {k: (v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) if torch.is_tensor(v) else v)
          for k, v in inp.items()}
    assert tm["K"].stride(2) == w.n_kv_heads * w.head_dim
    sel, out = run_gpu(w, tm)
    rep = compare(w, inp, sel, out)
    print(f"[prefill] token-major {w.name}: {rep}", flush=True)
