"""Token-Sparse prefill through the HIP path against the fp64 oracle (needs an MI355X).

Selections bit-exact: the budget, every head's position bitmap and list. Importance within
1e-12 relative (both sides fp64; the softmax normalisers are summed in different orders).
Outputs (fp32; q.K on the bf16 MFMA, P.V on the fp16 MFMA with P rounded to fp16 and the
normaliser summed from the rounded values, fp32 accumulation) within max-abs 2e-3 (for values of
the synthetic N(0,1) scale; the bound scales with |V|) and relative-L2 1e-3 of the oracle's fp64
attention; positions a head did not keep are exactly zero.
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


def compare(w, inp, sel, out, heads=None, rows_per_head=None, v_scale=1.0):
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
    assert rep["max_abs"] <= ATOL * v_scale and rep["rel_l2"] <= RTOL_L2, rep
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


def _oracle_select_threads(w, src, tag):
    """The oracle's selection of sequence 0, every head's importance computed by the oracle on a
    pool of host threads (numpy releases the GIL in its array loops), with a progress line per head."""
    from concurrent.futures import ThreadPoolExecutor
    done = []

    def pool_map(fn, heads):
        def run(h):
            r = fn(h)
            done.append(h)
            print(f"[{tag}] oracle importance of head {h} ({len(done)}/{w.n_q_heads})", flush=True)
            return r
        with ThreadPoolExecutor(max_workers=16) as ex:
            return list(ex.map(run, heads))

    return pref.tsa_select(w, src, 0, pool_map=pool_map)


def _check_128k(w, tag, sample_heads, seed):
    """Every head's importance (1e-12 relative), the budget and every head's position set and list
    against the oracle's own selection of the 128K prompt; sampled output rows of `sample_heads`."""
    print(f"[{tag}] generating inputs", flush=True)
    inp = gen.make_prefill_inputs(w, device="cuda")
    sel, out = run_gpu(w, inp)
    assert int(sel["status"][0]) == 0
    src = PrefillSource(inp)
    L = w.seq_len
    r = _oracle_select_threads(w, src, tag)
    imp_gpu = sel["importance"][0].numpy()
    modes = pref.head_modes(w)
    worst_rel = 0.0
    for h in range(w.n_q_heads):
        rel = float(np.max(np.abs(imp_gpu[h] - r["importance"][h]) / r["importance"][h]))
        worst_rel = max(worst_rel, rel)
        assert rel <= 1e-12, (h, rel)
    k = r["budget"]
    if not all(modes):
        assert int(sel["budget"][0]) == k, (int(sel["budget"][0]), k, r["margin"])
    for h in range(w.n_q_heads):
        S = r["sets"][h]
        bits = np.unpackbits(sel["head_bits"][0, h].numpy().view(np.uint8), bitorder="little")[:L]
        assert np.array_equal(np.nonzero(bits)[0], S), f"head {h} set (gap {r['gaps'][h]:.2e})"
        assert np.array_equal(sel["list"][0, h, :len(S)].numpy(), S), f"head {h} list"
    rng = np.random.default_rng(seed)
    got = out.cpu().numpy()
    worst = 0.0
    for h in sample_heads:
        S = r["sets"][h]
        rows = sorted(set(rng.choice(len(S), 16, replace=False).tolist()) | {0, len(S) - 1})
        print(f"[{tag}] head {h} ({'full' if modes[h] else 'sparse'}): oracle rows", flush=True)
        o, _ = pref.tsa_attend_rows(w, src, 0, h, S, rows)
        d = got[0, h, S[rows]] - o
        worst = max(worst, float(np.max(np.abs(d))))
        assert np.max(np.abs(d)) <= ATOL and np.linalg.norm(d) / np.linalg.norm(o) <= RTOL_L2, h
        keep = np.zeros(L, dtype=bool)
        keep[S] = True
        assert np.all(got[0, h, ~keep] == 0.0)
    print(f"[{tag}] budget {k} margin {r['margin']:.2e} importance rel {worst_rel:.1e} max_abs {worst:.2e}",
          flush=True)


@pytest.mark.timeout(900)
def test_prefill_128k_sampled():
    """The 128K prompt (32 heads): every head's importance, the budget and every head's set against
    the oracle's own (importances evaluated by the oracle for all 32 heads); sampled output rows."""
    _check_128k(configs.get("p1_tsa_llama31_8b_128k"), "prefill-128k", (3, 26), 5)


@pytest.mark.timeout(900)
def test_prefill_mixed_128k_sampled():
    """Head-wise routing at 128K (8 full-attention heads of 32): the budget is the oracle's coverage
    cut of the sparse heads' importances, full heads keep every position, every sparse head's set
    is the oracle's; sampled output rows of a full and a sparse head."""
    _check_128k(configs.get("p1m_elastic_llama31_8b_128k"), "prefill-mixed", (4, 5), 6)


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


def test_prefill_large_v():
    """V eight times larger (|v| up to about 35). Each output row is a softmax average of V rows;
    rounding P to fp16 with the normaliser summed from the rounded values is the exact average under
    logits moved by at most 2^-11, so the absolute error scales with |V|: the max-abs bound is the
    N(0,1) one times 8, the relative-L2 bound unchanged."""
    w = configs.get("p1t")
    inp = gen.make_prefill_inputs(w, device="cuda")
    inp["V"] = (inp["V"].float() * 8.0).to(torch.bfloat16)
    sel, out = run_gpu(w, inp)
    rep = compare(w, inp, sel, out, v_scale=8.0)
    print(f"[prefill] V x8: {rep}", flush=True)


def test_prefill_extreme_v_scales():
    """KV group 0's V scaled by 2^-126 (bf16 values down to the subnormal range) and group 1's by
    2^124 with one value of 3.2e38 (near the largest finite bf16): the per-head power-of-two
    conversion of V stays finite. The oracle runs on the same scaled inputs; outputs of each group
    are compared after dividing both sides by the group's scale."""
    w = configs.get("p1t")
    inp = gen.make_prefill_inputs(w, device="cuda")
    V = inp["V"].float()
    V[:, 0] *= 2.0 ** -126
    V[:, 1] *= 2.0 ** 124
    V[0, 1, 5, 7] = 3.2e38
    inp["V"] = V.to(torch.bfloat16)
    assert torch.isfinite(inp["V"].float()).all()
    sel, out = run_gpu(w, inp)
    src = PrefillSource(inp)
    o = pref.tsa_prefill(w, src)
    got = out.cpu().numpy().astype(np.float64)
    ref_out = o["out"]
    assert np.all(np.isfinite(got)), "non-finite output"
    for g, k in ((0, -126), (1, 124)):
        hs = slice(g * w.group, (g + 1) * w.group)
        a = got[:, hs] * 2.0 ** -k
        r = ref_out[:, hs] * 2.0 ** -k
        d = a - r
        max_abs = float(np.max(np.abs(d)))
        rel = float(np.linalg.norm(d) / np.linalg.norm(r))
        print(f"[prefill] V group {g} scaled 2^{k}: max_abs {max_abs:.2e} rel_l2 {rel:.2e}", flush=True)
        assert max_abs <= ATOL * max(1.0, float(np.max(np.abs(inp['V'][:, g].double().cpu().numpy()))) * 2.0 ** -k / 4.4)
        assert rel <= RTOL_L2
