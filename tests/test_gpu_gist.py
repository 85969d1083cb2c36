"""Gist-masked (SSA) prefill through the HIP path against the fp64 oracle (needs an MI355X).

Outputs (q.K on the bf16 MFMA, P.V on the fp16 MFMA with V under a per-head power-of-two scale and
P rounded to fp16, fp32 accumulation) within max-abs 2e-3 and relative-L2 1e-3 of the oracle's
fp64 attention over every query's visible keys: all queries on the reduced shapes, sampled ones
(the first and last tokens and gists included) on the 2K and 32K prompts, the latter in the launch
configuration the benchmark times; V eight times larger (max-abs bound times 8) and V at the ends
of the bf16 range (per KV head, compared after removing the head's scale).
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import GistPrefillSource, gref
from synth import configs, gen
from tests.parity import ATOL, RTOL_L2

pytestmark = pytest.mark.gpu


def run_gpu(w, inp):
    from query_adaptive_sparse_amd import GistPrefill, make_gist_tensors
    gp = GistPrefill(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                     n_tokens=w.n_tokens, chunk_size=w.chunk_size, softmax_scale=w.softmax_scale)
    t = make_gist_tensors(inp["Q"], inp["K"], inp["V"], inp["Qg"], inp["Kg"], inp["Vg"])
    out = torch.full((w.batch, w.n_q_heads, w.n_tokens, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    outg = torch.full((w.batch, w.n_q_heads, w.n_chunks, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    gp.attend(t, out, outg)
    torch.cuda.synchronize()
    return out, outg


def _rows(n, k, rng):
    if k is None or k >= n:
        return list(range(n))
    return sorted(set(rng.choice(n, k, replace=False).tolist()) | {0, 1, n - 2, n - 1} - {-1})


def compare(w, inp, out, outg, raw_k=None, gist_k=None, seed=0, v_scale=1.0):
    rng = np.random.default_rng(seed)
    rr, gr = _rows(w.n_tokens, raw_k, rng), _rows(w.n_chunks, gist_k, rng)
    o = gref.gist_prefill(w, GistPrefillSource(inp), raw_rows=rr, gist_rows=gr)
    rep = {}
    for key, got_t, rows in (("raw", out, rr), ("gist", outg, gr)):
        ref = o["out" if key == "raw" else "out_gist"][:, :, rows]
        got = got_t[:, :, rows].cpu().numpy()
        assert np.all(np.isfinite(got)), f"{key}: non-finite output"
        d = got - ref
        rep[key] = (float(np.max(np.abs(d))), float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30)), len(rows))
        assert rep[key][0] <= ATOL * v_scale and rep[key][1] <= RTOL_L2, rep
    return rep


CASES = [("p2t", {}), ("p2t", dict(chunk_size=1, n_tokens=300)), ("p2t", dict(chunk_size=128, n_tokens=512)),
         ("p2t", dict(chunk_size=200, n_tokens=600)), ("p2t", dict(chunk_size=16, n_tokens=64)),
         ("p2t", dict(chunk_size=7, n_tokens=7)), ("p2t", dict(n_q_heads=2, n_kv_heads=2, chunk_size=32, n_tokens=416))]


@pytest.mark.parametrize("name,kw", CASES, ids=[f"{n}-" + "-".join(f"{k}{v}" for k, v in kw.items()) for n, kw in CASES])
def test_gist_reduced(name, kw):
    w = replace(configs.get(name), **kw)
    print(f"[gist] {w.name} {kw}", flush=True)
    inp = gen.make_gist_inputs(w, device="cuda")
    out, outg = run_gpu(w, inp)
    rep = compare(w, inp, out, outg)
    print(f"[gist] {w.name}: {rep}", flush=True)


def test_gist_2k_sampled():
    w = configs.get("p2s")
    inp = gen.make_gist_inputs(w, device="cuda")
    out, outg = run_gpu(w, inp)
    rep = compare(w, inp, out, outg, raw_k=48, gist_k=24, seed=1)
    print(f"[gist] {w.name}: {rep}", flush=True)


def test_gist_deterministic():
    w = configs.get("p2s")
    inp = gen.make_gist_inputs(w, device="cuda")
    a, ag = run_gpu(w, inp)
    b, bg = run_gpu(w, inp)
    assert torch.equal(a, b) and torch.equal(ag, bg)


def test_gist_32k_sampled():
    """The benchmark's workload and launch: 28 query heads over a 32768-token prompt in chunks of 16."""
    w = configs.get("p2_ssa_qwen2_7b_32k")
    inp = gen.make_gist_inputs(w, device="cuda")
    out, outg = run_gpu(w, inp)
    rep = compare(w, inp, out, outg, raw_k=12, gist_k=6, seed=2)
    print(f"[gist] {w.name}: {rep}", flush=True)


def test_gist_token_major_layout():
    """Token-major storage ([B][N][H][d] viewed as [B][H][N][d]): the kernels take the strides."""
    w = replace(configs.get("p2t"), chunk_size=8, n_tokens=264)
    inp = gen.make_gist_inputs(w, device="cuda")
    tm = {k: (v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) if torch.is_tensor(v) else v)
          for k, v in inp.items()}
    assert tm["Q"].stride(2) == w.n_q_heads * w.head_dim
    out, outg = run_gpu(w, tm)
    rep = compare(w, inp, out, outg)
    print(f"[gist] token-major {w.name}: {rep}", flush=True)


def test_gist_large_v():
    """Raw and gist V eight times larger (|v| up to about 35): rounding P to fp16 with the
    normaliser summed from the rounded values is the exact average under logits moved by at most
    2^-11, so the absolute error scales with |V| (max-abs bound times 8, relative-L2 unchanged)."""
    w = replace(configs.get("p2t"), chunk_size=16, n_tokens=512)
    inp = gen.make_gist_inputs(w, device="cuda")
    for k in ("V", "Vg"):
        inp[k] = (inp[k].float() * 8.0).to(torch.bfloat16)
    out, outg = run_gpu(w, inp)
    rep = compare(w, inp, out, outg, v_scale=8.0)
    print(f"[gist] V x8: {rep}", flush=True)


def test_gist_extreme_v_scales():
    """KV head 0's values (raw and gist) scaled by 2^-126 (bf16 values down to the subnormal range)
    and KV head 1's by 2^124 with one value of 3.2e38 (near the largest finite bf16): the per-head
    power-of-two conversion of V stays finite. The oracle runs on the same inputs; each head's
    outputs are compared after dividing both sides by its scale."""
    w = replace(configs.get("p2t"), n_q_heads=4, n_kv_heads=2, chunk_size=16, n_tokens=256)
    inp = gen.make_gist_inputs(w, device="cuda")
    for k in ("V", "Vg"):
        V = inp[k].float()
        V[:, 0] *= 2.0 ** -126
        V[:, 1] *= 2.0 ** 124
        inp[k] = V
    inp["V"][0, 1, 5, 7] = 3.2e38
    for k in ("V", "Vg"):
        inp[k] = inp[k].to(torch.bfloat16)
        assert torch.isfinite(inp[k].float()).all()
    out, outg = run_gpu(w, inp)
    o = gref.gist_prefill(w, GistPrefillSource(inp), raw_rows=list(range(w.n_tokens)),
                          gist_rows=list(range(w.n_chunks)))
    G = w.n_q_heads // w.n_kv_heads
    for key, got_t in (("out", out), ("out_gist", outg)):
        got = got_t.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), f"{key}: non-finite output"
        for g, k in ((0, -126), (1, 124)):
            hs = slice(g * G, (g + 1) * G)
            a = got[:, hs] * 2.0 ** -k
            r = o[key][:, hs] * 2.0 ** -k
            d = a - r
            max_abs = float(np.max(np.abs(d)))
            rel = float(np.linalg.norm(d) / np.linalg.norm(r))
            vmax = max(float(np.max(np.abs(inp[n][:, g].double().cpu().numpy()))) for n in ("V", "Vg")) * 2.0 ** -k
            print(f"[gist] {key} KV head {g} scaled 2^{k}: max_abs {max_abs:.2e} rel_l2 {rel:.2e}", flush=True)
            assert max_abs <= ATOL * max(1.0, vmax / 4.4)
            assert rel <= RTOL_L2
