"""Helpers that run the HIP path and compare it with the fp64 oracle.

Tolerances: selections, candidate lists and group lists bit-exact; fp64 scores
bit-exact (both sides sum in index order, see the oracle and the score
kernels); attention outputs within max-abs 2e-3 and relative-L2 1e-3, lse within
max-abs 2e-3 (bf16 inputs, fp32 accumulation).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import HostSource, ref
from synth import configs, gen

ATOL = 2e-3
RTOL_L2 = 1e-3


def lib_tensors(inp):
    from query_adaptive_sparse_amd import make_tensors
    return make_tensors(inp["q"], inp["K"], inp["V"], Kg=inp.get("Kg"), Vg=inp.get("Vg"), Kmg=inp.get("Kmg"),
                        Kp=inp.get("Kp"), P=inp.get("P"))


def run_gpu(w, inp, **overrides):
    """One decode step through the C ABI; returns host copies of everything."""
    from query_adaptive_sparse_amd import SparseDecoder
    params = configs.library_params(w)
    params.update(overrides)
    dec = SparseDecoder(device="cuda", **params)
    t = lib_tensors(inp)
    T = w.n_queries
    # out [B][T][Hq][d] (T query tokens per sequence), compared as [B][T * Hq][d]
    out = torch.full((w.batch, T, w.n_q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((w.batch, T, w.n_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    dec.step(t, out, lse)
    torch.cuda.synchronize()
    sel = {k: v.cpu() for k, v in dec.selection().items()}
    return {"out": out.cpu().numpy().reshape(w.batch, T * w.n_q_heads, w.head_dim),
            "lse": lse.cpu().numpy().reshape(w.batch, T * w.n_q_heads), "sel": sel, "decoder": dec}


def bits_to_set(words: torch.Tensor) -> np.ndarray:
    w = words.numpy().view(np.uint32)
    bits = np.unpackbits(w.view(np.uint8), bitorder="little")
    return np.nonzero(bits)[0]


def oracle_step(w, inp, groups=None, attend_groups=None):
    return ref.decode_step(w, HostSource(inp), groups=groups, attend_groups=attend_groups)


def compare(w, g_res, o_res, check_scores=True):
    """Assert parity; returns a dict of the numbers behind the result."""
    sel = g_res["sel"]
    G = w.group
    report = {"heads": 0, "groups": 0, "min_margin": math.inf}
    for (b, g), r in o_res["sel"].items():
        report["min_margin"] = min(report["min_margin"], r["margin"])
        for h, S in r["heads"].items():
            got = bits_to_set(sel["head_bits"][b, h])
            assert np.array_equal(got, S), f"head set differs at b={b} h={h}: {len(got)} vs {len(S)} entries"
            report["heads"] += 1
            if check_scores and h in r["scores"]:
                s_ref = r["scores"][h]
                s_gpu = sel["scores0"][b, h].numpy()[:len(s_ref)]  # a growing cache scores a prefix
                assert np.array_equal(s_gpu, s_ref), (
                    f"scores differ at b={b} h={h}: max |d| {np.max(np.abs(s_gpu - s_ref)):.3g}")
            if h in r["cand"]:
                cand, s2 = r["cand"][h]
                assert np.array_equal(sel["cand1"][b, h].numpy(), cand), f"candidates differ at b={b} h={h}"
                if check_scores:
                    assert np.array_equal(sel["scores1"][b, h].numpy(), s2), f"level-1 scores differ b={b} h={h}"
        cnt = int(sel["count"][b, g])
        U = r["union"]
        assert cnt == len(U), f"union size differs at b={b} g={g}: {cnt} vs {len(U)}"
        assert np.array_equal(sel["list"][b, g, :cnt].numpy(), U), f"union list differs at b={b} g={g}"
        report["groups"] += 1
    o_ref, l_ref = o_res["out"], o_res["lse"]
    mask = ~np.isnan(l_ref)
    o_gpu, l_gpu = g_res["out"], g_res["lse"]
    assert np.all(np.isfinite(o_gpu[mask])) and np.all(np.isfinite(l_gpu[mask])), "non-finite GPU output"
    d = o_gpu[mask] - o_ref[mask]
    report["max_abs"] = float(np.max(np.abs(d))) if d.size else 0.0
    report["rel_l2"] = float(np.linalg.norm(d) / max(np.linalg.norm(o_ref[mask]), 1e-30)) if d.size else 0.0
    report["lse_max_abs"] = float(np.max(np.abs(l_gpu[mask] - l_ref[mask]))) if d.size else 0.0
    assert report["max_abs"] <= ATOL, report
    assert report["rel_l2"] <= RTOL_L2, report
    assert report["lse_max_abs"] <= ATOL, report
    return report


def gpu_inputs(w, seed=None):
    return gen.make_inputs(w, device="cuda", seed=seed)
