"""Degenerate and boundary cases of the HIP path against the oracle (needs an MI355X)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from synth import configs, gen
from tests import parity

pytestmark = pytest.mark.gpu


def _run(w, inp, **over):
    print(f"[edge] {w.name} {over}", flush=True)
    g = parity.run_gpu(w, inp, **over)
    o = parity.oracle_step(w, inp)
    rep = parity.compare(w, g, o)
    print(f"[edge] {w.name}: {rep}", flush=True)
    return g, o


@pytest.mark.parametrize("n_ctx", [4096, 32768])
def test_all_scores_equal_topk(n_ctx):
    """Every summary key identical: all scores tie, top-k keeps the lowest indices. At 2048 chunks
    the tie overflows both histogram levels and takes the whole-row sort."""
    w = replace(configs.get("c2s"), name="tie_topk", n_ctx=n_ctx, top_k=37)
    inp = gen.make_inputs(w, device="cuda")
    inp["Kg"][:] = inp["Kg"][:, :, :1]
    g, o = _run(w, inp)
    for (b, gg), r in o["sel"].items():
        for h, S in r["heads"].items():
            assert S.tolist() == list(range(37))


@pytest.mark.parametrize("n_ctx", [16384, 131072])
def test_all_scores_equal_topp(n_ctx):
    """All-equal masses: top-p keeps the shortest index prefix reaching p."""
    w = replace(configs.get("c3s"), name="tie_topp", n_ctx=n_ctx, top_p=0.3, keep_first=0, keep_last=0)
    inp = gen.make_inputs(w, device="cuda")
    inp["Kg"][:] = inp["Kg"][:, :, :1]
    _run(w, inp)


def test_clustered_scores():
    """Most scores packed in a narrow band far below a few large ones (second histogram level)."""
    w = replace(configs.get("c3s"), name="cluster", top_p=0.9, keep_first=0, keep_last=0)
    inp = gen.make_inputs(w, device="cuda")
    Kg = inp["Kg"].float()
    Kg = Kg * 1e-3
    Kg[:, :, :4] = inp["Kg"][:, :, :4].float() * 50
    inp["Kg"] = Kg.to(torch.bfloat16).contiguous()
    _run(w, inp)


@pytest.mark.parametrize("k", [1, 255, 256, 10_000])
def test_topk_bounds(k):
    w = replace(configs.get("c2s"), name=f"topk_{k}", top_k=k)
    _run(w, gen.make_inputs(w, device="cuda"))


@pytest.mark.parametrize("p", [1e-9, 0.5, 0.999999, 1.0])
def test_topp_bounds(p):
    w = replace(configs.get("c3s"), name=f"topp_{p}", top_p=p)
    _run(w, gen.make_inputs(w, device="cuda"))


def test_long_rows_topk():
    """Top-k over rows longer than the short-row limit (histogram path with unit weights):
    one summary row per token."""
    w = replace(configs.get("c2s"), name="long_topk", chunk_size=1, n_ctx=8192, top_k=700)
    _run(w, gen.make_inputs(w, device="cuda"))


def test_long_rows_topp_summary():
    """Top-p over long summary-routed rows (histogram path with softmax masses)."""
    w = replace(configs.get("c3s"), name="long_topp", batch=1, kv_batch=1, chunk_size=2, n_ctx=16384,
                keep_first=3, keep_last=5)
    _run(w, gen.make_inputs(w, device="cuda"))


@pytest.mark.parametrize("kind", ["proxy", "summary"])
def test_long_rows_odd_length(kind):
    """Long rows whose length is not a multiple of 8: the histogram pass takes its strided layout
    (8-byte loads, 2-byte bin stores) and the last slab and the last 8-entry piece are partial."""
    if kind == "proxy":
        w = replace(configs.get("c5s"), name="odd_proxy", n_ctx=40005, window=777, sink=5)
    else:
        w = replace(configs.get("c3s"), name="odd_summary", batch=1, kv_batch=1, chunk_size=2, n_ctx=16382,
                    keep_first=2, keep_last=3)
    _run(w, gen.make_inputs(w, device="cuda"))


@pytest.mark.parametrize("factor", [0.25, 2.0, 8.0])
def test_long_rows_bin_width(factor):
    """Proxy top-p rows with the selection scale multiplied by `factor`: coarse bins from about
    0.004 to 0.25 logit wide, so rows take the bin-edge Taylor weights (bins up to 1/16 logit),
    exp itself (wider bins), or a mix of both across the heads."""
    w0 = configs.get("c5s")
    w = replace(w0, name=f"bin_width_{factor}", n_ctx=32768, select_scale=w0.select_scale * factor)
    _run(w, gen.make_inputs(w, device="cuda"))


def test_token_topp_short_rows():
    """Token-level proxy top-p on rows short enough for the fused short-row kernel, mixed heads."""
    w = replace(configs.get("c5s"), name="tok_short", n_ctx=2048, window=100, sink=7)
    _run(w, gen.make_inputs(w, device="cuda"))


def test_only_local_heads():
    w = replace(configs.get("c5s"), name="local_only", n_ctx=16384, local_kv_heads=tuple(range(8)),
                sink=3, window=1111)
    _run(w, gen.make_inputs(w, device="cuda"))


def test_single_group_two_level_all_segments():
    """Two-level selection keeping every segment equals flat top-k."""
    w = replace(configs.get("c4s"), name="hier_all", top_k_seg=32, top_k=40)
    _run(w, gen.make_inputs(w, device="cuda"))


@pytest.mark.parametrize("blocks", [1, 7, 4096])
def test_attend_block_counts(blocks):
    """The attention result does not depend on how the tile sequence is cut into workgroups."""
    w = configs.get("c2s")
    inp = gen.make_inputs(w, device="cuda")
    _run(w, inp, attend_blocks=blocks)


def test_attend_many_partials_per_group():
    """One sequence with two KV groups cut into 4096 workgroups: about 2,000 partials per group,
    more than the combine's 1024 threads, so it takes several rounds of lse values and partial rows."""
    w = replace(configs.get("c3s"), name="c3s_two_groups", batch=1, kv_batch=1, n_q_heads=8, n_kv_heads=2)
    inp = gen.make_inputs(w, device="cuda")
    _run(w, inp, attend_blocks=4096)


@pytest.mark.parametrize("kind", ["proxy_topp", "summary_topp", "topk"])
def test_long_rows_all_tied(kind):
    """Long rows whose scores all tie: the crossing bin holds the whole row (more entries than the
    resolution buffer), and the selection is the lowest indices reaching the target."""
    if kind == "proxy_topp":
        w = replace(configs.get("c5s"), name="tie_long_proxy")
        inp = gen.make_inputs(w, device="cuda")
        inp["Kp"][:] = inp["Kp"][:, :, :1]
    elif kind == "summary_topp":
        w = replace(configs.get("c3s"), name="tie_long_summary", batch=1, kv_batch=1, chunk_size=2, n_ctx=16384,
                    keep_first=0, keep_last=0)
        inp = gen.make_inputs(w, device="cuda")
        inp["Kg"][:] = inp["Kg"][:, :, :1]
    else:
        w = replace(configs.get("c2s"), name="tie_long_topk", chunk_size=1, n_ctx=8192, top_k=5000)
        inp = gen.make_inputs(w, device="cuda")
        inp["Kg"][:] = inp["Kg"][:, :, :1]
    g, o = _run(w, inp)
    assert int(g["sel"]["status"][0]) == 0, "overflow flag set"


def test_two_handles_on_two_streams():
    """Two handles with their own workspaces, enqueued on two streams at once (both at the default
    priority), give bit for bit what each gives alone on the default stream."""
    from query_adaptive_sparse_amd import SparseDecoder
    cases = []
    for name in ("c3s", "c5s"):
        w = configs.get(name)
        inp = gen.make_inputs(w, device="cuda")
        alone = parity.run_gpu(w, inp)
        dec = SparseDecoder(device="cuda", **configs.library_params(w))
        dec.alloc_workspace()
        out = torch.full((w.batch, w.n_queries, w.n_q_heads, w.head_dim), float("nan"), device="cuda")
        lse = torch.full((w.batch, w.n_queries, w.n_q_heads), float("nan"), device="cuda")
        cases.append((w, inp, alone, dec, out, lse))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for rep in range(3):
        for (w, inp, _, dec, out, lse), s in zip(cases, streams):
            with torch.cuda.stream(s):
                dec.step(parity.lib_tensors(inp), out, lse)
    torch.cuda.synchronize()
    for w, inp, alone, dec, out, lse in cases:
        sel = dec.selection()
        assert torch.equal(sel["head_bits"].cpu(), alone["sel"]["head_bits"]), w.name
        assert torch.equal(sel["count"].cpu(), alone["sel"]["count"]), w.name
        o = out.cpu().numpy().reshape(alone["out"].shape)
        l_ = lse.cpu().numpy().reshape(alone["lse"].shape)
        assert np.array_equal(o, alone["out"]) and np.array_equal(l_, alone["lse"]), w.name
        print(f"[edge] {w.name}: concurrent run equals the run alone", flush=True)


DTYPE_DIM = [("c2s", dict(head_dim=64, softmax_scale=0.125)),
             ("c3s", dict(head_dim=64, softmax_scale=0.125, select_scale=0.125)),
             ("c2s", dict(head_dim=64, softmax_scale=0.125, n_queries=2)),  # 14 rows: two P.V MFMAs
             ("c2s", dict(dtype="f32", softmax_scale=128 ** -0.5)),
             ("c1s", dict(head_dim=128, softmax_scale=128 ** -0.5))]


@pytest.mark.parametrize("name,kw", DTYPE_DIM, ids=[f"{n}-{kw.get('dtype', 'bf16' if n != 'c1s' else 'f32')}"
                                                    f"-d{kw.get('head_dim', 128)}-T{kw.get('n_queries', 1)}"
                                                    for n, kw in DTYPE_DIM])
def test_dtype_and_head_dim(name, kw):
    """Every element type and head size the library is built for (bf16 / fp32 x d 64 / 128),
    against the oracle on reduced shapes."""
    w = replace(configs.get(name), name=f"{name}_dd", **kw)
    _run(w, gen.make_inputs(w, device="cuda"))


def _near_equal_proxy_inputs(w, kind):
    """c5s-shaped proxy inputs whose retrieval rows put the top-p crossing inside a crowd of
    near-equal scores. Every query is e_0 and every projection maps it to q_p = (1, 2^-11, 0, ...),
    so a token's proxy score is exactly kp[0] + 2^-11 kp[1]. A quarter of the tokens score about
    -60000 (they widen the row's range until one coarse bin spans every other token, and weigh
    nothing); the rest form the crowd:
      dense: kp[0] in 1 + {0..15} 2^-10 and kp[1] in 0.5 + {0..1023} 2^-11 by a seeded hash, up to
             16384 distinct scores within 0.016 of each other, about 49000 tokens;
      tied:  one score shared by about 49000 tokens, with 300 tokens just above it and 300 just
             below, so the crossing falls among exact ties far beyond the gather buffer."""
    inp = gen.make_inputs(w, device="cuda")
    Hq, Hk, d, N, r = w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx, w.route_dim
    q = torch.zeros_like(inp["q"])
    q[..., 0] = 1.0
    P = torch.zeros(Hk, d, r, dtype=torch.float32, device="cuda")
    P[:, 0, 0] = 1.0
    P[:, 0, 1] = 2.0 ** -11
    t = torch.arange(N, dtype=torch.int64, device="cuda")
    h = gen.hash32(w.seed, 99, t)
    low = (h & 3) == 0
    kp = torch.zeros(1, Hk, N, r, dtype=torch.float64, device="cuda")
    if kind == "dense":
        kp[0, :, :, 0] = 1.0 + ((h >> 2) & 15).double() * 2.0 ** -10
        kp[0, :, :, 1] = 0.5 + ((h >> 6) & 1023).double() * 2.0 ** -11
    else:
        sel = (h >> 8) % 1000
        kp[0, :, :, 0] = 1.0 + 2.0 ** -10
        kp[0, :, :, 0] = torch.where(sel < 6, 1.0 + 2.0 ** -9, kp[0, :, :, 0])
        kp[0, :, :, 0] = torch.where((sel >= 6) & (sel < 12), torch.ones_like(kp[0, :, :, 0]), kp[0, :, :, 0])
    kp[0, :, low, 0] = -60000.0
    kp[0, :, low, 1] = 0.0
    inp["q"], inp["P"], inp["Kp"] = q.contiguous(), P.contiguous(), kp.to(torch.float16).contiguous()
    return inp


@pytest.mark.parametrize("kind", ["dense", "tied"])
def test_long_rows_near_equal(kind):
    """Top-p over 64K-token proxy rows whose crossing coarse bin holds far more entries than the
    gather buffer: tens of thousands of distinct near-equal scores (dense), or a crossing among
    exact ties (tied). The selection is exact: bit-identical to the oracle, no status flag."""
    w = replace(configs.get("c5s"), name=f"near_equal_{kind}")
    inp = _near_equal_proxy_inputs(w, kind)
    s = inp["Kp"][0, 0, :, 0].double() + inp["Kp"][0, 0, :, 1].double() * 2.0 ** -11
    crowd = s > 0
    print(f"[edge] {w.name}: {int(crowd.sum())} crowd tokens, {int(torch.unique(s[crowd]).numel())} distinct "
          f"crowd scores", flush=True)
    g, o = _run(w, inp)
    assert int(g["sel"]["status"][0]) == 0
    for (b, gg), r in o["sel"].items():
        for hh, S in r["heads"].items():
            assert 1000 < len(S) < int(crowd.sum()), (hh, len(S))  # the crossing is inside the crowd


def test_selection_repeatable():
    """Twenty steps of the 16K top-p workload and of the near-equal proxy rows, each on its own
    fresh workspace: every selection bit and every output bit is the same every time (the bin
    masses are exact integer sums, so no atomic order reaches the result)."""
    cases = [(configs.get("c3s"), gen.make_inputs(configs.get("c3s"), device="cuda"))]
    w5 = replace(configs.get("c5s"), name="near_equal_dense")
    cases.append((w5, _near_equal_proxy_inputs(w5, "dense")))
    for w, inp in cases:
        first = parity.run_gpu(w, inp)
        for rep in range(19):
            again = parity.run_gpu(w, inp)
            for k in ("head_bits", "count"):
                assert torch.equal(first["sel"][k], again["sel"][k]), (w.name, rep, k)
            cnt = first["sel"]["count"]
            for bb in range(w.batch):
                for g in range(w.n_kv_heads):  # list entries past the count are unused workspace
                    n = int(cnt[bb, g])
                    assert torch.equal(first["sel"]["list"][bb, g, :n], again["sel"]["list"][bb, g, :n])
            assert np.array_equal(first["out"], again["out"]) and np.array_equal(first["lse"], again["lse"])
        print(f"[edge] {w.name}: 20 runs bit-identical", flush=True)
