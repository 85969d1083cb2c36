"""Benchmark: query-adaptive sparse decode attention on one MI355X.

One step = score -> select -> attend -> combine for every sequence and head of
the 128K-context top-p workload (4 sequences, 32 query / 8 KV heads, d = 128,
bf16, chunks of 64, top-p 0.95 over the chunk-score softmax with the first and
last chunk forced), inputs resident in HBM.

Prints one JSON line. ``value`` is queries/s (one query = one sequence's decode
position over all heads of one layer); the line also carries the step's
algorithmic HBM bandwidth, a live roofline of the attention kernel and the fp64
CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBPS = 8000.0

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-groups", type=int, default=0, help="0 = size the sample to ~10-30 s")
    ap.add_argument("--attend-blocks", type=int, default=None)
    ap.add_argument("--flush-mib", type=int, default=0, metavar="MIB",
                    help="before every timed step, overwrite a MIB MiB buffer (evicts the L2s and the "
                         "256 MB Infinity Cache); steps are then timed by events only, flush excluded")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run torch device-to-device copies of MIB MiB (counter calibration)")
    return ap.parse_args()


def copy_calibration(mib: int, reps: int = 5):
    """Plain device copies of a known size: the reference reading for HBM byte counters."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "reps": reps}), flush=True)


def algorithmic_bytes(w, counts: np.ndarray) -> dict:
    """Bytes the step must move, from the run's own selection sizes.

    counts[b, g] = entries in group (b, g)'s union (chunks, or tokens at chunk 1).
    """
    e = w.elem_bytes
    d, C, B, Hq = w.head_dim, w.chunk_size, w.batch, w.n_q_heads * w.n_queries  # query rows per sequence
    U = int(counts.sum())
    raw_kv = U * C * d * e * 2                        # selected raw K and V
    if w.mode == "proxy":
        local = [g for g in range(w.n_kv_heads) if g in w.local_kv_heads]
        retr = w.n_kv_heads - len(local)
        routing = w.kv_batch * retr * w.n_ctx * w.route_dim * 2 + retr * d * w.route_dim * 4
        sum_v = sum_k_sel = 0
    elif w.mode == "hier":
        routing = w.kv_batch * w.n_kv_heads * w.n_segments * d * e  # meta keys
        routing += B * Hq * min(w.top_k_seg, w.n_segments) * w.seg_size * d * e  # candidate summary keys
        sum_v = U * d * e
        sum_k_sel = U * d * e
    else:
        routing = w.kv_batch * w.n_kv_heads * w.n_chunks * d * e  # every summary key
        n_sum = B * w.n_kv_heads * w.n_chunks if w.all_summaries else U  # summary rows attended
        sum_v = n_sum * d * e if w.attend_summary else 0
        sum_k_sel = n_sum * d * e if w.attend_summary else 0
    q_out = B * Hq * d * (e + 4)
    step = routing + raw_kv + sum_v + q_out
    attend = raw_kv + sum_v + sum_k_sel + B * Hq * d * e + U * 4  # + list
    return {"step": step, "attend": attend, "routing": routing, "raw_kv": raw_kv, "entries": U}


class _OracleClock:
    """Wall and process CPU time of the timed oracle calls. Their ratio is the number of host threads
    the oracle actually kept busy: numpy's elementwise loops run on one, its BLAS calls on the pool."""

    def __init__(self):
        self.wall = self.cpu = 0.0

    def __enter__(self):
        self._w, self._c = time.perf_counter(), time.process_time()
        return self

    def __exit__(self, *exc):
        self.wall += time.perf_counter() - self._w
        self.cpu += time.process_time() - self._c

    def cores(self) -> float:
        return round(self.cpu / self.wall, 1) if self.wall > 0 else 1.0


def _blas_pool() -> int:
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])


def cpu_baseline(w, inp, target_s=15.0, max_groups=0):
    """The fp64 oracle (as it stands) on whole (sequence, KV group) units of the same workload:
    units in a fixed random order, cycling over the step until about target_s of CPU time."""
    from oracle import HostSource, ref

    groups = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
    rng = np.random.default_rng(0)
    order = [groups[i] for i in rng.permutation(len(groups))]
    # host copies of the inputs (PCIe time is not oracle time)
    host = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in inp.items()}
    src = HostSource(host)
    done, clk = 0, _OracleClock()
    margin = float("inf")
    while True:
        b, g = order[done % len(order)]
        with clk:
            r = ref.select_group(w, src, b, g)
            ref.attend_group(w, src, b, g, r["union"], r["heads"])
        margin = min(margin, r["margin"])
        t_total = clk.wall
        done += 1
        if (max_groups and done >= max_groups) or (not max_groups and t_total >= target_s):
            break
    per_group = t_total / done
    step_s = per_group * len(groups)
    return {"value": round(w.batch * w.n_queries / step_s, 4), "unit": "queries/s", "cores": clk.cores(), "kind": "oracle",
            "sample": f"{done} (sequence, KV group) units of {w.name} ({len(groups)} per step, cycled): "
                      f"selection + attention, {t_total:.1f} s, scaled to a full step ({step_s:.2f} s); "
                      f"cores = process CPU time / wall time (BLAS pool {_blas_pool()} threads)",
            "min_selection_margin": None if margin == float("inf") else float(f"{margin:.3g}"),
            **_host_info()}


def _host_info() -> dict:
    """The host the oracle ran on: CPU model, logical CPUs and the ones this process may use."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu": _cpu_model(), "nproc": os.cpu_count(), "affinity_cpus": affinity}


COUNTER_PROFILE = os.path.join(ROOT, "profiles", "c3_128k_attend_counters.md")


def counter_traffic(workload: str, attend_blocks: int):
    """HBM bytes per attention launch from the committed FETCH_SIZE / WRITE_SIZE summary, scaled by
    its copy calibration; None when the summary is for another workload or launch shape, or when
    the attention sources have changed since the counters were taken."""
    import hashlib
    import re

    try:
        text = open(COUNTER_PROFILE).read()
        rec = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
        h = hashlib.sha256()
        for s in rec["sources"]:
            with open(os.path.join(ROOT, s), "rb") as f:
                h.update(f.read())
    except (OSError, AttributeError, KeyError, ValueError):
        return None
    if rec["workload"] != workload or rec["attend_blocks"] != attend_blocks or h.hexdigest() != rec["sources_sha256"]:
        return None
    return int(round(rec["fetch_kib_per_dispatch"] * 1024 * rec["fetch_factor"]
                     + rec["write_kib_per_dispatch"] * 1024 * rec["write_factor"]))


def prefill_cpu_baseline(w, inp, sel, target_s=15.0):
    """The fp64 prefill oracle (as it stands) on a bounded sample: one head's proxy-map importance
    and the compressed attention of sampled query rows of one sparse head (and of one full-attention
    head, if the routing has any; the oracle's per-row cost grows with the row's causal range, so
    rows are drawn uniformly over the head's sequence), scaled to a full layer (every head's
    importance, every head's rows)."""
    from oracle import PrefillSource, pref

    src = PrefillSource({k: (v.cpu() if torch.is_tensor(v) else v) for k, v in inp.items() if k in ("Q", "K", "V")})
    L, W = w.seq_len, w.window
    modes = pref.head_modes(w)
    clk = _OracleClock()
    with clk:
        pref.proxy_importance(src.q_rows(0, 0, np.arange(L - W, L)), src.k_all(0, 0), w.softmax_scale, L - W)
    t_imp = clk.wall
    k = int(sel["budget"][0])
    kinds = [m for m in (0, 1) if m in modes]
    rng = np.random.default_rng(0)
    step_s, notes = w.batch * w.n_q_heads * t_imp, []
    for m in kinds:
        h = modes.index(m)
        n = L if m else k
        S = sel["list"][0, h, :n].cpu().numpy().astype(np.int64)
        done, t_rows = 0, 0.0
        while t_rows < target_s / len(kinds) and done < n:
            i = int(rng.integers(0, n))
            w0 = clk.wall
            with clk:
                pref.tsa_attend_rows(w, src, 0, h, S, [i])
            t_rows += clk.wall - w0
            done += 1
        step_s += w.batch * modes.count(m) * n * t_rows / done
        notes.append(f"{done} of {n} attention rows of {'full' if m else 'sparse'} head {h} ({t_rows:.1f} s)")
    return {"value": round(w.batch * L / step_s, 4), "unit": "prompt tokens/s", "cores": clk.cores(), "kind": "oracle",
            "sample": f"{w.name}: importance of 1 of {w.batch * w.n_q_heads} heads ({t_imp:.1f} s), "
                      + ", ".join(notes) + f"; scaled to a full layer ({step_s:.0f} s); cores = process CPU "
                      f"time / wall time (BLAS pool {_blas_pool()} threads)",
            **_host_info()}


def bench_prefill(args, w):
    """Token-Sparse prefill layer: select (proxy map, budget, per-head top-k) then compressed causal
    attention, over a seeded synthetic prompt resident in HBM."""
    from synth import gen
    from query_adaptive_sparse_amd import SparsePrefill, make_prefill_tensors

    torch.cuda.init()
    dev = torch.device("cuda:0")
    print(f"[bench] prefill workload {w.name}: generating inputs on {torch.cuda.get_device_name(0)}",
          file=sys.stderr, flush=True)
    inp = gen.make_prefill_inputs(w, device=dev)
    sp = SparsePrefill(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                       seq_len=w.seq_len, window=w.window, tau=w.tau, softmax_scale=w.softmax_scale, device=dev)
    sp.alloc_workspace()
    hm = None if w.head_mode is None else torch.tensor(w.head_mode, dtype=torch.int8, device=dev)
    t = make_prefill_tensors(inp["Q"], inp["K"], inp["V"], head_mode=hm)
    out = torch.empty(w.batch, w.n_q_heads, w.seq_len, w.head_dim, dtype=torch.float32, device=dev)
    warm, K = max(1, min(args.warmup, 3)), max(1, min(args.steps, 10))
    for _ in range(warm):
        sp.step(t, out)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({warm} steps)", file=sys.stderr, flush=True)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        sp.select(t)
        ev[i][1].record()
        sp.attend(t, out)
        ev[i][2].record()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / K
    select_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    attend_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    print(f"[bench] timed {K} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)
    sel = sp.selection()
    budgets = sel["budget"].cpu().numpy().astype(np.int64)
    status = int(sel["status"].cpu().numpy()[0])
    # useful attention flops: per head, causal compact attention over k tokens (every token for a
    # full-attention head), 2 (q.k) + 2 (p.v) flops per (query, key, dimension)
    modes = list(w.head_mode) if w.head_mode is not None else [0] * w.n_q_heads
    flops = float(sum((w.seq_len if m else kk) * ((w.seq_len if m else kk) + 1) // 2 * w.head_dim * 4
                      for kk in budgets for m in modes))
    tflops = flops / (attend_ms * 1e-3) / 1e12
    line = {
        "metric": ("token-sparse prefill attention prompt tokens/s at 128K ctx" if w.head_mode is None else
                   "mixed full / token-sparse head prefill attention prompt tokens/s at 128K ctx"),
        "value": round(w.batch * w.seq_len / (ms_per_step * 1e-3), 2),
        "unit": "prompt tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based N(0,1) Q, K, V with a planted Zipf key-importance profile per KV group)",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "context": w.seq_len, "window": w.window, "tau": w.tau,
                   "full_attention_heads": sum(modes)},
        "budget_tokens": budgets.tolist(),
        "stages_ms": {"select": round(select_ms, 4), "attend": round(attend_ms, 4),
                      "note": "attend = zero rows for unkept positions + compressed attention"},
        "roofline": {"kernel": "k_pf_attend (compressed causal attention)", "bound": "mfma",
                     "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": None, "flops_per_launch": flops,
                     "avg_launch_ms": round(attend_ms, 4)},
        "status_flags": status,
    }
    if not args.no_cpu_baseline:
        print("[bench] prefill cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = prefill_cpu_baseline(w, inp, sel)
    print(json.dumps(line), flush=True)


def gist_pairs(w) -> int:
    """(query, visible key) pairs of one head of a gist-masked layer: raw token t sees t // C gists
    and t % C + 1 raw tokens, gist m sees m + 1 gists and C raw tokens."""
    C, M = w.chunk_size, w.n_chunks
    return C * M * (M - 1) // 2 + M * C * (C + 1) // 2 + M * (M + 1) // 2 + M * C


def gist_cpu_baseline(w, inp, target_s=15.0):
    """The fp64 gist-prefill oracle (as it stands) on a bounded sample: query rows of one head drawn
    uniformly over the raw tokens and the gists, scaled to a full layer (every head, every row)."""
    from oracle import GistPrefillSource, gref

    src = GistPrefillSource({k: inp[k].cpu() for k in ("Q", "K", "V", "Qg", "Kg", "Vg")})
    rng = np.random.default_rng(0)
    n_rows = w.n_tokens + w.n_chunks
    done, clk = 0, _OracleClock()
    while clk.wall < target_s and done < n_rows:
        i = int(rng.integers(0, n_rows))
        kind, row = ("raw", i) if i < w.n_tokens else ("gist", i - w.n_tokens)
        with clk:
            gref.gp_attend_rows(w, src, 0, 0, kind, [row])
        done += 1
    t_rows = clk.wall
    step_s = w.batch * w.n_q_heads * n_rows * t_rows / done
    return {"value": round(w.batch * w.n_tokens / step_s, 4), "unit": "prompt tokens/s", "cores": clk.cores(),
            "kind": "oracle",
            "sample": f"{w.name}: {done} of {n_rows} query rows (raw and gist, uniform) of 1 of "
                      f"{w.batch * w.n_q_heads} heads ({t_rows:.1f} s), scaled to a full layer ({step_s:.0f} s); "
                      f"cores = process CPU time / wall time (BLAS pool {_blas_pool()} threads)",
            **_host_info()}


def bench_gist(args, w):
    """Gist-masked (SSA) prefill layer: every raw and gist query over its visible keys (a gist prefix
    and its chunk's raw run), over a seeded synthetic prompt resident in HBM."""
    from synth import gen
    from query_adaptive_sparse_amd import GistPrefill, make_gist_tensors

    torch.cuda.init()
    dev = torch.device("cuda:0")
    print(f"[bench] gist prefill workload {w.name}: generating inputs on {torch.cuda.get_device_name(0)}",
          file=sys.stderr, flush=True)
    inp = gen.make_gist_inputs(w, device=dev)
    gp = GistPrefill(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                     n_tokens=w.n_tokens, chunk_size=w.chunk_size, softmax_scale=w.softmax_scale)
    t = make_gist_tensors(inp["Q"], inp["K"], inp["V"], inp["Qg"], inp["Kg"], inp["Vg"])
    out = torch.empty(w.batch, w.n_q_heads, w.n_tokens, w.head_dim, dtype=torch.float32, device=dev)
    outg = torch.empty(w.batch, w.n_q_heads, w.n_chunks, w.head_dim, dtype=torch.float32, device=dev)
    warm, K = max(1, args.warmup), max(1, min(args.steps, 200))
    for _ in range(warm):
        gp.attend(t, out, outg)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({warm} steps)", file=sys.stderr, flush=True)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        gp.attend(t, out, outg)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / K
    attend_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    print(f"[bench] timed {K} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)
    # useful flops: 2 (q.k) + 2 (p.v) per (query, visible key, dimension)
    flops = float(w.batch * w.n_q_heads * gist_pairs(w) * w.head_dim * 4)
    tflops = flops / (attend_ms * 1e-3) / 1e12
    dense = float(w.batch * w.n_q_heads * (w.n_tokens + w.n_chunks) * (w.n_tokens + w.n_chunks + 1) // 2
                  * w.head_dim * 4)
    line = {
        "metric": "gist-masked (SSA) prefill attention prompt tokens/s at 32K ctx",
        "value": round(w.batch * w.n_tokens / (ms_per_step * 1e-3), 2),
        "unit": "prompt tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based N(0,1) raw and gist Q, K, V)",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "context": w.n_tokens, "chunk_size": w.chunk_size,
                   "gists": w.n_chunks},
        "useful_fraction_of_dense": round(flops / dense, 4),
        "roofline": {"kernel": "k_gp_attend (gist-masked block-sparse attention)", "bound": "mfma",
                     "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": None, "flops_per_launch": flops,
                     "avg_launch_ms": round(attend_ms, 4)},
    }
    if not args.no_cpu_baseline:
        print("[bench] gist prefill cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = gist_cpu_baseline(w, inp)
    print(json.dumps(line), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the decode path "
              "shards by sequence and KV group across GPUs, which this benchmark does not run)", file=sys.stderr)
        sys.exit(2)
    from synth import configs, gen
    from query_adaptive_sparse_amd import SparseDecoder, make_tensors

    if args.workload in configs.PREFILL:
        return bench_prefill(args, configs.get(args.workload))
    if args.workload in configs.GIST:
        return bench_gist(args, configs.get(args.workload))
    w = configs.get(args.workload) if args.workload else configs.BENCH
    params = configs.library_params(w)
    if args.attend_blocks is not None:
        params["attend_blocks"] = args.attend_blocks
    torch.cuda.init()
    dev = torch.device("cuda:0")
    print(f"[bench] workload {w.name}: generating inputs on {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    inp = gen.make_inputs(w, device=dev)
    dec = SparseDecoder(device=dev, **params)
    dec.alloc_workspace()
    t = make_tensors(inp["q"], inp["K"], inp["V"], Kg=inp.get("Kg"), Vg=inp.get("Vg"), Kmg=inp.get("Kmg"),
                     Kp=inp.get("Kp"), P=inp.get("P"))
    out = torch.empty(w.batch, w.n_queries, w.n_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    lse = torch.empty(w.batch, w.n_queries, w.n_q_heads, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        dec.step(t, out, lse)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # timed steps, each one sparse_decode_step call. The attention launch is bracketed by events
    # (on the stream the library launches on) on every `stride`-th timed step, which then runs the
    # stages as separate calls: an event pair adds ~6 us of idle time to its step, so it is recorded
    # on a sample of about five steps rather than on every step; the per-stage breakdown is taken
    # in a separate, untimed loop below.
    K = args.steps
    stride = max(1, K // 5)
    sampled = [i for i in range(K) if i % stride == 0]
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in sampled}
    scratch = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev) if args.flush_mib else None
    fl = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)] if scratch is not None else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = ev.get(i)
        if scratch is not None:
            scratch.fill_(i & 0xFF)
            fl[i][0].record()
        if e is None:
            dec.step(t, out, lse)  # the whole step in one library call
        else:
            for level in range(dec.levels):
                dec.score_chunks(t, level)
                dec.select(level)
            e[0].record()
            dec.attend(t)
            e[1].record()
            dec.combine(out, lse)
        if scratch is not None:
            fl[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    if scratch is not None:  # the flush is not part of the step
        ms_per_step = float(np.mean([f[0].elapsed_time(f[1]) for f in fl]))
    attend_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev.values()]))
    print(f"[bench] timed {K} steps: {ms_per_step:.4f} ms/step", file=sys.stderr, flush=True)

    # per-stage breakdown and per-step latency distribution (not part of the timed region)
    KS = min(K, 20)
    sv = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(KS)]
    for i in range(KS):
        e = sv[i]
        e[0].record()
        for level in range(dec.levels):
            dec.score_chunks(t, level)
            dec.select(level)
        e[1].record()
        dec.attend(t)
        e[2].record()
        dec.combine(out, lse)
        e[3].record()
    ps = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(K):
        ps[i][0].record()
        dec.step(t, out, lse)
        ps[i][1].record()
    torch.cuda.synchronize()
    route_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in sv]))
    combine_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in sv]))
    step_ev = np.array([e[0].elapsed_time(e[1]) for e in ps])
    pct = {f"p{q}": round(float(np.percentile(step_ev, q)), 5) for q in (10, 50, 90)}

    sel = dec.selection()
    counts = sel["count"].cpu().numpy()
    status = sel["status"].cpu().numpy()
    nb = algorithmic_bytes(w, counts)
    qps = w.batch * w.n_queries / (ms_per_step * 1e-3)  # a query: one token of one sequence, all heads
    step_gbps = nb["step"] / (ms_per_step * 1e-3) / 1e9
    attend_gbps = nb["attend"] / (attend_ms * 1e-3) / 1e9

    line = {
        "metric": "sparse decode attn queries/s + achieved HBM GB/s (% peak) at 128K ctx",
        "value": round(qps, 2),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded counter-based N(0,1) inputs with a planted Zipf chunk-mass profile)",
        "config": {"workload": w.name, "batch": w.batch, "n_queries": w.n_queries, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "context": w.n_ctx, "chunk": w.chunk_size, "mode": w.mode,
                   "top_p": w.top_p if w.mode in ("topp", "proxy") else None,
                   "top_k": w.top_k or None, "attend_blocks": dec.attend_blocks,
                   "cache_flush_mib": args.flush_mib},
        "hbm_gbps": round(step_gbps, 1),
        "hbm_frac": round(step_gbps / HBM_PEAK_GBPS, 4),
        "step_bytes": nb["step"],
        "selected_entries": nb["entries"],
        "stages_ms": {"score_select": round(route_ms, 4), "attend": round(attend_ms, 4),
                      "combine": round(combine_ms, 4), "note": "score_select and combine from a separate "
                      "event-bracketed loop; attend from every %d-th timed step (%d launches)" % (stride, len(ev))},
        "step_ms_events": {**pct, "steps": K, "note": "one event pair around each whole step, separate loop"},
        "roofline": {"kernel": "k_attend (gathered split-K attention)", "bound": "hbm",
                     "achieved": round(attend_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(attend_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": counter_traffic(w.name, dec.attend_blocks),
                     "bytes_per_launch": nb["attend"], "avg_launch_ms": round(attend_ms, 5),
                     "timed_launches": len(ev)},
        "status_flags": int(status[0]),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on a host sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, inp, max_groups=args.cpu_sample_groups)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
