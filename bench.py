"""Throughput of the DSA hot path on one MI355X.

One step = the whole path over one batch: lightning-indexer scores, per-row
top-k, then sparse MLA on every layer (one full layer, plus IndexShare layers
where the workload has them).  Inputs are seeded synthetic tensors already
resident in HBM; several independent input sets are rotated so the 256 MB
MALL cannot serve repeat reads.

Default workload (decode128): 256 decode requests, contexts U[2048, 32768],
one query each, index_topk 2048, indexer 64 x 128 bf16, sparse MLA with all
128 heads over a 512+64 bf16 paged latent cache (page size 64, random page
tables), one full layer followed by two IndexShare layers that reuse its
indices -- batch-256 steady decode, the largest decode workload that runs on
one GPU.  `--config N` benchmarks another workload of the same family
instead (1: the 16-head per-GPU share of tensor-parallel decode, 3: a
chunked prefill, 4: long-context fp8 MTP decode).

Prints one JSON line.  `value` is query rows through the whole path per
second; `roofline` reports the dominant kernel against MI355X's HBM (8 TB/s)
or dense bf16 MFMA (2.5 PFLOP/s) peak, with its average duration taken from
HIP events on the launch stream inside the timed region; `cpu_baseline` is
the CPU oracle on a bounded sample of the same workload.  Exactly `--steps`
steps are timed, each a replay of one input set's captured step, with an
event between consecutive steps: `step_ms` gives their median, p10 and p90.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-MLA decode queries/s + indexer top-k rows/s; % HBM / MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0
MFMA_FP8_PEAK_TFS = 5000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated (0 = auto)")
    ap.add_argument("--mode", default="perf", choices=["perf", "parity"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--prep", action="store_true",
                    help="each step starts with the indexer preparation (query RoPE, key LayerNorm "
                         "and RoPE, paged key store)")
    ap.add_argument("--score-budget", type=float, default=None, metavar="MB",
                    help="scores + top-k through dsa_index_topk with a score workspace of at most "
                         "this many MB (query rows in chunks) instead of a [T, ld] score buffer")
    ap.add_argument("--kv", choices=["bf16", "fp8", "int8"], default=None,
                    help="latent cache format instead of the workload's own (fp8: e4m3 with a scale "
                         "per 128 dims; int8: affine codes with a scale and bias per 128 dims)")
    ap.add_argument("--key-fp8", action="store_true",
                    help="indexer keys cached as e4m3 codes with one f32 scale per token "
                         "(queries stay bf16); reports the top-k overlap with bf16 keys")
    ap.add_argument("--q-fp8", action="store_true",
                    help="with --key-fp8: the indexer's queries are quantised per (row, head) to e4m3 "
                         "at a power-of-two scale and contracted on the fp8 matrix cores")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (f32 multiply by 1) four times, the "
                         "reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


# HBM traffic of the dominant kernel per launch, from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE) over `bench.py --no-cpu --steps 8 --warmup 2`,
# each counter scaled by bytes / counter-bytes of the copy calibration kernel.
# Keyed by (workload name, stage); `src` is the sha256 of the kernel's sources when the
# counters were taken -- a changed kernel reports traffic null.
# Copy calibration of those runs: FETCH_SIZE x 2.000, WRITE_SIZE x 1.000.
TRAFFIC = {
    ("decode128", "index_scores"): {"src": "ed9bbcfdbb2c6e95", "fetch_bytes": 1153000000.0, "write_bytes": 17840000.0, "dispatches": 50},
    ("decode128", "sparse_mla"): {"src": "94deeeeeb4ee34d3", "fetch_bytes": 645700000.0, "write_bytes": 33690000.0, "dispatches": 150},
    ("decode128", "topk"): {"src": "fe973313bb18ed5f", "fetch_bytes": 18690000.0, "write_bytes": 2097000.0, "dispatches": 50},
    ("decode16", "index_scores"): {"src": "ed9bbcfdbb2c6e95", "fetch_bytes": 81190000.0, "write_bytes": 1182000.0, "dispatches": 49},
    ("decode16", "sparse_mla"): {"src": "94deeeeeb4ee34d3", "fetch_bytes": 157000000.0, "write_bytes": 5290000.0, "dispatches": 49},
    ("decode16", "topk"): {"src": "fe973313bb18ed5f", "fetch_bytes": 2290000.0, "write_bytes": 524300.0, "dispatches": 49},
    ("mtp_fp8", "index_scores"): {"src": "ed9bbcfdbb2c6e95", "fetch_bytes": 848200000.0, "write_bytes": 64380000.0, "dispatches": 43},
    ("mtp_fp8", "sparse_mla"): {"src": "94deeeeeb4ee34d3", "fetch_bytes": 345800000.0, "write_bytes": 63350000.0, "dispatches": 43},
    ("mtp_fp8", "topk"): {"src": "fe973313bb18ed5f", "fetch_bytes": 85520000.0, "write_bytes": 11800000.0, "dispatches": 43},
    ("prefill", "index_scores"): {"src": "ed9bbcfdbb2c6e95", "fetch_bytes": 885400000.0, "write_bytes": 302100000.0, "dispatches": 50},
    ("prefill", "sparse_mla"): {"src": "94deeeeeb4ee34d3", "fetch_bytes": 5241000000.0, "write_bytes": 539000000.0, "dispatches": 50},
    ("prefill", "topk"): {"src": "fe973313bb18ed5f", "fetch_bytes": 335800000.0, "write_bytes": 33550000.0, "dispatches": 50},
}
KERNEL_SOURCES = {"sparse_mla": ["sparse_mla.hip", "dsa_device.h"],
                  "index_scores": ["index_scores.hip", "dsa_device.h"],
                  "topk": ["topk.hip", "topk_select.h", "dsa_device.h"]}


def source_digest(stage):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[stage]:
        with open(os.path.join(ROOT, "sparse_attention_07_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic(workload, stage):
    """Measured HBM bytes per launch (fetch + write), or None if not measured for
    this workload or the kernel's sources changed since."""
    tr = TRAFFIC.get((workload, stage))
    if tr is None or tr["src"] != source_digest(stage):
        return None
    return tr["fetch_bytes"] + tr["write_bytes"]


def copy_calibration():
    n = 1 << 28                                    # 2^28 f32 = 1 GiB read + 1 GiB written
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"read_bytes": 4 * n, "write_bytes": 4 * n, "launches": 4}}),
          flush=True)


def measured_stream_peak():
    """Bytes/s a plain 1 GiB f32 multiply (read + write) reaches on this GPU: the
    practical HBM stream rate, reported beside the published peak."""
    n = 1 << 28
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(10):
        torch.mul(src, 1.0, out=dst)
    b.record()
    torch.cuda.synchronize()
    rate = 2 * 4 * n * 10 / (a.elapsed_time(b) / 1e3)
    del src, dst
    torch.cuda.empty_cache()
    return rate


def algorithmic(sb, path):
    """Algorithmic bytes / flops per launch of each stage (what the method must move)."""
    cfg = sb.cfg
    T, K = sb.T, cfg.topk
    pos = np.array(sb.positions(), dtype=np.int64)
    n_scored = int((pos + 1).sum())
    idx_es = 2 if cfg.idx_fmt == 1 else 4
    q_es = 2 if cfg.q_fmt == 1 else 4
    # a cached key: di elements, or di e4m3 codes plus one f32 scale
    key_bytes = cfg.di + 4 if cfg.key_fmt == 2 else cfg.di * idx_es
    st = {}
    st["index_scores"] = dict(
        bytes=int(sum(sb.seq_lens)) * key_bytes + T * cfg.hi * cfg.di * idx_es + T * cfg.hi * 4
        + n_scored * 4,
        flops=n_scored * 2 * cfg.hi * cfg.di)
    st["topk"] = dict(bytes=n_scored * 4 + T * K * 4, flops=0)
    st["index_topk"] = dict(bytes=st["index_scores"]["bytes"] + st["topk"]["bytes"],
                            flops=st["index_scores"]["flops"])
    if path.prep is not None:
        pr = path.prep
        # queries read and written, keys read and stored, two table rows per row, LayerNorm params
        st["indexer_prepare"] = dict(
            bytes=2 * T * cfg.hi * cfg.di * idx_es + 2 * T * cfg.di * idx_es + T * pr.rope_dim * 4
            + 2 * cfg.di * 4, flops=0)
    from sparse_attention_07_amd.synth import kv_row_bytes
    row = kv_row_bytes(cfg.kv_fmt, cfg.dc, cfg.dr)
    idx = path.idx.cpu().numpy()
    union = 0
    n_valid = int((idx >= 0).sum())
    cu = np.cumsum([0] + sb.q_lens)
    for b in range(sb.B):
        sel = idx[cu[b]:cu[b + 1]]
        union += len(np.unique(sel[sel >= 0]))
    per_layer_bytes = union * row + T * cfg.heads * (cfg.dc + cfg.dr) * q_es \
        + T * cfg.heads * cfg.dc * q_es + T * cfg.heads * 4
    st["sparse_mla"] = dict(bytes=per_layer_bytes * len(sb.q),
                            flops=n_valid * cfg.heads * 2 * (cfg.dc + cfg.dr + cfg.dc) * len(sb.q),
                            launches_per_step=len(sb.q))
    return st


def key_fp8_overlap(path, cfg_id, mode):
    """Mean fraction of each row's selected tokens that stay selected when the
    same key draws are cached in bf16 instead of fp8 (input set 0)."""
    from sparse_attention_07_amd import synth
    from sparse_attention_07_amd.path import DSAPath
    sb = synth.make_batch(cfg_id, mode=mode, device=path.sb.q_idx.device, layers=0)
    # with the preparation in the step, both sides rotate the same queries and store the same keys
    ref = DSAPath(sb, prep=synth.make_prep(sb, seed=4242) if path.prep is not None else None)
    if ref.prep is not None:
        ref.indexer_prepare()
        path.indexer_prepare()
    ref.index_scores()
    ref.topk()
    path.index_scores()
    path.topk()
    torch.cuda.synchronize()
    a, b = path.idx.cpu().numpy(), ref.idx.cpu().numpy()
    frac = []
    for x, y in zip(a, b):
        x, y = x[x >= 0], y[y >= 0]
        frac.append(len(np.intersect1d(x, y)) / max(1, len(y)))
    return float(np.mean(frac))


def cpu_model():
    """The host CPU as /proc/cpuinfo names it (first processor: model name, family and
    model numbers), with the logical CPUs this process may use and the total."""
    f = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if not line.strip():
                    break
                k, _, v = line.partition(":")
                f[k.strip()] = v.strip()
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return "%s (family %s, model %s, stepping %s; %d of %d logical CPUs usable)" % (
        f.get("model name", "unknown"), f.get("cpu family", "?"), f.get("model", "?"), f.get("stepping", "?"),
        usable, os.cpu_count() or 0)


def _oracle_rate(sb, threads, budget_s):
    """Query rows per second of the oracle's whole path over rows of `sb`, on
    `threads` threads, in chunks of one row per thread until about budget_s."""
    import oracle
    oracle.set_threads(threads)
    order = np.random.default_rng(0).permutation(sb.T)
    t0 = time.perf_counter()
    done = 0
    while time.perf_counter() - t0 < budget_s:
        for i in range(0, sb.T, threads):
            oracle.run_path(sb, rows=sorted(order[i:i + threads].tolist()))
            done += len(order[i:i + threads])
            if time.perf_counter() - t0 > budget_s:
                break
    return done, time.perf_counter() - t0


def cpu_baseline(sb, budget_s=20.0, one_thread_s=6.0):
    """The oracle on a bounded sample of the same workload: rows of the first
    input set (its tensors stay on the GPU; the oracle copies the pages of the
    requests that own each chunk's rows to the host), through scores, top-k and
    every layer, on all host threads; then a short 1-thread run."""
    import oracle
    cores = oracle.threads()
    done, dt = _oracle_rate(sb, cores, budget_s)
    done1, dt1 = _oracle_rate(sb, 1, one_thread_s)
    oracle.set_threads(cores)
    layers = len(sb.q)
    return {"value": done / dt, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "%d query rows of one %d-row %s batch through the whole path (scores, top-k, "
                      "%d MLA layer%s) in float64 on %d threads, %.1f s"
                      % (done, sb.T, sb.cfg.name, layers, "s" if layers > 1 else "", cores, dt),
            "one_thread": {"value": done1 / dt1, "unit": "queries/s",
                           "sample": "%d query rows, same path, 1 thread, %.1f s" % (done1, dt1)}}


def spread(xs):
    """Median, p10 and p90 of a list of times (ms)."""
    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.q_fp8 and not args.key_fp8:
        print("--q-fp8 contracts fp8 queries with fp8 keys: add --key-fp8", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    from sparse_attention_07_amd import synth
    from sparse_attention_07_amd.path import DSAPath

    cfg_id = args.config
    base = synth.CONFIGS[cfg_id]
    # independent input sets rotated so that the 256 MB MALL cannot serve
    # repeat reads (decode16's and mtp_fp8's per-step data would fit in it)
    sets = args.sets or {0: 1, 1: 8, 2: 1, 3: 1, 4: 2}[cfg_id]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    paths = []
    for i in range(sets):
        sb = synth.make_batch(cfg_id, mode=args.mode, device=dev, seed_offset=i,
                              key_fmt=synth.FMT_FP8_E4M3_B128 if args.key_fp8 else None,
                              kv_fmt=None if args.kv is None else
                              {"bf16": synth.FMT_BF16, "fp8": synth.FMT_FP8_E4M3_B128,
                               "int8": synth.FMT_INT8_AFFINE_B128}[args.kv])
        paths.append(DSAPath(sb, prep=synth.make_prep(sb, seed=4242 + i) if args.prep else None,
                             score_budget=None if args.score_budget is None
                             else int(args.score_budget * 2 ** 20), q_fp8=args.q_fp8))
    workload = (base.name + ("+fp8keys" if args.key_fp8 else "") + ("+fp8q" if args.q_fp8 else "")
                + ("+prep" if args.prep else "")
                + ("+kv-" + args.kv if args.kv is not None else "")
                + ("+budget" if args.score_budget is not None else ""))
    torch.cuda.synchronize()

    stages = ((["indexer_prepare"] if args.prep else [])
              + (["index_topk"] if args.score_budget is not None else ["index_scores", "topk"])
              + ["sparse_mla"])

    def run_stage(p, s):
        if s == "indexer_prepare":
            p.indexer_prepare()
        elif s == "index_topk":
            p.index_topk()
        elif s == "index_scores":
            p.index_scores()
        elif s == "topk":
            p.topk()
        else:
            for layer in range(len(p.kv)):
                p.mla(layer)

    for i in range(args.warmup):
        paths[i % sets].step()
    torch.cuda.synchronize()

    # Eager loop with events around every stage (includes host launch gaps).
    stream = torch.cuda.current_stream()
    ev = {s: [] for s in stages}
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_eager = min(args.steps, 4 * sets)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(n_eager)]
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(n_eager):
        p = paths[i % sets]
        e = evs[i]
        e[0].record(stream)
        for j, s in enumerate(stages):
            run_stage(p, s)
            e[j + 1].record(stream)
            ev[s].append((e[j], e[j + 1]))
    stop.record(stream)
    torch.cuda.synchronize()
    eager_ms_step = start.elapsed_time(stop) / n_eager
    eager_stage_ms = {s: float(np.mean([a.elapsed_time(b) for a, b in ev[s]])) for s in stages}

    # Timed region: exactly `steps` steps, step i a replay of input set
    # i % sets's captured step (as a serving loop would replay it), with an
    # event between consecutive steps for the per-step spread.
    g_sets = []
    for p in paths:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            p.step()
        g_sets.append(g)
    for g in g_sets:
        g.replay()
    torch.cuda.synchronize()
    n_steps = args.steps
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps + 1)]
    step_ev[0].record(stream)
    for i in range(n_steps):
        g_sets[i % sets].replay()
        step_ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms_step = step_ev[0].elapsed_time(step_ev[n_steps]) / n_steps
    step_spread = spread([step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(n_steps)])

    # Per-kernel durations: one graph per stage over all input sets, events
    # around each of its replays on the launch stream.  A graph holds at least
    # 8 launches (the rotation repeated when there are fewer sets), so that a
    # short kernel's replays are not bound by the host's graph submissions;
    # the spread is over replays (each the mean of its launches).
    stage_ms, stage_spread = {}, {}
    rounds = max(1, (8 + sets - 1) // sets)
    reps = max(3, (n_steps + sets - 1) // sets)
    for s in stages:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(rounds):
                for p in paths:
                    run_stage(p, s)
        g.replay()
        torch.cuda.synchronize()
        ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev_s[0].record(stream)
        for r in range(reps):
            g.replay()
            ev_s[r + 1].record(stream)
        torch.cuda.synchronize()
        per = [ev_s[r].elapsed_time(ev_s[r + 1]) / (sets * rounds) for r in range(reps)]
        stage_ms[s] = ev_s[0].elapsed_time(ev_s[reps]) / (reps * sets * rounds)
        stage_spread[s] = spread(per)

    T = paths[0].sb.T
    alg = [algorithmic(p.sb, p) for p in paths]
    report = {}
    # the indexer's contraction runs on the fp8 matrix cores with fp8 queries
    peak_tfs = {s: (MFMA_FP8_PEAK_TFS if args.q_fp8 and s in ("index_scores", "index_topk") else MFMA_BF16_PEAK_TFS)
                for s in stages}
    for s in stages:
        by = float(np.mean([a[s]["bytes"] for a in alg]))
        fl = float(np.mean([a[s]["flops"] for a in alg]))
        launches = alg[0][s].get("launches_per_step", 1)
        t = stage_ms[s] / 1e3
        report[s] = {"ms": stage_ms[s], "ms_spread": stage_spread[s], "launches_per_step": launches,
                     "alg_bytes": by, "alg_flops": fl,
                     "GB_s": by / t / 1e9, "TFLOP_s": fl / t / 1e12,
                     "frac_hbm": by / t / 1e9 / HBM_PEAK_GBS,
                     "frac_mfma": fl / t / 1e12 / peak_tfs[s],
                     "traffic": traffic(workload, s)}
    dom = max(stages, key=lambda s: stage_ms[s])
    r = report[dom]
    t_hbm = r["alg_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = r["alg_flops"] / (peak_tfs[dom] * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    launches = r["launches_per_step"]
    if bound == "hbm":
        ach = r["alg_bytes"] / launches / (stage_ms[dom] / launches / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS, "traffic": None}
    else:
        ach = r["alg_flops"] / (stage_ms[dom] / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": peak_tfs[dom], "unit": "TFLOP/s",
                "frac": ach / peak_tfs[dom], "traffic": None}
    roof["traffic"] = r["traffic"]
    roof["kernel"] = dom
    roof["alg_bytes_per_launch"] = r["alg_bytes"] / launches
    roof["alg_flops_per_launch"] = r["alg_flops"] / launches
    roof["avg_launch_ms"] = stage_ms[dom] / launches
    # the practical stream rate of this GPU, beside the published peak
    stream = measured_stream_peak() / 1e9
    roof["measured_stream_GB_s"] = stream
    if bound == "hbm":
        roof["frac_of_measured_stream"] = roof["achieved"] / stream

    cfg = paths[0].sb.cfg
    out = {
        "metric": METRIC,
        "value": T / (ms_step / 1e3),
        "unit": "queries/s",
        "n_gpus": 1, "steps": n_steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "step_ms": step_spread,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.q_fmt == 1 else "f32",
        "data": "synthetic (seeded, %s mode; %d rotated input sets)" % (args.mode, sets),
        "config": {"workload": "%s: batch %d, q_len %d, contexts U[%d,%d], index_topk %d, "
                               "indexer %dx%d, MLA %d heads %d+%d %s cache, page %d, %d layer(s)"
                               % (cfg.name, cfg.batch, cfg.q_len, cfg.ctx_lo, cfg.ctx_hi, cfg.topk,
                                  cfg.hi, cfg.di, cfg.heads, cfg.dc, cfg.dr,
                                  {0: "f32", 1: "bf16", 2: "fp8-e4m3-b128", 3: "int8-affine-b128"}[cfg.kv_fmt],
                                  cfg.page_size, cfg.layers)
                               + (", fp8 index keys (per-token scale)" if args.key_fp8 else "")
                               + (", fp8 index queries (per-head power-of-two scale) on fp8 MFMA"
                                  if args.q_fp8 else "")
                               + (", indexer preparation in the step" if args.prep else "")
                               + (", scores + top-k in a %.0f MB workspace (%d rows per chunk)"
                                  % (paths[0].itk_ws_bytes / 2 ** 20,
                                     paths[0].itk_ws_bytes // (4 * ((paths[0].sb.max_seq_len + 63) // 64 * 64)))
                                  if args.score_budget is not None else ""),
                   "query_rows": T},
        "indexer_topk_rows_per_s": T / ((stage_ms["index_topk"] if "index_topk" in stage_ms
                                         else stage_ms["index_scores"] + stage_ms["topk"]) / 1e3),
        "sparse_mla_queries_per_s": T / (stage_ms["sparse_mla"] / len(paths[0].kv) / 1e3),
        "timing": "HIP graph replays of whole steps (one captured step per input set, sets "
                  "rotated), an event between steps; stage times from per-stage graphs of >= 8 "
                  "launches (input sets repeated when fewer), spread over replays; eager figures "
                  "include host launch gaps",
        "eager_ms_per_step": eager_ms_step,
        "eager_stage_ms": eager_stage_ms,
        "stages": report,
        "roofline": roof,
    }
    if args.key_fp8:
        out["topk_overlap_vs_bf16_keys"] = key_fp8_overlap(paths[0], cfg_id, args.mode)
    if (not args.no_cpu and not args.key_fp8 and not args.prep and args.score_budget is None
            and args.kv is None):
        out["cpu_baseline"] = cpu_baseline(paths[0].sb)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
