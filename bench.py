#!/usr/bin/env python3
"""Throughput of the DSA decode path (indexer -> top-2048 -> sparse MLA) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload share|decode|ragged|prefill]
    python bench.py --workload writer               # the index-cache writer at the prefill shape
    python bench.py --copy-calibration MIB          # a plain device copy, for counter scaling
    python bench.py --gather-ceiling [--workload W] # the sparse-MLA row gathers alone (a bound)
    python bench.py --read-ceiling [--workload W]   # the indexer's load stream alone (a bound)
    python bench.py --rocprof-summary CSV [CSV ..]  # per-kernel table of rocprofv3 output
    python bench.py --traffic-from FETCH WRITE COPY_FETCH COPY_WRITE [--workload W] [--copy-mib M]

One step = one pass of the whole path over one batch of synthetic input.  The default
workload is the largest decode workload, IndexShare decode: 32 sequences of 131072 tokens,
one indexer pass over the fp8 index cache (32 heads x 128) and one top-2048 whose indices
feed four sparse-MLA layers, each over its own fp8 latent cache (64 heads, 512 + 64).
A step makes three library calls: dsa_index_scores_hist (the indexer, which also builds the
top-k's score histogram where the kernels allow), dsa_topk_after_hist (the selection) and
the sparse-MLA call; the same steps with the two plain calls (dsa_index_scores, then dsa_topk
with its own histogram pass) are timed beside it.
Smaller workloads fit in the 256 MB Infinity Cache, so the timed loop rotates over enough
independent input sets (> 1 GB in total) that every step reads HBM.  The line prints one
JSON object; after the headline workload the two other decode workloads (batch 8 x 8192
bf16, ragged batch 64) are measured the same way and summarised under "other_workloads"
(outside the headline's timed region; --no-others skips them).

Timing: W untimed steps, then exactly K steps between two device synchronisations.  A
second loop of K steps records HIP events around each stage on the stream the kernels run
on (torch's current stream) to get every kernel's duration per step (mean, median, min,
max); the roofline object is reported for the kernel with the largest share of the step,
from its mean.  The CPU baseline is the fp64 oracle on the host cores, on the same input
bytes.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA

WORKLOADS = {"decode": 2, "ragged": 3, "prefill": 4, "share": 5, "writer": 4}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="share", choices=sorted(WORKLOADS))
    p.add_argument("--no-others", action="store_true",
                   help="measure the headline workload only (no other_workloads summary)")
    p.add_argument("--no-compare", dest="no_compare", action="store_true",
                   help="skip the comparison timing of indexer and top-k as the two plain calls "
                        "(profiler runs: only the headline's kernels)")
    p.add_argument("--sets", type=int, default=0, help="input sets to rotate (0: enough for > 1 GB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run --steps device-to-device copies of MIB MiB (counter calibration)")
    p.add_argument("--gather-ceiling", action="store_true",
                   help="time the workload's sparse-MLA row gathers alone (dsa_gather_ceiling) beside the stage")
    p.add_argument("--read-ceiling", action="store_true",
                   help="decode workloads: time the indexer's load stream alone (dsa_read_ceiling) beside "
                        "the indexer stage")
    p.add_argument("--rocprof-summary", nargs="+", metavar="CSV", help="summarise rocprofv3 CSV files")
    p.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                   help="HBM bytes per stage call from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs")
    p.add_argument("--copy-mib", type=int, default=512, help="size of the calibration copy (MiB)")
    p.add_argument("--paged", type=int, default=0, metavar="PAGE",
                   help="run on paged caches: every cache scattered over shuffled pages of PAGE tokens")
    p.add_argument("--batch", type=int, default=0, metavar="B",
                   help="decode workload only: B sequences of 8192 tokens instead of 8 (a sweep of "
                        "the same layer shape; the headline line is the default)")
    p.add_argument("--graph", action="store_true",
                   help="capture each input set's step once as a HIP graph and time graph replays")
    return p.parse_args()


# ------------------------------------------------------------------------------- byte models

def algorithmic_model(case):
    """Algorithmic bytes / flops per stage for one step.  Each stage counts the bytes it must
    read and write: the indexer its keys, scales, q and w and its score output; the top-k the
    scores and its indices; sparse MLA the selected rows, q, indices and its output.  The path
    total counts the score array's round trip (the indexer's write, the top-k's read) zero
    times: it exists only because the two stages are separate calls."""
    n = [case.ctx[b] - case.q_len[b] + j + 1 for b in range(case.B) for j in range(case.q_len[b])]
    sum_n = float(sum(n))
    T = case.T
    H_I, D_I = case.H_I, case.D_I
    q_bytes = {"f32": 4, "bf16": 2, "fp8": 1}[case.iq_dt]
    k_row = D_I * {"f32": 4, "bf16": 2, "fp8": 1}[case.ik_dt] + (4 if case.ik_scale is not None else 0)
    idx_in = sum_n * k_row + T * H_I * (D_I * q_bytes + 4 + (4 if case.iq_scale is not None else 0))
    idx_bytes = idx_in + sum_n * 4  # + the scores written
    idx_flops = 2.0 * H_I * D_I * sum_n
    sel = [min(case.topk, x) for x in n]
    topk_bytes = sum_n * 4 + T * case.topk * 4
    Dqk = case.Dc + case.Dr
    L = len(case.layers)
    kv_row = Dqk * {"f32": 4, "bf16": 2, "fp8": 1}[case.layers[0].kv_dt]
    qb = {"f32": 4, "bf16": 2}[str(case.layers[0].q.dtype).split(".")[-1].replace("float32", "f32").replace("bfloat16", "bf16")]
    ob = 4 if case.out_dt == "f32" else 2
    mla_bytes = L * (sum(sel) * kv_row + T * case.H * (Dqk * qb + case.Dc * ob) + T * case.topk * 4)
    mla_flops = L * 2.0 * case.H * sum(sel) * (Dqk + case.Dc)
    return {
        "indexer": {"bytes": idx_bytes, "flops": idx_flops},
        "topk": {"bytes": topk_bytes, "flops": 0.0},
        "mla": {"bytes": mla_bytes, "flops": mla_flops},
        "path_bytes": idx_in + T * case.topk * 4 + mla_bytes,
    }


# ------------------------------------------------------------------------------- GPU bench

def make_sets(cfg, nsets, device, batch=0):
    from deepseek_sparse_mla_amd import synth
    if batch:  # the decode layer at another batch size
        return [synth.make_case("glm52_decode_b%d_ctx8192" % batch, cfg, ctx=[8192] * batch, sm_scale=1.0 / 16,
                                kv_dt="bf16", seed=s, device=device) for s in range(nsets)]
    return [synth.config(cfg, device=device, seed=s) for s in range(nsets)]


def case_bytes(case):
    tot = 0
    for t in (case.iq, case.iw, case.ik, case.ik_scale, case.iq_scale):
        if t is not None:
            tot += t.numel() * t.element_size()
    for L in case.layers:
        tot += L.q.numel() * L.q.element_size() + L.kv.numel() * L.kv.element_size()
    return tot


def paged_caches(case, page, seed=0):
    """The case's per-token caches scattered page by page over a pool in a shuffled order,
    with the matching block table: (layout, index keys, key scales, latent caches)."""
    import torch
    import deepseek_sparse_mla_amd as dsa
    dev = case.iq.device
    kvp = case.kv_indptr.cpu()
    ctx = [int(x) for x in (kvp[1:] - kvp[:-1])]
    npages = [-(-c // page) for c in ctx]
    total = sum(npages)
    perm = torch.randperm(total, generator=torch.Generator().manual_seed(seed))
    width = max(max(npages), -(-case.max_ctx // page))
    bt = torch.zeros((len(ctx), width), dtype=torch.int32)
    k0 = 0
    for b, n in enumerate(npages):
        bt[b, :n] = perm[k0:k0 + n].to(torch.int32)
        k0 += n
    # physical row of every cached token, in kv_indptr order
    b_of = torch.repeat_interleave(torch.arange(len(ctx)), torch.tensor(ctx))
    s_of = torch.arange(int(kvp[-1])) - kvp[:-1][b_of]
    dst = (bt[b_of, s_of // page].to(torch.int64) * page + s_of % page).to(dev)
    rows = total * page

    def scatter(x):
        pool = torch.zeros((rows,) + tuple(x.shape[1:]), dtype=x.dtype, device=dev)
        pool[dst] = x
        return pool

    lay = dsa.Layout(case.kv_indptr, case.q_indptr, case.T, case.max_ctx, block_table=bt.to(dev),
                     page_size=page, cache_rows=rows)
    return (lay, scatter(case.ik), scatter(case.ik_scale) if case.ik_scale is not None else None,
            [scatter(L.kv) for L in case.layers])


class Runner:
    """Buffers and calls of one input set (all allocations happen before timing)."""

    def __init__(self, case, paged=None):
        import torch
        import deepseek_sparse_mla_amd as dsa
        self.dsa = dsa
        self.case = case
        self.layout = dsa.Layout.of_case(case)
        self.ik, self.ik_scale, self.kvs = case.ik, case.ik_scale, [L.kv for L in case.layers]
        if paged:
            self.layout, self.ik, self.ik_scale, self.kvs = paged
        dev = case.iq.device
        self.ld = dsa.score_pitch(case.max_ctx)
        self.scores = torch.empty((case.T, self.ld), dtype=torch.float32, device=dev)
        self.idx = torch.empty((case.T, case.topk), dtype=torch.int32, device=dev)
        odt = torch.float32 if case.out_dt == "f32" else torch.bfloat16
        self.outs = [torch.empty((case.T, case.H, case.Dc), dtype=odt, device=dev) for _ in case.layers]
        self.ws = dsa.mla_workspace(self.layout, case.H, case.Dc, case.Dr, case.topk, len(case.layers), dev)
        self.tk_ws = dsa.topk_workspace(self.layout, self.ld, case.topk, dev)
        self.prefill = case.q_indptr is not None
        self.hist_built = 0

    def indexer(self):
        """The indexer; where the kernels allow it also builds the top-k's histogram."""
        c = self.case
        _, self.hist_built = self.dsa.dsa_index_scores_hist(self.layout, c.iq, c.iw, self.ik, c.topk, self.tk_ws,
                                                            k_scale=self.ik_scale, q_scale=c.iq_scale,
                                                            scores=self.scores)

    def topk(self):
        """The selection (on the indexer's histogram when it built one)."""
        self.dsa.dsa_topk_after_hist(self.layout, self.scores, self.case.topk, self.hist_built, indices=self.idx,
                                     workspace=self.tk_ws)

    def indexer_alone(self):
        c = self.case
        self.dsa.dsa_index_scores(self.layout, c.iq, c.iw, self.ik, k_scale=self.ik_scale, q_scale=c.iq_scale,
                                  scores=self.scores)

    def topk_alone(self):
        self.dsa.dsa_topk(self.layout, self.scores, self.case.topk, indices=self.idx, workspace=self.tk_ws)

    def mla(self):
        c = self.case
        if len(c.layers) == 1:
            L = c.layers[0]
            fn = self.dsa.sparse_mla_prefill if self.prefill else self.dsa.sparse_mla_decode
            fn(self.layout, L.q, self.kvs[0], self.idx, c.sm_scale, c.Dc, L.kv_scale, out=self.outs[0],
               workspace=self.ws)
        else:
            self.dsa.sparse_mla_decode_shared(self.layout, [L.q for L in c.layers], self.kvs,
                                              [L.kv_scale for L in c.layers], self.idx, c.sm_scale, c.Dc,
                                              outs=self.outs, workspace=self.ws)

    def step(self):
        self.indexer()
        self.topk()
        self.mla()


def cpu_baseline(case, target_s):
    """Time the fp64 oracle on the host for whole query rows of the same workload."""
    import numpy as np
    import oracle
    from deepseek_sparse_mla_amd import synth

    kvp = synth.host(case.kv_indptr)
    qi = synth.host(case.q_indptr)
    idx_in = dict(q=synth.host(case.iq), w=synth.host(case.iw), k=synth.host(case.ik),
                  k_scale=synth.host(case.ik_scale), q_scale=synth.host(case.iq_scale))
    layers = [dict(q=synth.host(L.q), kv=synth.host(L.kv), kv_scale=L.kv_scale) for L in case.layers]
    oracle.build()
    rows_done = 0
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.index_share(kvp, qi, idx_in, layers, case.topk, case.sm_scale, case.Dc)
        rows_done += case.T
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            break
    threads = oracle.num_threads()
    return {"value": rows_done / el, "unit": "query-tokens/s", "cores": int(min(threads, case.T)),
            "kind": "oracle", "cpu": cpu_model_name(),
            "sample": "%d full passes of the %s batch (%d query rows each: indexer + top-%d + sparse MLA, "
                      "fp64) in %.1f s on %d host threads (%d usable: OpenMP over query rows)"
                      % (reps, case.name, case.T, case.topk, el, threads, min(threads, case.T))}


# ------------------------------------------------------------------------------- counters

STAGE_SOURCES = {"indexer": "indexer.hip", "topk": "topk.hip", "mla": "sparse_mla.hip",
                 "writer": "index_quant.hip"}
STAGE_KERNELS = {"indexer": ("idx_",), "topk": ("topk_",), "mla": ("mla_",), "writer": ("index_front",)}


def _short(name):
    """Kernel name without namespace, template arguments and parameter list."""
    base = name.split("(")[0]
    base = base.split("<")[0]
    return base.replace("void ", "").replace("dsa::", "").strip()


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def source_digest(stage):
    import hashlib
    path = os.path.join(ROOT, "deepseek_sparse_mla_amd", "csrc", STAGE_SOURCES[stage])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def counter_means(path, by_grid=False):
    """{(kernel, counter): (mean value per dispatch, dispatches)} of a counter_collection CSV
    (kernel names carry "@<grid size>" with by_grid, to tell launches of one kernel apart)."""
    acc = {}
    for r in _read_csv(path):
        name = _short(r["Kernel_Name"]) + ("@" + r["Grid_Size"] if by_grid else "")
        key = (name, r["Counter_Name"])
        tot, n = acc.get(key, (0.0, 0))
        acc[key] = (tot + float(r["Counter_Value"]), n + 1)
    return {k: (v[0] / v[1], v[1]) for k, v in acc.items()}


def rocprof_summary(paths):
    for path in paths:
        rows = _read_csv(path)
        print("# %s" % os.path.basename(path))
        if rows and "AverageNs" in rows[0]:
            print("%-28s %7s %12s %9s" % ("kernel", "calls", "avg_us", "share_%"))
            for r in rows:
                print("%-28s %7s %12.2f %9.2f" % (_short(r["Name"])[:28], r["Calls"], float(r["AverageNs"]) / 1e3,
                                                  float(r["Percentage"])))
        elif rows and "Counter_Name" in rows[0]:
            print("%-28s %-12s %10s %16s" % ("kernel", "counter", "dispatches", "mean_per_dispatch"))
            for (k, c), (m, n) in sorted(counter_means(path).items()):
                print("%-28s %-12s %10d %16.1f" % (k[:28], c, n, m))


def traffic_from(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes, workload):
    """HBM bytes per stage call: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) summed over a
    stage's kernels, each scaled by what the counter reads for a copy of known size."""
    def copy_factor(path, counter):
        vals = [(m, n) for (k, c), (m, n) in counter_means(path).items()
                if c == counter and "copy" in k.lower()]
        if not vals:
            raise SystemExit("no copy kernel in %s" % path)
        m = max(v[0] for v in vals)  # the large copy (the fill kernel is not a copy)
        return m * 1024.0 / copy_bytes
    ff = copy_factor(copy_fetch_csv, "FETCH_SIZE")
    wf = copy_factor(copy_write_csv, "WRITE_SIZE")
    # The writer workload times the front-end kernel; counters are kept per grid size so
    # that only its own launches (the largest grid of its name) are counted.
    writer = workload == "writer"
    fm, wm = counter_means(fetch_csv, writer), counter_means(write_csv, writer)
    out = {"workload": workload, "copy_bytes": copy_bytes, "fetch_factor": round(ff, 4),
           "write_factor": round(wf, 4), "stages": {}}
    for st, prefixes in STAGE_KERNELS.items():
        kern = sorted({k for (k, c) in fm if c == "FETCH_SIZE" and k.startswith(prefixes)})
        if writer and kern:
            kern = [max(kern, key=lambda k: int(k.split("@")[1]))]
        if not kern:
            continue
        # calls of the stage = dispatches of its most frequent kernel
        calls = max(fm[(k, "FETCH_SIZE")][1] for k in kern)
        fetch = sum(fm[(k, "FETCH_SIZE")][0] * fm[(k, "FETCH_SIZE")][1] for k in kern) / calls
        write = sum(wm[(k, "WRITE_SIZE")][0] * wm[(k, "WRITE_SIZE")][1] for k in kern
                    if (k, "WRITE_SIZE") in wm) / calls
        out["stages"][st] = {"kernels": kern, "calls": calls, "fetch_kib_per_call": round(fetch, 1),
                             "write_kib_per_call": round(write, 1),
                             "hbm_bytes_per_call": round(fetch * 1024.0 / ff + write * 1024.0 / wf),
                             "source_sha256": source_digest(st)}
    print(json.dumps(out, indent=1))


def measured_traffic(workload, stage):
    """HBM bytes per call of a stage from the committed counter summary, or None when there is
    none for this workload or the stage's source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    st = d.get("stages", {}).get(stage)
    if not st or st.get("source_sha256") != source_digest(stage):
        return None
    return st["hbm_bytes_per_call"]


def gather_ceiling(workload, steps, warmup):
    """The workload's own top-k rows gathered with no arithmetic (dsa_gather_ceiling, the
    sparse-MLA kernels' load path), timed beside the sparse-MLA stage on the same indices."""
    import torch
    from deepseek_sparse_mla_amd import synth
    torch.cuda.set_device(0)
    case = synth.config(WORKLOADS[workload], "cuda:0")
    run = Runner(case)
    run.indexer()
    run.topk()
    # positions -> absolute cache rows (contiguous caches: the sequence's first row added)
    kv_base = case.kv_indptr[:-1]
    if case.q_indptr is None:
        seq_of_row = torch.arange(case.T, device="cuda:0")
    else:
        seq_of_row = torch.repeat_interleave(torch.arange(case.B, device="cuda:0"),
                                             (case.q_indptr[1:] - case.q_indptr[:-1]).long())
    absidx = torch.where(run.idx >= 0, run.idx + kv_base[seq_of_row].unsqueeze(1).to(torch.int32),
                         torch.full_like(run.idx, -1)).contiguous()
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda:0")
    tables = [kv.view(torch.uint8) if kv.dtype != torch.bfloat16 else kv for kv in run.kvs]

    def gather():
        for tab in tables:
            run.dsa.dsa_gather_ceiling(tab, absidx, sink)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        for i in range(steps):
            ev[i].record()
            fn()
        ev[steps].record()
        torch.cuda.synchronize()
        t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        return {"median": round(t[steps // 2], 5), "min": round(t[0], 5), "max": round(t[-1], 5)}

    g = timed(gather)
    m = timed(run.mla)
    row_bytes = tables[0].shape[1] * tables[0].element_size()
    nrows = int((absidx >= 0).sum().item()) * len(tables)
    gbytes = nrows * row_bytes
    print(json.dumps({
        "workload": case.name,
        "gathered_rows": nrows, "row_bytes": row_bytes, "gathered_bytes": gbytes,
        "gather_only_ms": g, "gather_only_GBps": round(gbytes / (g["median"] * 1e-3) / 1e9, 1),
        "sparse_mla_stage_ms": m, "stage_GBps_of_gathers": round(gbytes / (m["median"] * 1e-3) / 1e9, 1),
        "stage_over_gather_only": round(m["median"] / g["median"], 3),
        "steps": steps, "warmup": warmup}))


def _timed(fn, steps, warmup):
    """HIP-event times (ms) of `steps` calls of fn after `warmup` untimed ones."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        ev[i].record()
        fn()
    ev[steps].record()
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return {"median": round(t[steps // 2], 5), "min": round(t[0], 5), "max": round(t[-1], 5)}


def read_ceiling(workload, steps, warmup):
    """The decode indexer's load stream with no arithmetic and no stores (dsa_read_ceiling, the
    same shares, tiles and lanes), on the workload's own index cache, timed beside the indexer
    stage (plain call): 132 bytes read per token either way.  Pattern 0 keeps the indexer's
    lanes for rows it cannot read as contiguous tiles, pattern 1 reads 1 KB of consecutive bytes
    per load instruction, pattern 2 does so with nontemporal loads: the indexer's own stream on
    these key planes."""
    import torch
    from deepseek_sparse_mla_amd import synth
    if workload not in ("share", "ragged", "decode"):
        print("--read-ceiling applies to the decode workloads (share, ragged, decode)", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    case = synth.config(WORKLOADS[workload], "cuda:0")
    run = Runner(case)
    n = int(case.kv_indptr[-1].item())
    sink = torch.zeros(512, dtype=torch.int32, device="cuda:0")
    rb = n * 132
    out = {"workload": case.name, "tokens": n, "bytes_read": rb}
    for pattern in (0, 1, 2):
        t = _timed(lambda: run.dsa.dsa_read_ceiling(case.ik, case.ik_scale, sink, n, pattern), steps, warmup)
        out["pattern%d_ms" % pattern] = t
        out["pattern%d_GBps" % pattern] = round(rb / (t["median"] * 1e-3) / 1e9, 1)
    t = _timed(run.indexer_alone, steps, warmup)
    out["indexer_ms"] = t
    out["indexer_GBps_read"] = round(rb / (t["median"] * 1e-3) / 1e9, 1)
    out["indexer_over_pattern0"] = round(t["median"] / out["pattern0_ms"]["median"], 3)
    out["indexer_over_pattern2"] = round(t["median"] / out["pattern2_ms"]["median"], 3)
    out.update({"steps": steps, "warmup": warmup})
    print(json.dumps(out))


def copy_calibration(mib, copies):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(copies):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": copies}))


# ------------------------------------------------------------------------------- writer bench

def writer_bytes(T, H_I):
    """Algorithmic bytes of the writer per prefill chunk: per query head 256 B read (bf16) and
    128 B codes + 4 B scale written; per row an 8-byte position and the 256-byte rope-table row
    read once; per key 256 B read, 8 B position, 8 B slot, 256 B table row, 132 B written."""
    q = T * (H_I * (256 + 128 + 4) + 8 + 256)
    k = T * (256 + 8 + 8 + 256 + 132)
    return q, k


def writer_cpu_baseline(wc, tab, target_s):
    """The oracle's writer on the host for whole rows (32 query heads + one key each)."""
    import oracle
    from deepseek_sparse_mla_amd import synth
    oracle.build()
    q, k = synth.host(wc.q), synth.host(wc.k)
    pos, tabh = synth.host(wc.positions), synth.host(tab)
    rows, t0, el = 0, time.perf_counter(), 0.0
    chunk = 64
    while el < target_s and rows < wc.q.shape[0]:
        r = slice(rows, rows + chunk)
        oracle.index_quant(q[r], positions=pos[r], cos_sin=tabh)
        oracle.index_quant(k[r].reshape(-1, 1, 128), positions=pos[r], cos_sin=tabh)
        rows += chunk
        el = time.perf_counter() - t0
    threads = oracle.num_threads()
    return {"value": rows / el, "unit": "query-rows/s", "cores": int(threads), "kind": "oracle",
            "sample": "the first %d rows of the chunk (32 query heads + one key each, rope + fp8 "
                      "quantisation) in %.1f s on %d host threads" % (rows, el, threads)}


def writer_main(args):
    import torch
    import deepseek_sparse_mla_amd as dsa
    from deepseek_sparse_mla_amd import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    probe = synth.writer_case(0, dev)
    T, H_I = probe.q.shape[:2]
    tab = synth.rope_table(probe.cache_rows, device=dev)
    per_set = T * H_I * (256 + 132) + T * (256 + 132)
    nsets = args.sets or max(1, min(32, math.ceil(1.2e9 / per_set)))
    sets = []
    for sd in range(nsets):
        wc = probe if sd == 0 else synth.writer_case(sd, dev)
        sets.append(dict(wc=wc, cache=torch.zeros((wc.cache_rows, 128), dtype=torch.uint8, device=dev),
                         scale=torch.zeros(wc.cache_rows, dtype=torch.float32, device=dev),
                         q8=torch.empty((T, H_I, 128), dtype=torch.uint8, device=dev),
                         qs=torch.empty((T, H_I), dtype=torch.float32, device=dev)))

    def fused(st):
        wc = st["wc"]
        dsa.dsa_index_front_end(wc.q, wc.k, wc.slots, st["cache"], st["scale"], positions=wc.positions,
                                cos_sin=tab, q_fp8=st["q8"], q_scale=st["qs"])

    def q_part(st):
        dsa.dsa_index_q_quant(st["wc"].q, positions=st["wc"].positions, cos_sin=tab, q_fp8=st["q8"],
                              q_scale=st["qs"])

    def k_part(st):
        dsa.dsa_index_k_cache_write(st["wc"].k, st["wc"].slots, st["cache"], st["scale"],
                                    positions=st["wc"].positions, cos_sin=tab)

    torch.cuda.synchronize()
    for s in range(args.warmup):
        fused(sets[s % nsets])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        fused(sets[s % nsets])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # Per-call durations: HIP events around K back-to-back launches of one call on the launch
    # stream, so the GPU is not left waiting for the host between two events.
    stream = torch.cuda.current_stream()
    ms = {}
    for name, fn in (("front", fused), ("q", q_part), ("k", k_part)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(args.steps):
            fn(sets[s % nsets])
        e1.record(stream)
        torch.cuda.synchronize()
        ms[name] = e0.elapsed_time(e1) / args.steps
    qb, kb = writer_bytes(T, H_I)
    achieved = (qb + kb) / (ms["front"] * 1e-3) / 1e9
    line = {
        "metric": "prefill index-writer query-rows/s (rope + fp8 ue8m0 quantisation of 32 index-query "
                  "heads and one index key per row) and % of peak HBM GB/s",
        "value": round(T * args.steps / elapsed, 1),
        "unit": "query-rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": probe.name, "query_rows": T, "index_heads": H_I, "index_dim": 128,
                   "rope_dims": 64, "rope": "interleaved", "cache": "split planes",
                   "input_sets_rotated": nsets},
        "kernels_ms": {"dsa_index_front_end: index_front_kernel": round(ms["front"], 5),
                       "dsa_index_q_quant: index_quant_kernel (alone)": round(ms["q"], 5),
                       "dsa_index_k_cache_write: index_quant_kernel (alone)": round(ms["k"], 5)},
        "roofline": {"kernel": "dsa_index_front_end: index_front_kernel", "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic": qb + kb,
                     "traffic": measured_traffic("writer", "writer")},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = writer_cpu_baseline(probe, tab, min(args.cpu_seconds, 12.0))
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.rocprof_summary:
        return rocprof_summary(args.rocprof_summary)
    if args.traffic_from:
        return traffic_from(*args.traffic_from, copy_bytes=args.copy_mib << 20, workload=args.workload)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.batch and args.workload != "decode":
        print("--batch applies to the decode workload only", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration, args.steps)
    if args.gather_ceiling:
        return gather_ceiling(args.workload, min(args.steps, 20), min(args.warmup, 3))
    if args.read_ceiling:
        return read_ceiling(args.workload, min(args.steps, 20), min(args.warmup, 3))
    if args.workload == "writer":
        return writer_main(args)
    import torch

    torch.cuda.set_device(0)
    line = measure(args.workload, args, args.steps, args.warmup, headline=True)
    if not args.no_others and not (args.paged or args.batch or args.graph) and args.workload == "share":
        others = {}
        for wl in ("decode", "ragged"):
            torch.cuda.empty_cache()
            o = measure(wl, args, min(args.steps, 20), min(args.warmup, 3), headline=False)
            others[o["config"]["workload"]] = {
                "ms_per_step": o["ms_per_step"], "value": o["value"], "unit": o["unit"],
                "step_ms_events": o["step_ms_events"], "path_hbm": o["path_hbm"],
                "kernels_ms": o["kernels_ms"], "roofline": o["roofline"], "steps": o["steps"],
                "dtype": o["dtype"], "plain_index_topk": o["plain_index_topk"]}
        line["other_workloads"] = others
    print(json.dumps(line), flush=True)


def cpu_model_name():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.lower().startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def dtypes_of(case):
    """What each stage computes in, for the line's "dtype" and "dtypes"."""
    kv = case.layers[0].kv_dt
    idx = ("fp8 keys x fp8 q (per-head scale), fp8 MFMA" if case.iq_dt == "fp8" else
           "fp8 keys x %s q, keys widened exactly to bf16, bf16 MFMA" % case.iq_dt) + ", fp32 accumulate"
    mla = ("fp8 latent x bf16 q, bf16 MFMA on exactly widened fp8" if kv == "fp8" else
           "%s latent x %s q, %s MFMA" % (kv, kv, kv)) + ", fp32 softmax and accumulate"
    d = {"indexer": idx, "topk": "fp32 scores, integer keys", "mla": mla}
    short = "bf16" if kv == "bf16" else "fp8/bf16" if kv == "fp8" else kv
    return short, d


def measure(workload, args, steps, warmup, headline):
    """One workload: build its input sets, warm up, time exactly `steps` steps, then time
    each stage with HIP events.  Returns the JSON object of the line."""
    import torch
    from deepseek_sparse_mla_amd import synth  # noqa: F401

    cfg = WORKLOADS[workload]
    dev = "cuda:0"
    probe = make_sets(cfg, 1, dev, args.batch if headline else 0)[0]
    per_set = case_bytes(probe)
    nsets = (args.sets if headline else 0) or max(1, min(16, math.ceil(1.2e9 / per_set)))
    cases = [probe] + (make_sets(cfg, nsets, dev, args.batch if headline else 0)[1:] if nsets > 1 else [])
    paged = args.paged if headline else 0
    runners = [Runner(c, paged_caches(c, paged, seed=j) if paged else None)
               for j, c in enumerate(cases)]
    model = algorithmic_model(probe)
    torch.cuda.synchronize()

    # warmup
    for s in range(warmup):
        runners[s % nsets].step()
    torch.cuda.synchronize()

    steppers = [r.step for r in runners]
    graph = args.graph and headline
    if graph:
        # one graph per input set, each holding one whole step (the library only enqueues
        # kernels: nothing in a step allocates, clears or synchronises)
        graphs = []
        for r in runners:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                r.step()
            graphs.append(g)
        torch.cuda.synchronize()
        steppers = [g.replay for g in graphs]
        for s in range(warmup):
            steppers[s % nsets]()
        torch.cuda.synchronize()

    # timed region: exactly K steps
    t0 = time.perf_counter()
    for s in range(steps):
        steppers[s % nsets]()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / steps

    # per-kernel durations with HIP events on the launch stream
    stream = torch.cuda.current_stream()
    stages = ("indexer", "topk", "mla")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for s in range(steps):
        r = runners[s % nsets]
        e = ev[s]
        e[0].record(stream)
        r.indexer()
        e[1].record(stream)
        r.topk()
        e[2].record(stream)
        r.mla()
        e[3].record(stream)
    torch.cuda.synchronize()
    per = {st: [ev[s][k].elapsed_time(ev[s][k + 1]) for s in range(steps)] for k, st in enumerate(stages)}
    per_step = [ev[s][0].elapsed_time(ev[s][3]) for s in range(steps)]
    dur = {st: sum(v) / steps for st, v in per.items()}  # ms

    def spread(v):
        a = sorted(v)
        return {"median": round(a[len(a) // 2] if len(a) % 2 else 0.5 * (a[len(a) // 2 - 1] + a[len(a) // 2]), 5),
                "min": round(a[0], 5), "max": round(a[-1], 5), "mean": round(sum(a) / len(a), 5)}

    # the same steps with indexer and top-k as the two plain calls, the top-k with its own
    # histogram pass (reported beside the headline)
    ncmp = 0 if args.no_compare else steps
    fz = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(ncmp)]
    for s in range(ncmp):
        r = runners[s % nsets]
        e = fz[s]
        e[0].record(stream)
        r.indexer_alone()
        e[1].record(stream)
        r.topk_alone()
        e[2].record(stream)
        r.mla()
        e[3].record(stream)
    torch.cuda.synchronize()
    alone_idx = [fz[s][0].elapsed_time(fz[s][1]) for s in range(ncmp)]
    alone_topk = [fz[s][1].elapsed_time(fz[s][2]) for s in range(ncmp)]
    alone_step = [fz[s][0].elapsed_time(fz[s][3]) for s in range(ncmp)]

    T = probe.T
    value = T * steps / elapsed
    dominant = max(stages, key=lambda st: dur[st])
    st_model = model[dominant]
    prefill = probe.q_indptr is not None
    if dominant == "indexer" and prefill:
        bound, unit, peak = "mfma", "TFLOP/s", FP8_PEAK_TFLOPS
        achieved = st_model["flops"] / (dur[dominant] * 1e-3) / 1e12
    elif dominant == "mla" and prefill:
        bound, unit, peak = "mfma", "TFLOP/s", BF16_PEAK_TFLOPS
        achieved = st_model["flops"] / (dur[dominant] * 1e-3) / 1e12
    else:
        bound, unit, peak = "hbm", "GB/s", HBM_PEAK_GBS
        achieved = st_model["bytes"] / (dur[dominant] * 1e-3) / 1e9
    split = runners[0].ws is not None and runners[0].ws.numel() > 0
    hist = runners[0].hist_built  # the indexer built the top-k's histogram
    kernel_names = {
        "indexer": "dsa_index_scores_hist: " + ("idx_fp8_kernel" if prefill else "idx_decode_kernel")
        + (" (+ top-k histogram)" if hist else ""),
        "topk": "dsa_topk_after_hist: " + ("topk_direct_kernel" if probe.max_ctx <= 32768 else
                                           ("" if hist else "topk_hist_kernel + ")
                                           + ("topk_mark_kernel + topk_select_kernel"
                                              if probe.T <= 512 or probe.max_ctx > (1 << 18) else
                                              "topk_select_kernel")),
        "mla": ("sparse_mla_prefill: " if prefill else "sparse_mla_decode%s: " % ("_shared" if len(probe.layers) > 1 else ""))
        + ("mla_fp8_kernel" if probe.layers[0].kv_dt == "fp8" else
           "mla_hh_kernel" if probe.T <= 64 else "mla_bf16_team_kernel")
        + (" + mla_combine_kernel" if split else ""),
    }
    path_gbs = model["path_bytes"] / (ms_per_step * 1e-3) / 1e9
    dshort, dstages = dtypes_of(probe)
    line = {
        "metric": "decode query-tokens/s (indexer+top-2048+sparse MLA) and % of peak HBM GB/s",
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dshort,
        "dtypes": dstages,
        "data": "synthetic",
        "config": {"workload": probe.name, "batch": probe.B, "query_rows": T, "context": probe.ctx[0] if len(set(probe.ctx)) == 1 else "ragged",
                   "index_heads": probe.H_I, "index_dim": probe.D_I, "topk": probe.topk, "mla_heads": probe.H,
                   "latent": probe.Dc, "rope": probe.Dr, "kv_cache": probe.layers[0].kv_dt,
                   "layers": len(probe.layers), "input_sets_rotated": nsets,
                   "launch": "hip graph replay" if graph else "eager",
                   "caches": "paged, %d tokens per page, shuffled pages" % paged if paged
                   else "contiguous"},
        "path_hbm": {"algorithmic_bytes": model["path_bytes"], "achieved_GBps": round(path_gbs, 1),
                     "frac_of_peak": round(path_gbs / HBM_PEAK_GBS, 4)},
        "step_ms_events": spread(per_step),
        "kernels_ms": {kernel_names[s]: round(dur[s], 5) for s in stages},
        "kernels_ms_spread": {kernel_names[s]: spread(per[s]) for s in stages},
        "plain_index_topk": None if args.no_compare else {
            "calls": "dsa_index_scores, then dsa_topk with its own histogram pass",
            "indexer_ms": spread(alone_idx), "topk_ms": spread(alone_topk),
            "step_ms_events": spread(alone_step)},
        "roofline": {"kernel": kernel_names[dominant], "bound": bound, "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "algorithmic": st_model["bytes"] if bound == "hbm" else st_model["flops"],
                     # counters are taken on the contiguous default shapes only
                     "traffic": None if (paged or (args.batch and headline)) else measured_traffic(workload, dominant)},
    }
    if headline and not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(probe, args.cpu_seconds)
    del runners, cases, probe
    return line


if __name__ == "__main__":
    main()
