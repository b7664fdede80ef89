#!/usr/bin/env python3
"""Benchmark of the QSA indexer hot path on one MI355X.

One step = qsa_pool_prep (the pool of every block and the prep of every
query row, one launch) -> qsa_score_prepped (every row) -> qsa_select_mask_ws
(every row; few long rows split over workgroups through a workspace
allocated once) over one batch of a seeded synthetic workload, inputs
resident in HBM.  The pool and the prep are also timed alone, as the
separate qsa_pool_keys and qsa_prep_queries calls.  W untimed warm-up steps, then K timed steps between
two device synchronisations; per-kernel durations come from HIP events
recorded on the launch stream around each call.

Prints ONE JSON line.  `value` is scored (row, block) pairs per second of the
whole step on the main workload (default: the 8192-row prefill chunk over a
65536-token cache).  The same line carries select+mask microseconds per row
on the 64k- and 256k-context decode workloads and on the one-row shapes, the
roofline of the dominant kernel and the CPU oracle baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU reaches its steady clocks only after ~100 ms of this load: with 5
    # warm-up steps (2 ms) the timed steps measured 12% slower than at 300.
    ap.add_argument("--steps", type=int, default=1000, help="timed steps (~0.35 s on the main workload)")
    ap.add_argument("--warmup", type=int, default=300, help="untimed steps first")
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side", action="store_true", help="skip the decode and one-row figures")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU-oracle budget for the baseline sample")
    ap.add_argument("--only", default=None,
                    help="counter pass: run these comma-separated stages (pool,prep,pool_prep,score,select) "
                         "--reps times each on --workload, after a plain copy of a known size")
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 counter runs of --only (FETCH_SIZE, then "
                         "WRITE_SIZE) into profiles/traffic.json")
    return ap.parse_args()


# ----------------------------------------------------------------------------
# workload on the device
# ----------------------------------------------------------------------------

class Device:
    def __init__(self, w, torch, qsa):
        self.w, self.torch, self.qsa = w, torch, qsa
        dev = "cuda:0"
        np_ = __import__("numpy")
        T = w["tokens"]
        rows = len(w["pos"])
        self.T, self.rows, self.cols = T, rows, T // 4
        self.raw = torch.from_numpy(w["raw_keys"].view(np_.int16)).to(dev)
        self.q = torch.from_numpy(w["queries"].reshape(rows, 512).view(np_.int16)).to(dev)
        self.wk = torch.from_numpy(w["k_norm_w"].view(np_.int16)).to(dev)
        self.wq = torch.from_numpy(w["q_norm_w"].view(np_.int16)).to(dev)
        self.pos = torch.from_numpy(w["pos"].astype(np_.int32)).to(dev)
        self.pooled = torch.empty((T // 4, 128), dtype=torch.int16, device=dev)
        self.qhat = torch.empty((rows, 4, 128), dtype=torch.int16, device=dev)
        self.scores = torch.empty(rows * max(self.cols, 1), dtype=torch.float32, device=dev)
        self.mask = torch.empty((rows, T), dtype=torch.uint8, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        ws = qsa.qsa_select_workspace_bytes(rows, T)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev) if ws else None
        n = (w["pos"].astype(np_.int64) + 1) // 4
        self.pairs = int(n.sum())
        self.nmax = int(n.max())

    def pool(self):
        w = self.w
        self.qsa.qsa_pool_keys(self.raw, self.wk, w["rotary_dim"], w["theta"], w["eps"], self.pooled)

    def prep(self):
        w = self.w
        self.qsa.qsa_prep_queries(self.q, self.pos, self.wq, w["rotary_dim"], w["theta"], w["eps"],
                                  self.T, self.qhat, self.status)

    def pool_prep(self):
        """The pool and the query prep in one launch (qsa_pool_prep): the step's first kernel."""
        w = self.w
        self.qsa.qsa_pool_prep(self.raw, self.wk, self.q, self.pos, self.wq, w["rotary_dim"], w["theta"],
                               w["eps"], self.pooled, self.qhat, self.status)

    def score(self):
        self.qsa.qsa_score_prepped(self.qhat, self.pos, self.pooled, self.T, self.scores, self.cols,
                                   self.status)

    def select(self):
        self.qsa.qsa_select_mask_ws(self.scores, self.cols, self.pos, self.T, self.w["budget"],
                                    self.mask, self.status, self.ws)

    # algorithmic bytes / flops per launch
    def pool_bytes(self):
        return (self.T // 4) * (4 * 256 + 256)

    def prep_bytes(self):
        return self.rows * (1024 + 4 + 1024) + 256

    def pool_prep_bytes(self):
        return self.pool_bytes() + self.prep_bytes()

    def score_bytes(self):
        return self.nmax * 256 + self.rows * (1024 + 4) + 4 * self.pairs

    def score_flops(self):
        return 1024 * self.pairs

    def select_bytes(self):
        return 4 * self.pairs + self.rows * (self.T + 4)


def step_stages(d: Device):
    """The step's launches: pool and query prep (one launch), score, select."""
    return (("pool_prep", d.pool_prep), ("score", d.score), ("select", d.select))


def kernel_stages(d: Device):
    """Every kernel reported: the step's three, and the pool and the prep
    launched alone (the separate C-ABI calls)."""
    return (("pool", d.pool), ("prep", d.prep)) + step_stages(d)


def event_steps(d: Device, n: int, warmup: int, torch, stages=None):
    """Per-kernel microseconds of `n` steps after `warmup` untimed ones, each
    launch between its own HIP event pair."""
    stages = step_stages(d) if stages is None else stages
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for _, fn in stages:
            fn()
    ev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(n)] for name, _ in stages}
    for k in range(n):
        for name, fn in stages:
            a, b = ev[name][k]
            a.record(stream)
            fn()
            b.record(stream)
    torch.cuda.synchronize()
    return {name: [a.elapsed_time(b) * 1e3 for a, b in ev[name]] for name, _ in stages}


def time_steps(d: Device, steps: int, warmup: int, torch, probe_steps: int = 50, profile_steps: int = 300):
    """Warm-up steps; `probe_steps` steps with HIP events around every kernel
    to find the dominant kernel; the `steps` timed steps between device
    synchronisations, with events around the dominant kernel only (an event
    pair around each launch costs ~5-7 us of GPU time); then `profile_steps`
    steps with events around every kernel, and the pool and prep alone, for
    the other kernels' durations.  Returns the timed steps' wall time, the
    per-kernel durations (the dominant kernel's from the timed steps) and
    its name."""
    stages = step_stages(d)
    stream = torch.cuda.current_stream()
    probe = event_steps(d, probe_steps, warmup, torch)
    dom = max(probe, key=lambda n: sum(probe[n]))
    tev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        for name, fn in stages:
            if name == dom:
                tev[k][0].record(stream)
                fn()
                tev[k][1].record(stream)
            else:
                fn()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = event_steps(d, profile_steps, 0, torch, kernel_stages(d))
    per[dom] = [a.elapsed_time(b) * 1e3 for a, b in tev]
    return wall, per, dom


def prime(torch):
    """Keep the GPU busy for ~2 ms so the host can queue a whole measured
    sequence ahead of it: small launches then run back to back on the GPU
    instead of waiting for the Python binding's per-call host time."""
    torch.cuda._sleep(4_000_000)


def back_to_back_us(d: Device, torch, reps: int = 20):
    """Per-launch microseconds of each stage launched `reps` times back to back
    between one pair of HIP events, queued behind a busy GPU (no event between
    launches: an event pair costs ~4.5 us of GPU time around a single launch)."""
    stream = torch.cuda.current_stream()
    out = {}
    for name, fn in kernel_stages(d):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        prime(torch)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        out[name] = round(a.elapsed_time(b) * 1e3 / reps, 3)
    return out


def progress(msg: str) -> None:
    """A progress line on stderr (stdout carries only the result line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def launch_floor_us(torch, reps: int = 50):
    """Microseconds per launch of a one-element fill (torch's own kernel)
    launched back to back behind a busy GPU: the per-kernel floor that every
    launch in a dependent chain pays, whatever it computes."""
    x = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    for _ in range(5):
        x.fill_(1.0)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    prime(torch)
    a.record(stream)
    for _ in range(reps):
        x.fill_(1.0)
    b.record(stream)
    torch.cuda.synchronize()
    return round(a.elapsed_time(b) * 1e3 / reps, 3)


def flush_caches(flush):
    """Read a 512 MiB buffer: evicts L2 and the MALL without leaving dirty
    lines whose write-back would land in the next measurement, and keeps the
    GPU busy while the host queues what follows."""
    flush.sum()


def cold_step_us(d: Device, torch, reps: int = 10):
    """Whole-step microseconds (pool + prep, score, select back to back) with L2
    and MALL flushed before every step; one HIP event pair around each step,
    so the figure includes the launch gaps and one event pair's GPU overhead
    and is an upper bound on the kernels' cold time."""
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    ts = []
    for i in range(reps + 2):
        flush_caches(flush)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        d.pool_prep()
        d.score()
        d.select()
        b.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            ts.append(a.elapsed_time(b) * 1e3)
    # the same bracket around nothing: the event pair's own GPU time
    fl = []
    for i in range(reps + 2):
        flush_caches(flush)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        b.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            fl.append(a.elapsed_time(b) * 1e3)
    del flush
    return round(sum(ts) / len(ts), 2), round(sum(fl) / len(fl), 2)


def median(xs):
    s = sorted(xs)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def kernel_report(d: Device, per_us):
    mean = {k: sum(v) / len(v) for k, v in per_us.items()}
    rep = {}
    for name, b in (("pool", d.pool_bytes()), ("prep", d.prep_bytes()), ("pool_prep", d.pool_prep_bytes()),
                    ("score", d.score_bytes()), ("select", d.select_bytes())):
        if name not in mean:
            continue
        t = mean[name]
        gbs = b / (t * 1e-6) / 1e9
        rep[name] = {"mean_us": round(t, 3), "median_us": round(median(per_us[name]), 3),
                     "min_us": round(min(per_us[name]), 3), "max_us": round(max(per_us[name]), 3),
                     "alg_bytes": b, "achieved_GBs": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    tf = d.score_flops() / (mean["score"] * 1e-6) / 1e12
    rep["score"]["alg_flops"] = d.score_flops()
    rep["score"]["achieved_TFs"] = round(tf, 1)
    rep["score"]["mfma_frac"] = round(tf / MFMA_BF16_PEAK_TFS, 4)
    return rep, mean


# the sources each stage's kernel is built from: its counters go stale when they change
STAGE_SOURCES = {
    "pool": ["pool.hip", "pool_body.h", "qsa_device.h", "qsa_rope_math.h"],
    "prep": ["prep.hip", "prep_body.h", "qsa_device.h", "qsa_rope_math.h"],
    "pool_prep": ["pool_prep.hip", "pool_body.h", "prep_body.h", "qsa_device.h", "qsa_rope_math.h"],
    "score": ["score.hip", "qsa_device.h"],
    "select": ["select.hip", "select_split.hip", "select_common.h", "qsa_device.h"],
}
# kernel-name prefix of each stage in rocprofv3 output, matched against the
# unqualified kernel name (a stage may launch several kernels: the split
# select launches a chunk and a merge kernel)
STAGE_KERNELS = {"pool": "pool_kernel", "prep": "prep_kernel", "pool_prep": "pool_prep_kernel",
                 "score": "score_", "select": "select_"}


def kernel_base(name: str) -> str:
    """Unqualified kernel name without template arguments or parameters."""
    n = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return n.split("(")[0].split("<")[0].split("::")[-1]


def stage_of(name: str, stage: str) -> bool:
    frag = STAGE_KERNELS[stage]
    base = kernel_base(name)
    return base.startswith(frag) if frag.endswith("_") else base == frag
COPY_BYTES = 512 << 20  # the counter pass's calibration copy


def source_hash(stage: str) -> str:
    h = hashlib.sha256()
    for name in STAGE_SOURCES[stage]:
        with open(os.path.join(ROOT, "sparse_attention_token_qsa_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(stage: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if the
    stage's sources are unchanged since the counters were taken; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    entry = table.get(f"{stage}:{workload}")
    if not entry or entry.get("source_sha") != source_hash(stage):
        return None
    return entry["hbm_bytes_per_launch"]


def counter_pass(args, torch, qsa, synth):
    """Counter pass for rocprofv3 --pmc: one whole step so every stage's inputs
    are in place, a plain device-to-device copy of COPY_BYTES run --reps times
    (the calibration of the byte counters), then each --only stage --reps
    times."""
    w = synth.make_workload(args.workload)
    d = Device(w, torch, qsa)
    d.pool_prep(); d.score(); d.select()
    src = torch.full((COPY_BYTES,), 1, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    fns = {"pool": d.pool, "prep": d.prep, "pool_prep": d.pool_prep, "score": d.score, "select": d.select}
    stages = [s for s in args.only.split(",") if s]
    for st in stages:
        for _ in range(args.reps):
            fns[st]()
        torch.cuda.synchronize()
    print(json.dumps({"counter_pass": w["name"], "stages": stages, "reps": args.reps,
                      "copy_bytes": COPY_BYTES, "status": qsa.check_status(d.status)}))


def _counter_rows(run_dir: str, counter: str):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {run_dir}")
    return rows


def traffic_table(fetch_dir: str, write_dir: str, workload: int):
    """profiles/traffic.json from two counter passes: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch) of each stage's kernel, each scaled by bytes / counter of
    the calibration copy (the largest device-to-device copy dispatches), medians
    over the dispatches."""
    import synth
    name = synth.WORKLOADS[workload]["name"]
    out_path = os.path.join(ROOT, "profiles", "traffic.json")
    table = {}
    if os.path.exists(out_path):
        with open(out_path) as f:
            table = json.load(f)
    per = {}
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(run_dir, counter)
        copies = [v for _, k, v in rows if "copyBuffer" in k]
        top = max(copies)
        cal = median([v for v in copies if v >= 0.5 * top])
        factor = COPY_BYTES / cal  # bytes per counter unit
        for st, frag in STAGE_KERNELS.items():
            names = sorted({k for _, k, _ in rows if stage_of(k, st)})
            if not names:
                continue
            # one launch of the stage: the median dispatch of each of its kernels
            total = sum(median([v for _, k, v in rows if k == name]) for name in names)
            n = min(sum(1 for _, k, _ in rows if k == name) for name in names)
            short = [name.replace("void ", "").replace("qsa::(anonymous namespace)::", "").split("(")[0]
                     for name in names]
            per.setdefault(st, {})[counter] = (total, factor, n, short)
    for st, c in per.items():
        if "FETCH_SIZE" not in c or "WRITE_SIZE" not in c:
            continue
        fk, ff, n1, names = c["FETCH_SIZE"]
        wk, wf, n2, _ = c["WRITE_SIZE"]
        rd, wr = fk * ff, wk * wf
        table[f"{st}:{name}"] = {
            "kernel": " + ".join(names), "fetch_kib": fk, "write_kib": wk,
            "fetch_bytes_per_unit": round(ff, 2), "write_bytes_per_unit": round(wf, 2),
            "dispatches": [n1, n2], "read_bytes": round(rd), "write_bytes": round(wr),
            "hbm_bytes_per_launch": round(rd + wr), "source_sha": source_hash(st)}
    with open(out_path, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({k: v["hbm_bytes_per_launch"] for k, v in table.items()}))


# ----------------------------------------------------------------------------
# CPU oracle baseline
# ----------------------------------------------------------------------------

def cpu_baseline(w, budget_s: float):
    import numpy as np
    import oracle as O
    T = w["tokens"]
    pos = w["pos"]
    rows_total = len(pos)
    t0 = time.perf_counter()
    pooled = O.pool_keys(w["raw_keys"], w["k_norm_w"], w["rotary_dim"], w["theta"], w["eps"])
    t_pool = time.perf_counter() - t0
    # score + select per row, on as many rows as the budget allows
    rng = np.random.default_rng(0)
    order = rng.permutation(rows_total)
    done, pairs, t_rows = 0, 0, 0.0
    cols = T // 4
    while done < rows_total and (t_pool + t_rows) < budget_s:
        r = order[done: done + 8]
        t1 = time.perf_counter()
        qhat = O.prep_queries(w["queries"][r], pos[r], w["q_norm_w"], w["rotary_dim"], w["theta"], w["eps"])
        sc = O.score_rows(qhat, pos[r], pooled, T)
        dense = np.zeros((len(r), cols), dtype=np.float32)
        for i, s in enumerate(sc):
            dense[i, : len(s)] = s
        O.select_mask(dense, cols, pos[r], T, w["budget"])
        t_rows += time.perf_counter() - t1
        pairs += int(sum(len(s) for s in sc))
        done += len(r)
    t_step = t_pool * done / rows_total + t_rows
    cores = len(os.sched_getaffinity(0))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": pairs / t_step, "unit": "pairs/s", "cores": cores, "kind": "oracle",
            "sample": (f"{w['name']}: oracle pool of all {T // 4} blocks ({t_pool:.2f} s, "
                       f"charged pro rata), then prep+score+select of {done} of {rows_total} "
                       f"rows ({pairs} pairs, {t_rows:.2f} s); numpy, f64 BLAS matmul over "
                       f"{cores} threads; {model}")}


# ----------------------------------------------------------------------------

def launch_us(fn, torch, reps: int = 20):
    """Per-launch microseconds of `fn` launched `reps` times back to back
    between one pair of HIP events, queued behind a busy GPU."""
    stream = torch.cuda.current_stream()
    for _ in range(3):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    prime(torch)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return round(a.elapsed_time(b) * 1e3 / reps, 3)


def cold_launch_us(fn, torch, reps: int = 8):
    """Median microseconds of one launch of `fn` between a HIP event pair,
    with L2 and the MALL flushed before each (includes the event pair's own
    GPU time, ~4.4 us)."""
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    fn()
    ts = []
    for _ in range(reps):
        flush_caches(flush)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    del flush
    ts.sort()
    return round(ts[len(ts) // 2], 3)


KV_DIM = 512     # synthetic attention K/V vector: 2 KV heads x head dim 256, bf16
PAGE_SIZE = 16   # tokens per cache page


def decode_next(d: Device, torch, qsa):
    """The decode consumers of the selection on one workload: the index-list
    selector and the K/V gather from a paged cache (seeded random K/V, pages
    in a random order) into contiguous scratch."""
    w = d.w
    budget = w["budget"]
    stride = budget + 3
    slots = -(-stride // PAGE_SIZE) * PAGE_SIZE
    idx = torch.empty((d.rows, stride), dtype=torch.int32, device="cuda:0")
    counts = torch.empty(d.rows, dtype=torch.int32, device="cuda:0")
    d.pool()
    d.prep()
    d.score()
    sel_us = launch_us(lambda: qsa.qsa_select_indices_ws(d.scores, d.cols, d.pos, d.T, budget, idx, counts,
                                                         d.status, d.ws), torch)
    n_pages = -(-d.T // PAGE_SIZE)
    g = torch.Generator(device="cuda:0")
    g.manual_seed(1000 + int(w.get("wid", 0)))
    kc = torch.randint(-(1 << 15), 1 << 15, (n_pages, PAGE_SIZE, KV_DIM), dtype=torch.int16, device="cuda:0",
                       generator=g)
    vc = torch.randint(-(1 << 15), 1 << 15, (n_pages, PAGE_SIZE, KV_DIM), dtype=torch.int16, device="cuda:0",
                       generator=g)
    table = torch.randperm(n_pages, device="cuda:0", generator=g).to(torch.int32)
    ko = torch.empty((d.rows, slots, KV_DIM), dtype=torch.int16, device="cuda:0")
    vo = torch.empty_like(ko)
    otab = torch.empty((d.rows, slots // PAGE_SIZE), dtype=torch.int32, device="cuda:0")
    gather = lambda: qsa.qsa_gather_kv(kc, vc, table, 0, n_pages, idx, counts, ko, vo, otab, d.status)
    g_us = launch_us(gather, torch)
    g_cold = cold_launch_us(gather, torch)
    if qsa.check_status(d.status) != 0:
        raise RuntimeError("device status set in the decode gather")
    n_sel_pre = int(counts.sum().item())
    gather_bytes = (4 * KV_DIM * n_sel_pre + 4 * KV_DIM * d.rows * slots
                    + 4 * d.rows * (stride + 1 + slots // PAGE_SIZE))
    graph_fig = decode_graph(d, torch, qsa, idx, counts, kc, vc, table, n_pages, ko, vo, otab, gather_bytes)
    n_sel = int(counts.sum().item())
    alg = 4 * KV_DIM * n_sel + 4 * KV_DIM * d.rows * slots + 4 * d.rows * (stride + 1 + slots // PAGE_SIZE)
    gbs = alg / (g_us * 1e-6) / 1e9
    gbs_cold = alg / (g_cold * 1e-6) / 1e9
    del kc, vc, ko, vo
    # Back to back, the same lists re-read the same K/V, which partly stays in
    # the 256 MiB MALL (all of it for the 16-row batch): that figure is a
    # cache-warm rate.  The cold figure (caches flushed, one event pair
    # around the launch) bounds the HBM rate from below.
    return {"select_indices_us": sel_us,
            "kv_gather": {"us": g_us, "us_cold": g_cold, "kv_dim": KV_DIM, "page_size": PAGE_SIZE,
                          "slots": slots, "entries": n_sel, "alg_bytes": alg, "achieved_GBs": round(gbs, 1),
                          "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                          "achieved_GBs_cold": round(gbs_cold, 1),
                          "hbm_frac_cold": round(gbs_cold / HBM_PEAK_GBS, 4)},
            "decode_step": graph_fig}


def decode_graph(d: Device, torch, qsa, idx, counts, kc, vc, table, n_pages, ko, vo, otab, gather_bytes):
    """One production decode step with the cache length in a device word:
    pool the block the new token completed and prep the queries (one
    launch), score, index-list select, K/V gather.  Timed as eager launches and as one captured HIP graph
    replayed back to back (positions and cache fixed; each replay redoes the
    same step), and cold (caches flushed before each step, one event pair
    around it), with the step's algorithmic bytes: one pooled block, the
    queries, the score stage's bytes, the scores read and index lists
    written by the select, and the gather's bytes."""
    w = d.w
    rd, th, eps = w["rotary_dim"], w["theta"], w["eps"]
    dt = torch.full((1,), d.T, dtype=torch.int32, device="cuda:0")

    def step():
        qsa.qsa_pool_prep_dev(d.raw, d.wk, d.q, d.pos, d.wq, rd, th, eps, dt, 1, d.pooled, d.qhat, d.status)
        qsa.qsa_score_prepped_dev(d.qhat, d.pos, d.pooled, dt, d.T, d.scores, d.cols, d.status)
        qsa.qsa_select_indices_dev(d.scores, d.cols, d.pos, dt, d.T, w["budget"], idx, counts, d.status, d.ws)
        qsa.qsa_gather_kv(kc, vc, table, 0, n_pages, idx, counts, ko, vo, otab, d.status)

    eager_us = launch_us(step, torch)
    cold_us = cold_launch_us(step, torch)
    stride = idx.shape[1]
    alg = (4 * 256 + 256 + d.prep_bytes() + d.score_bytes() + 4 * d.pairs
           + d.rows * (4 * stride + 4) + gather_bytes)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    replay_us = launch_us(graph.replay, torch)
    if qsa.check_status(d.status) != 0:
        raise RuntimeError("device status set in the captured decode step")
    del graph
    return {"stages": "pool_prep(1 block + queries) + score + select_indices + gather",
            "eager_us": eager_us, "graph_replay_us": replay_us, "cold_us": cold_us, "alg_bytes": alg,
            "hbm_frac_eager": round(alg / (eager_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "hbm_frac_cold": round(alg / (cold_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def fused_prefill(d: Device, torch, qsa):
    """qsa_score_select_mask (score -> select without the score matrix) on
    the main workload, beside the two-call path it replaces; masks compared."""
    budget = d.w["budget"]
    n = qsa.qsa_score_select_workspace_bytes(d.rows, d.T, budget)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    mask = torch.empty_like(d.mask)
    d.pool()
    d.prep()
    fused_us = launch_us(lambda: qsa.qsa_score_select_mask(d.qhat, d.pos, d.pooled, d.T, budget, mask, d.status,
                                                           ws), torch, reps=10)

    def two():
        d.score()
        d.select()
    sep_us = launch_us(two, torch, reps=10)
    same = bool(torch.equal(mask, d.mask))
    del ws, mask
    torch.cuda.empty_cache()
    return {"fused_us": fused_us, "score_then_select_us": sep_us, "masks_equal": same,
            "workspace_bytes": n}


def side_figures(torch, qsa, synth):
    """The 4096-row prefill over 4k tokens, select+mask us/row on the 64k/256k
    decode workloads and the one-row 64k/256k shapes: per-kernel event means over 20 launches after 5 warm-ups
    (each launch between its own event pair), per-kernel back-to-back launch
    times, and the cold-cache step with its aggregate HBM fraction."""
    out = {"launch_floor_us": launch_floor_us(torch)}
    for key, w in (("prefill_4k", synth.make_workload(2)),
                   ("decode_64k_x64", synth.make_workload(3)),
                   ("decode_256k_x16", synth.make_workload(4)),
                   ("one_row_64k", synth.single_row(3, 65535)),
                   ("one_row_256k", synth.single_row(4, 262143))):
        d = Device(w, torch, qsa)
        per = event_steps(d, 20, 5, torch, kernel_stages(d))
        rep, mean = kernel_report(d, per)
        b2b = back_to_back_us(d, torch)
        cold, floor = cold_step_us(d, torch)
        step = [n for n, _ in step_stages(d)]
        alg = d.pool_prep_bytes() + d.score_bytes() + d.select_bytes()
        out[key] = {"rows": d.rows, "tokens": d.T, "pairs": d.pairs,
                    "select_mask_us_per_row": round(b2b["select"] / d.rows, 3),
                    "step_kernels": step,
                    "step_us_events": round(sum(mean[n] for n in step), 2),
                    "step_us_back_to_back": round(sum(b2b[n] for n in step), 2),
                    "step_us_cold": cold,
                    "event_pair_floor_us": floor,
                    "alg_bytes_step": alg,
                    "hbm_frac_back_to_back": round(alg / (sum(b2b[n] for n in step) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "hbm_frac_cold_step": round(alg / (cold * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "pairs_per_s": round(d.pairs / (sum(b2b[n] for n in step) * 1e-6), 1),
                    "kernels_back_to_back_us": b2b,
                    "kernels": rep}
        if key != "prefill_4k":  # decode consumers of the selection
            out[key].update(decode_next(d, torch, qsa))
        progress(f"side workload {key} measured")
        del d
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.traffic_from:
        traffic_table(args.traffic_from[0], args.traffic_from[1], args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the indexer path here "
              f"is a single-GPU kernel set with no cross-GPU sharding.", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_attention_token_qsa_amd as qsa
    import synth

    qsa.load()
    if args.only:
        counter_pass(args, torch, qsa, synth)
        return
    w = synth.make_workload(args.workload)
    d = Device(w, torch, qsa)
    wall, per, dom = time_steps(d, args.steps, args.warmup, torch)
    progress(f"{args.steps} timed steps done")
    st = qsa.check_status(d.status)
    if st != 0:
        raise RuntimeError(f"device status {st} on a clean workload")
    rep, mean = kernel_report(d, per)
    ms_per_step = wall / args.steps * 1e3
    value = d.pairs / (wall / args.steps)

    # dominant kernel (timed with events over the timed steps) and its roofline
    if dom == "score":
        t_hbm = d.score_bytes() / (HBM_PEAK_GBS * 1e9)
        t_mfma = d.score_flops() / (MFMA_BF16_PEAK_TFS * 1e12)
        bound = "mfma" if t_mfma > t_hbm else "hbm"
    else:
        bound = "hbm"
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": rep["score"]["achieved_TFs"], "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": rep["score"]["mfma_frac"]}
    else:
        roof = {"bound": "hbm", "achieved": rep[dom]["achieved_GBs"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": rep[dom]["hbm_frac"]}
    roof["kernel"] = dom
    roof["traffic"] = traffic_for(dom, w["name"])

    side = {} if args.no_side else side_figures(torch, qsa, synth)
    fused = None if args.no_side else fused_prefill(d, torch, qsa)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_seconds)
    progress("cpu baseline done")

    line = {
        "metric": "scored (row,block) pairs/s + select+mask us/row at 64k and 256k ctx",
        "value": round(value, 1),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w["name"], "rows": d.rows, "tokens": d.T, "budget": w["budget"],
                   "heads": 4, "head_dim": 128, "rotary_dim": w["rotary_dim"],
                   "pairs_per_step": d.pairs, "parallelism": "single-gpu"},
        "select_mask_us_per_row": {
            "64k": side.get("decode_64k_x64", {}).get("select_mask_us_per_row"),
            "256k": side.get("decode_256k_x16", {}).get("select_mask_us_per_row"),
            "one_row_64k": side.get("one_row_64k", {}).get("select_mask_us_per_row"),
            "one_row_256k": side.get("one_row_256k", {}).get("select_mask_us_per_row"),
            "main_workload": round(mean["select"] / d.rows, 4),
        },
        "kernels": rep,
        "kernel_timing": f"{dom}: HIP events over the timed steps; the others: HIP events around every "
                         "kernel in 300 steps after them",
        "roofline": roof,
        "side_workloads": side,
        "fused_score_select": fused,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
