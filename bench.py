"""Benchmark of the eviction round on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workloads batch,paged,...] [--no-cpu-baseline]

A step is one whole eviction round (score -> pin + select -> compact) over one
batch of synthetic inputs resident in HBM.  The headline workload is the
decode-time batch round (128 requests x 36 layers x 8 KV heads, D=128,
n=1088, K=1024, prot=128, contiguous storage, per-head random draw).  By
default the other configurations are timed too and reported under
"workloads": the tiny round, the paged round in per-head and shared-draw
modes, the GateSight-shaped global round and the 30-round long generation
(exactly its 30 rounds after the warmup, with the survival curve).  Prints
ONE JSON line.

Timing: W untimed rounds, then exactly K rounds between two synchronisations;
HIP events on the launch stream bracket every kernel launch of the round, so
each step of the round gets its own average duration.  Every workload carries
a roofline entry for its dominant kernel, the K/V gather, priced at its
algorithmic bytes (the kept K and V rows, each read once and written once),
with the HBM bytes its FETCH_SIZE/WRITE_SIZE counters measured
(profiles/gather_traffic.json, null once the gather's source has changed).
Workloads whose round takes under 1 ms and leaves its inputs intact are also
replayed from a HIP graph of ten rounds (graph_ms_per_round).  Out-of-place
rounds are also timed over selection + compaction alone as one interval
(select_compact: eager, and from a HIP graph), with no event between the
select and the gather.  The paged rounds carry a ceiling: a plain copy of the
same bytes, whole pages through the same random page tables.

    python bench.py --summarize-traffic WORKLOAD FETCH.csv WRITE.csv

folds the per-dispatch counters of two rocprofv3 --pmc runs (FETCH_SIZE, then
WRITE_SIZE) of `bench.py --profile-workload WORKLOAD` into
profiles/gather_traffic.json, scaled by a plain copy's counters
(`--summarize-traffic copy` over two runs of `bench.py --copy-calibration`).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
METRIC = "eviction rounds/sec and achieved HBM GB/s (fraction of peak) per MI355X"
TRAFFIC_FILE = os.path.join(HERE, "profiles", "gather_traffic.json")
COMPACT_SRC = os.path.join(HERE, "kv_cache_eviction_05_amd", "csrc", "compact.hip")
DEFAULT_WORKLOADS = "batch,tiny,paged,paged_shared,global,longgen"
ALL_WORKLOADS = ["batch", "tiny", "paged", "paged_shared", "global", "global_fused", "longgen",
                 "layers", "paged_shared_max", "keydiff", "paged_inplace", "longgen_inplace",
                 "paged_fused", "longgen_fused", "paged_pages", "paged_single"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workloads", default=DEFAULT_WORKLOADS,
                    help="comma list of workload names from configs.ALL (or 'all'); the "
                         "headline batch round is always timed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for PMC scaling)")
    ap.add_argument("--profile-workload", default=None,
                    help="time this one workload only (no headline, no baselines): the "
                         "process that rocprofv3 counter runs wrap")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV"),
                    help="fold two rocprofv3 --pmc counter files into " + TRAFFIC_FILE)
    return ap.parse_args()


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def describe(cfg) -> str:
    layout = "paged 16-token pages" if cfg.layout == "paged" else "contiguous"
    if cfg.select in ("global", "layers"):
        rule = ("global top-B" if cfg.select == "global"
                else "gate-proportional per-layer top-K_l at the same total")
        if cfg.fuse_score:
            rule += " (score and top-B in one call, the scorer filling the first radix level)"
        return (f"{cfg.name}: {cfg.L} layers x {cfg.H} KV heads, D={cfg.D}, n={cfg.n}, "
                f"prot={cfg.prot}, p={cfg.p}, weighted GDN score over 48 GDN layers x 48 heads, "
                f"{rule}, {layout}")
    if cfg.inplace:
        layout += ", compacted in place (unchanged prefix stays, freed pages to a list)"
    if cfg.fused:
        layout += ", draw + top-K + move in one launch"
    if cfg.page_draw:
        return (f"{cfg.name}: {cfg.R} requests x {cfg.L} layers x {cfg.H} KV heads, D={cfg.D}, "
                f"n={cfg.n}, K={cfg.K}, prot={cfg.prot}, paged {cfg.page_size}-token pages, "
                f"one random draw per page and (request, layer), whole pages kept, compaction "
                f"as page-table edits (no K/V bytes move)")
    draw = ("shared draw per layer" if cfg.shared else
            "one list per layer by the max of per-head random scores, kept count a multiple of 4"
            if cfg.shared_max else
            "KeyDiff scores (-cosine to the head's mean key)" if cfg.scorer == "keydiff" else
            "per-head random draw")
    return (f"{cfg.name}: {cfg.R} requests x {cfg.L} layers x {cfg.H} KV heads, D={cfg.D}, "
            f"n={cfg.n}, K={cfg.K}, prot={cfg.prot}, {layout}, {draw}"
            + (f", {cfg.rounds} rounds with r={cfg.r} appended" if cfg.rounds > 1 else ""))


class Timer:
    """HIP events on the launch stream around each step of the round."""

    def __init__(self, torch, names):
        self.torch = torch
        self.names = names
        self.marks = []

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.marks.append(e)

    def per_step_ms(self, steps):
        """Average duration of each named interval over `steps` rounds."""
        k = len(self.names)
        tot = [0.0] * k
        for s in range(steps):
            base = s * (k + 1)
            for i in range(k):
                tot[i] += self.marks[base + i].elapsed_time(self.marks[base + i + 1])
        return {n: t / steps for n, t in zip(self.names, tot)}

    def step_ms(self, steps):
        """Duration of each round, first launch to last, from the same events."""
        k = len(self.names)
        return [self.marks[s * (k + 1)].elapsed_time(self.marks[s * (k + 1) + k])
                for s in range(steps)]


def percentiles(xs):
    """p10, p50 and p90 of a list (nearest rank)."""
    ys = sorted(xs)
    pick = lambda q: ys[min(len(ys) - 1, max(0, int(round(q * (len(ys) - 1)))))]
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


def time_workload(torch, rounds, cfg, steps, warmup):
    st = rounds.make_state(cfg, "cuda")
    phases = rounds.phases(cfg)
    torch.cuda.synchronize()
    round_id = 0
    survival = None
    if cfg.rounds > 1:
        # repeated rounds: after the warmup rounds, exactly cfg.rounds rounds of the
        # persistent-budget loop are timed, one step each, and the survival curve follows
        # the entries present when they start; the append of r fresh tokens between rounds
        # is input synthesis and stays untimed, and so does the survival bookkeeping on
        # sampled lists
        steps = cfg.rounds
        for _ in range(warmup):
            rounds.run_round(st, round_id)
            rounds.append_tokens(st, round_id)
            rounds.swap(st)
            round_id += 1
        torch.cuda.synchronize()
        survival = rounds.SurvivalTracker(st)
        timer = Timer(torch, [name for name, _ in phases])
        total_ms = 0.0
        for _ in range(steps):
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            timer.mark()
            for _, fn in phases:
                fn(st, round_id)
                timer.mark()
            t1.record()
            st.applied_rounds += 1
            survival.after_round(st)
            rounds.append_tokens(st, round_id)
            rounds.swap(st)
            round_id += 1
            torch.cuda.synchronize()
            total_ms += t0.elapsed_time(t1)
        ms_per = total_ms / steps
    elif cfg.inplace:
        # one round in place: the cache is restored before every round, untimed
        for _ in range(warmup):
            rounds.restore(st)
            rounds.run_round(st, 0)
        timer = Timer(torch, [name for name, _ in phases])
        total_ms = 0.0
        for s in range(steps):
            rounds.restore(st)
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            timer.mark()
            for _, fn in phases:
                fn(st, s)
                timer.mark()
            t1.record()
            st.applied_rounds += 1
            torch.cuda.synchronize()
            total_ms += t0.elapsed_time(t1)
        ms_per = total_ms / steps
    else:
        for _ in range(warmup):
            rounds.run_round(st, 0)
        torch.cuda.synchronize()
        timer = Timer(torch, [name for name, _ in phases])
        t_start = time.perf_counter()
        for s in range(steps):
            timer.mark()
            for _, fn in phases:
                fn(st, s)
                timer.mark()
            st.applied_rounds += 1
        torch.cuda.synchronize()
        ms_per = (time.perf_counter() - t_start) * 1e3 / steps
    kern = timer.per_step_ms(steps)
    dist = percentiles(timer.step_ms(steps))
    kv_bytes = st.kv_bytes_moved()
    errors = int(st.errors.item())
    out = {"state": st, "ms_per_step": ms_per, "kernels_ms": kern, "kv_bytes": kv_bytes,
           "round_ms_dist": dist, "algorithmic_bytes": st.algorithmic_bytes(), "steps": steps,
           "errors": errors, "applied_rounds": st.applied_rounds - warmup,
           "budget": st.budget, "survival": survival.report(st) if survival else None}
    return out


GRAPH_ROUNDS = 10  # rounds recorded per HIP graph


def graph_replay_ms(torch, rounds, st, steps):
    """Round time with the rounds replayed from a HIP graph of GRAPH_ROUNDS rounds (round
    ids 0..GRAPH_ROUNDS-1): the same launches without the host launch path, which rounds
    of tens of microseconds are bound by."""
    g = rounds.capture_rounds(st, range(GRAPH_ROUNDS))
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // GRAPH_ROUNDS)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (reps * GRAPH_ROUNDS)


SELECT_PHASES = ("select", "draw_select", "compact")


def select_compact_ms(torch, rounds, st, steps):
    """Selection + compaction (every phase of the round after a standalone scorer) timed as
    one interval, with no event between the select and the gather: eager, `steps`
    repetitions between two events; and replayed from a HIP graph of GRAPH_ROUNDS
    repetitions, which also takes the host launch path out.  The scores stay those of
    the last full round, so every repetition does the same work."""
    fns = [fn for name, fn in rounds.phases(st.cfg) if name in SELECT_PHASES]
    for s in range(2):
        for fn in fns:
            fn(st, s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(steps):
        for fn in fns:
            fn(st, s)
    e1.record()
    torch.cuda.synchronize()
    eager = e0.elapsed_time(e1) / steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(GRAPH_ROUNDS):
            for fn in fns:
                fn(st, s)
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // GRAPH_ROUNDS)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return eager, e0.elapsed_time(e1) / (reps * GRAPH_ROUNDS)


GATHER_KERNELS = ("compact_list_kernel", "compact_group_kernel")


def load_traffic() -> dict:
    try:
        with open(TRAFFIC_FILE) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {}


def traffic_for(name):
    """Measured HBM bytes per launch of a workload's gather, if its counters were taken on
    the gather's current source (else None: the kernel changed since)."""
    t = load_traffic().get("workloads", {}).get(name)
    if not t or t.get("source_sha256_16") != source_hash(COMPACT_SRC):
        return None
    return t.get("bytes_per_launch")


def read_counter_csv(path, counter, match):
    """Per-dispatch sums of `counter` (KiB) over the dispatches whose kernel name contains
    one of `match`, from a rocprofv3 counter_collection.csv."""
    import csv

    per = {}
    names = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter or not any(m in row["Kernel_Name"] for m in match):
                continue
            d = row["Dispatch_Id"]
            per[d] = per.get(d, 0.0) + float(row["Counter_Value"])
            names[d] = row["Kernel_Name"]
    return per, names


def summarize_traffic(name, fetch_csv, write_csv):
    """Fold two counter runs into TRAFFIC_FILE: the plain copy's scale factors (name
    'copy', over runs of --copy-calibration: 3 copies of 4 GiB), or a workload's gather
    bytes per launch (over runs of --profile-workload), scaled by those factors."""
    t = load_traffic()
    if name == "copy":
        f, _ = read_counter_csv(fetch_csv, "FETCH_SIZE", ("copyBuffer",))
        w, _ = read_counter_csv(write_csv, "WRITE_SIZE", ("copyBuffer",))
        big = lambda d: [v for v in d.values() if v > 1e6]  # the 4 GiB copies, not set-up fills
        fk, wk = big(f), big(w)
        copied = 4 << 30
        t["copy_calibration"] = {
            "bytes": copied, "dispatches": [len(fk), len(wk)],
            "fetch_kib": sum(fk) / len(fk), "write_kib": sum(wk) / len(wk),
            "fetch_scale": copied / (1024 * sum(fk) / len(fk)),
            "write_scale": copied / (1024 * sum(wk) / len(wk)),
            "commands": {c: f"rocprofv3 --pmc {c} --output-format csv -d <dir> -- "
                            f"python3 bench.py --copy-calibration" for c in ("FETCH_SIZE",
                                                                                "WRITE_SIZE")}}
    else:
        cal = t["copy_calibration"]
        f, names = read_counter_csv(fetch_csv, "FETCH_SIZE", GATHER_KERNELS)
        w, _ = read_counter_csv(write_csv, "WRITE_SIZE", GATHER_KERNELS)
        fb = 1024 * cal["fetch_scale"] * sum(f.values()) / len(f)
        wb = 1024 * cal["write_scale"] * sum(w.values()) / len(w)
        t.setdefault("workloads", {})[name] = {
            "kernel": sorted(set(names.values()))[0],
            "source": os.path.relpath(COMPACT_SRC, HERE),
            "source_sha256_16": source_hash(COMPACT_SRC),
            "dispatches": [len(f), len(w)],
            "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
            "bytes_per_launch": fb + wb,
            "commands": {c: f"rocprofv3 --pmc {c} --output-format csv -d <dir> -- "
                            f"python3 bench.py --profile-workload {name} --steps 2 --warmup 0"
                         for c in ("FETCH_SIZE", "WRITE_SIZE")}}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(t, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(t.get("workloads", {}).get(name, t.get("copy_calibration"))))


def roofline(name, cfg, kv_bytes, comp_ms):
    """The workload's dominant kernel, the K/V gather, against the HBM peak."""
    achieved = kv_bytes / (comp_ms * 1e-3) / 1e9
    kernel = ("compact_group_kernel (paged K/V gather)" if cfg.layout == "paged" else
              "compact_list_kernel (contiguous K/V gather)")
    return {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic_for(name),
            "algorithmic_bytes": kv_bytes, "ms": round(comp_ms, 4)}


def paged_copy_ceiling(torch, binding, st, cfg, gather_gbps, reps=5):
    """A plain copy of the paged gather's bytes through the same random page tables: every
    destination page of the round filled whole, K and V, from the source page its group's
    table holds at the same position (kvevict_copy_pages), in page-table order and in the
    order the gather walks them (destination pages in increasing physical order, each of the
    eight XCDs taking one contiguous range; the order is set up untimed).  Overwrites the
    destination."""
    kp = cfg.K // cfg.page_size
    src_ids = st.src_pt[:, :kp].reshape(-1).contiguous()
    dst_ids = st.dst_pt[:, :kp].reshape(-1).contiguous()
    o = torch.argsort(dst_ids)
    m = o.numel() // 8 * 8
    o = torch.cat([o[:m].view(8, -1).t().reshape(-1), o[m:]])  # workgroup b on XCD b % 8
    page_bytes = cfg.page_size * cfg.H * cfg.D * 2
    moved = 2 * 2 * src_ids.numel() * page_bytes  # K and V, read and written
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {"bytes_moved": moved}
    for label, s_ids, d_ids in (("table_order", src_ids, dst_ids),
                                ("physical_order", src_ids[o].contiguous(), dst_ids[o].contiguous())):
        run = lambda: binding.kvevict_copy_pages(st.k_src, st.v_src, s_ids, st.k_dst, st.v_dst,
                                                 d_ids, page_bytes, err)
        run()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbps = moved / (ms * 1e-3) / 1e9
        out[label] = {"ms": round(ms, 4), "gbps": gbps, "frac_of_peak": gbps / PEAK_HBM_GBPS,
                      "gather_vs_copy": gather_gbps / gbps}
    out["bad_pages"] = int(err.item())
    return out


def contig_copy_ceiling(torch, binding, st, gather_gbps, reps=10):
    """A plain copy of the gather's bytes between the same K and V stores: the leading
    kv_bytes / 4 bytes of each source store copied whole to its destination store in 32 KiB
    pieces with kvevict_copy_pages (identity piece lists), so that reads and writes are
    contiguous.  The ceiling for a gather of this many bytes, launch ramp and drain included;
    the gather's scattered rows can approach it but not pass it.  Overwrites the destination."""
    piece = 32 << 10
    count = st.kv_bytes_moved() // 4 // piece
    ids = torch.arange(count, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    moved = 4 * count * piece  # K and V, read and written
    run = lambda: binding.kvevict_copy_pages(st.k_src, st.v_src, ids, st.k_dst, st.v_dst, ids,
                                             piece, err)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbps = moved / (ms * 1e-3) / 1e9
    return {"bytes_moved": moved, "ms": round(ms, 4), "gbps": gbps,
            "frac_of_peak": gbps / PEAK_HBM_GBPS, "gather_vs_copy": gather_gbps / gbps,
            "bad_pages": int(err.item())}


def cpu_baseline(torch, cfg, st, seconds):
    """The oracle timed on the host cores over a bounded sample of the same workload."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    threads = max(1, min(16, os.cpu_count() or 1))
    req = max(1, min(cfg.R, 16))
    lists = req * cfg.L * cfg.H
    ks = st.k_src[:lists].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    vs = st.v_src[:lists].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    kd = np.zeros((lists, cfg.K, cfg.D), np.uint16)
    vd = np.zeros_like(kd)
    groups = lists // cfg.H
    bounds = [groups * t // threads for t in range(threads + 1)]

    def part(t):
        g0, g1 = bounds[t], bounds[t + 1]
        if g1 <= g0:
            return
        l0, l1 = g0 * cfg.H, g1 * cfg.H
        s = oracle.score_random(cfg.L, cfg.H, cfg.n, cfg.prot, cfg.seed, 0, False, l0, l1)
        kept = oracle.select_topk(s, cfg.K, cfg.prot)
        # the slices [l0, l1) are whole groups of H lists, addressed from their own base
        oracle.compact({"list_stride": cfg.n * cfg.D}, ks[l0:l1], vs[l0:l1],
                       {"list_stride": cfg.K * cfg.D}, kd[l0:l1], vd[l0:l1], kept, cfg.K, cfg.D,
                       cfg.H, 0, g1 - g0, ipg=cfg.H)

    reps = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            list(ex.map(part, range(threads)))
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
    el = time.perf_counter() - t0
    frac = lists / cfg.lists
    return {"value": reps * frac / el, "unit": "rounds/s", "cores": threads, "kind": "oracle",
            "sample": f"{req} of {cfg.R} requests ({lists} of {cfg.lists} lists: score, select, "
                      f"compact) x {reps} repetitions in {el:.1f} s on {threads} threads",
            "cpu_model": cpu_model()}


def device_info(torch) -> dict:
    """What the runtime reports for the GPU the bench ran on."""
    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", None),
            "compute_units": pr.multi_processor_count,
            "hbm_bytes": pr.total_memory,
            "l2_bytes": getattr(pr, "L2_cache_size", None)}


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_single_thread(torch, cfg, st, min_seconds=2.0):
    """The oracle on one host thread over the whole round of a small workload (the tiny
    round, or the global round: weighted score, global top-B and compaction), on the same
    inputs, downloaded first (download untimed)."""
    import numpy as np

    import oracle

    def bits(t):
        return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    ks, vs = bits(st.k_src), bits(st.v_src)
    kd = np.zeros(tuple(st.k_dst.shape), np.uint16)
    vd = np.zeros_like(kd)
    if cfg.select == "global":
        beta, vnorm = st.beta.cpu().numpy(), st.vnorm.cpu().numpy()
        w = st.weights.cpu().numpy()

        def one_round():
            s = oracle.score_weighted(beta, vnorm, w, *oracle.gdn_windows(cfg.L, cfg.G, cfg.win_width),
                                      cfg.prot)
            kept, counts, _ = oracle.select_global(s, cfg.prot, cfg.p)
            oracle.compact({"list_stride": cfg.n * cfg.D}, ks, vs, {"list_stride": cfg.n * cfg.D},
                           kd, vd, kept, cfg.n, cfg.D, cfg.H, 0, cfg.groups, ipg=cfg.H,
                           kept_count=counts)
        what = "weighted score, global top-B and compaction"
    else:
        def one_round():
            s = oracle.score_random(cfg.L, cfg.H, cfg.n, cfg.prot, cfg.seed, 0, False, 0,
                                    cfg.lists)
            kept = oracle.select_topk(s, cfg.K, cfg.prot)
            oracle.compact({"list_stride": cfg.n * cfg.D}, ks, vs, {"list_stride": cfg.K * cfg.D},
                           kd, vd, kept, cfg.K, cfg.D, cfg.H, 0, cfg.groups, ipg=cfg.H)
        what = "random score, top-K and compaction"
    reps = 0
    t0 = time.perf_counter()
    while True:
        one_round()
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    el = time.perf_counter() - t0
    return {"value": reps / el, "unit": "rounds/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole round ({what}) x {reps} in {el:.1f} s on 1 thread",
            "cpu_model": cpu_model()}


def dtod_copy(torch, kv_bytes, gather_gbps, reps=5):
    """A plain device-to-device copy moving the same bytes as the gather (half read, half
    written): the ceiling a gather of contiguous rows could reach, and the gather's ratio."""
    half = kv_bytes // 2
    a = torch.empty(half, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbps = 2 * half / (ms * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return {"bytes_moved": 2 * half, "ms": round(ms, 4), "gbps": gbps,
            "gather_vs_copy": gather_gbps / gbps}


def copy_calibration(torch):
    """A plain device-to-device copy of 4 GiB: reference for scaling FETCH/WRITE counters."""
    n = 4 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)


def measure(torch, binding, configs, rounds, name, args, headline):
    """Times one workload and returns its entry (and the state, for the baselines)."""
    cfg = configs.ALL[name]
    print(f"# timing {name}", file=sys.stderr, flush=True)
    r = time_workload(torch, rounds, cfg, args.steps, args.warmup)
    steps = r["steps"]
    main_phase = "pages" if cfg.page_draw else "fused" if cfg.fused else "compact"
    comp_ms = r["kernels_ms"][main_phase]
    achieved = r["kv_bytes"] / (comp_ms * 1e-3) / 1e9
    entry = {
        "workload": describe(cfg),
        "rounds_per_s": 1e3 / r["ms_per_step"],
        "ms_per_round": r["ms_per_step"],
        "steps": steps,
        "kernel_ms": {k: round(v, 4) for k, v in r["kernels_ms"].items()},
        "kv_bytes_per_round": r["kv_bytes"],
        "kv_gbps_round": r["kv_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9,
        "compact_gbps": achieved if not cfg.page_draw else None,
        "compact_frac_of_peak": achieved / PEAK_HBM_GBPS if not cfg.page_draw else None,
        "round_ms_p10_p50_p90": [round(r["round_ms_dist"][q], 4) for q in ("p10", "p50", "p90")],
        "algorithmic_bytes_per_round": r["algorithmic_bytes"],
        "applied_rounds": r["applied_rounds"],
        "bad_rows": r["errors"],
    }
    if not cfg.page_draw:
        entry["roofline"] = roofline(name, cfg, r["kv_bytes"], comp_ms)
    if cfg.scorer in ("weighted", "keydiff") and "score" in r["kernels_ms"]:
        # the scorer as it runs in the round: its inputs (GDN signals, or the keys) read
        # once and the scores written once (keys a KeyDiff kernel reads a second time are
        # not algorithmic bytes; the round's score bytes count the select's read as well).
        # KeyDiff lists of at most 1088 keys at D = 128 in a contiguous store are held on
        # chip whole by their own kernel.
        lists = cfg.L * cfg.H * cfg.R
        sb = r["algorithmic_bytes"]["inputs"] + (
            lists * r["state"].n * 4 if cfg.scorer == "weighted"
            else r["algorithmic_bytes"]["scores"] // 2)
        ms = r["kernels_ms"]["score"]
        sg = sb / (ms * 1e-3) / 1e9
        entry["roofline_score"] = {
            "bound": "hbm",
            "kernel": ("score_weighted_lds_kernel" if cfg.scorer == "weighted"
                       else "score_keydiff_resident_kernel"
                       if cfg.D == 128 and cfg.n <= 1088 and cfg.layout == "contig"
                       else "score_keydiff_kernel"),
            "achieved": sg, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": sg / PEAK_HBM_GBPS,
            "algorithmic_bytes": sb, "ms": round(ms, 4)}
    st = r["state"]
    if r["ms_per_step"] < 1.0 and not (cfg.inplace or cfg.page_draw or cfg.rounds > 1):
        # latency-bound rounds: also replayed from a HIP graph
        g_ms = graph_replay_ms(torch, rounds, st, max(steps, 10 * GRAPH_ROUNDS))
        entry["graph_ms_per_round"] = g_ms
        entry["graph_rounds_per_s"] = 1e3 / g_ms
    if (not (cfg.inplace or cfg.page_draw or cfg.fused or cfg.fuse_score)
            and any(p in ("select", "draw_select") for p, _ in rounds.phases(cfg))):
        sc_eager, sc_graph = select_compact_ms(torch, rounds, st, max(steps, 20))
        entry["select_compact"] = {
            "ms": round(sc_eager, 4), "graph_ms": round(sc_graph, 4),
            "kv_gbps": r["kv_bytes"] / (sc_eager * 1e-3) / 1e9,
            "frac_of_peak": r["kv_bytes"] / (sc_eager * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "frac_of_peak_graph": r["kv_bytes"] / (sc_graph * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        }
    if cfg.select in ("global", "layers"):
        entry["budget"] = r["budget"]
    if cfg.select == "layers":
        entry["vs_global_top_b"] = rounds.compare_with_global(st)
    if cfg.page_draw:
        P, Kp = cfg.n // cfg.page_size, cfg.K // cfg.page_size
        entry["pages_evicted_per_round"] = cfg.groups * (P - Kp)
        entry["table_bytes_per_round"] = cfg.groups * (P * 4 * 2 + (P - Kp) * 4)
    if r["survival"] is not None:
        entry["survival"] = r["survival"]
    if args.profile_workload is None:
        if name in ("tiny", "global") and not args.no_cpu_baseline:
            print(f"# cpu baseline on one thread (oracle): {name}", file=sys.stderr, flush=True)
            entry["cpu_baseline_1_thread"] = cpu_single_thread(torch, cfg, st)
        if headline:
            entry["dtod_copy"] = dtod_copy(torch, r["kv_bytes"], achieved)
            if not args.no_cpu_baseline:
                print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
                entry["cpu"] = cpu_baseline(torch, cfg, st, args.cpu_seconds)
        if cfg.layout == "paged" and not (cfg.inplace or cfg.page_draw):
            # last: the copy overwrites the round's destination pages
            entry["page_copy_ceiling"] = paged_copy_ceiling(torch, binding, st, cfg, achieved)
        if cfg.select in ("global", "layers") and cfg.layout == "contig" and not cfg.inplace:
            # two same-size copies as the gather's ceiling: torch's device copy, and
            # (last: it overwrites the round's destination rows) the library's page copy
            entry["dtod_copy"] = dtod_copy(torch, r["kv_bytes"], achieved)
            entry["copy_ceiling"] = contig_copy_ceiling(torch, binding, st, achieved)
    del r["state"], st
    r.clear()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return cfg, entry


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(every list is independent, so throughput at N GPUs is N x the one-GPU value "
              f"under request sharding)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration:
        copy_calibration(torch)
        return
    from kv_cache_eviction_05_amd import binding, configs, rounds

    binding.load()
    if args.profile_workload is not None:
        _, e = measure(torch, binding, configs, rounds, args.profile_workload, args, False)
        print(json.dumps({"workload": args.profile_workload, "kernel_ms": e["kernel_ms"],
                          "roofline": e.get("roofline")}), flush=True)
        return
    names = [w for w in args.workloads.split(",") if w]
    if names == ["all"]:
        names = list(ALL_WORKLOADS)
    names = ["batch"] + [n for n in names if n != "batch"]
    head = None
    extra = {}
    for name in names:
        cfg, entry = measure(torch, binding, configs, rounds, name, args, name == "batch")
        if name == "batch":
            head = (cfg, entry)
        else:
            extra[name] = entry

    cfg, e = head
    line = {
        "metric": METRIC,
        "value": e["rounds_per_s"],
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": e["ms_per_round"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": e["workload"], "lists": cfg.lists, "n": cfg.n, "K": cfg.K,
                   "prot": cfg.prot, "head_dim": cfg.D},
        "kv_gbps": e["kv_gbps_round"],
        "kernel_ms": e["kernel_ms"],
        "roofline": e["roofline"],
        "round_ms_p10_p50_p90": e["round_ms_p10_p50_p90"],
        "select_compact": e.get("select_compact"),
        "algorithmic_bytes_per_round": e["algorithmic_bytes_per_round"],
        "dtod_copy": e["dtod_copy"],
        "cpu_baseline": e.get("cpu"),
        "bad_rows": e["bad_rows"],
        "device": device_info(torch),
    }
    if extra:
        line["workloads"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
