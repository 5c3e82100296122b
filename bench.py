#!/usr/bin/env python3
"""Benchmark of the serial-episode counting library on one MI355X.

One step = one ep_count_episodes call (every kernel of the scheme, plus its
scratch allocation and episode-table upload) over one batch of synthetic,
GPU-resident input.  Default workload: the long-chain stress configuration,
500,000,000 events over 256 types with bursty Gamma(0.5)-distributed gaps,
4 eight-node episodes with delays (0,3] .. (10,50], MapConcatenate over
65,536 segments.

Prints ONE JSON line: episode-events/s (events x episodes / step time), the
roofline of the dominant kernel measured live with HIP events (for the event
filter: one read of the stream, 6 B per event, against HBM), the whole call
as a fraction of one pass over the stream at HBM peak, and the CPU oracle
timed on a bounded sample of the same workload on the host cores.

--scheme upper counts the relaxed episodes (every lower delay bound 0);
--scheme two-pass runs the two-pass elimination for a support threshold (the
relaxed count of every episode, then the exact count of those reaching the
threshold): one step is then one ep_count_two_pass call.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X figures: 256 CUs x 4 SIMDs x 16 int32 lanes per clock x 2.4 GHz.
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
HBM_PEAK_GBS = 8000.0
# Algorithmic work of the counting machine per (episode, relevant event): the
# node-type test, the window check and the window update, ~10 int32 ops.
OPS_PER_RELEVANT_PAIR = 10
# the Map-step phases the library times, and the name profile_begin_kernel takes
PHASES = {"map_filter_ms": "filter", "map_prune_ms": "prune", "map_ticks_ms": "ticks",
          "map_positions_ms": "positions"}
# Device code of every kernel (host code is not hashed: a change there leaves
# the kernels and their traffic as they were).
KERNEL_SOURCES = ["frequent_episode_mining_amd/csrc/ep_device.hpp",
                  "frequent_episode_mining_amd/csrc/ep_inst.hip",
                  "frequent_episode_mining_amd/csrc/ep_kernels.hpp",
                  "frequent_episode_mining_amd/csrc/ep_slice.hpp"]


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def relevant_pairs(wl) -> int:
    """Sum over episodes of the events whose type sits on one of its nodes."""
    cnt = np.bincount(wl.types, minlength=65536).astype(np.int64)
    total = 0
    for row in wl.ep_types:
        total += int(cnt[np.unique(row)].sum())
    return total


def relevant_pairs_rows(wl, rows) -> int:
    cnt = np.bincount(wl.types, minlength=65536).astype(np.int64)
    return int(sum(int(cnt[np.unique(wl.ep_types[r])].sum()) for r in rows))


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the kernel from the committed counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_val or m_sha.group(1) != kernel_source_sha():
        return None
    return float(m_val.group(1))


def oracle_timed(wl, idx, scheme: str, threshold: int, threads: int):
    """The oracle on episodes ``idx``: (results, seconds, threads used).  The
    results are the counts, the relaxed counts, or both stacked (two-pass)."""
    import oracle
    t0 = time.perf_counter()
    if scheme in ("alpha", "stream"):
        want, _, used = oracle.count_timed(wl.times, wl.types, wl.ep_types[idx], wl.t_low[idx],
                                           wl.t_high[idx], n_threads=threads)
    elif scheme == "upper":
        want = oracle.count_upper(wl.times, wl.types, wl.ep_types[idx], wl.t_high[idx],
                                  n_threads=threads)
    else:
        want = np.stack(oracle.two_pass(wl.times, wl.types, wl.ep_types[idx], wl.t_low[idx],
                                        wl.t_high[idx], threshold, n_threads=threads))
    dt = time.perf_counter() - t0
    return want, dt, min(threads, len(idx))


def cpu_baseline(wl, gpu_result, target_s: float, scheme: str = "alpha", threshold: int = 0):
    """The oracle, as it stands, on a bounded sample of the workload's episodes:
    as many episodes (evenly spaced) as fit the time budget, and when all of
    them fit, the whole workload repeated until the budget is spent.
    ``gpu_result`` is indexed by episode along its last axis."""
    threads = min(os.cpu_count() or 1, 16)
    S = wl.n_episodes
    probe = min(S, max(threads, 8))
    _, dt, _ = oracle_timed(wl, np.arange(probe), scheme, threshold, threads)
    per_ep = dt / probe
    m = int(min(S, max(probe, target_s / max(per_ep, 1e-9))))
    idx = np.unique(np.linspace(0, S - 1, m).astype(np.int64))
    reps, total, used, ok = 0, 0.0, threads, True
    while True:
        want, dt, used = oracle_timed(wl, idx, scheme, threshold, threads)
        ok = ok and bool(np.array_equal(gpu_result[..., idx], want))
        reps += 1
        total += dt
        if total >= 0.9 * target_s or reps >= 1000:
            break
    value = wl.n_events * idx.size * reps / total
    return {"value": value, "unit": "episode-events/s", "cores": int(used), "kind": "oracle",
            "sample": "%d of %d episodes (evenly spaced) over all %d events, %d pass(es), %.2f s"
                      % (idx.size, S, wl.n_events, reps, total)}, ok, idx.size


def calibrate_copy(nbytes: int, reps: int):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "launches": reps}))


def mining_candidates(mined, bins):
    """The candidate lists ep_mine counted, rebuilt from its frequent sets with
    the same rule (for the work figure of the roofline): {k: [types tuple]}."""
    index = {b: i for i, b in enumerate(bins)}
    out = {}
    ks = sorted(mined)
    for k in ks:
        if k == 1:
            continue
        prev = mined.get(k - 1)
        if prev is None:
            break
        ep, lo, hi, _ = prev
        rows = [(tuple(int(x) for x in ep[i]),
                 tuple(index[(int(lo[i, j]), int(hi[i, j]))] for j in range(k - 2)))
                for i in range(ep.shape[0])]
        cands = []
        if k == 2:
            for (a,), _ in rows:
                for b in range(len(bins)):
                    for (c,), _ in rows:
                        cands.append((a, c))
        else:
            by_prefix = {}
            for t, bs in rows:
                by_prefix.setdefault((t[:-1], bs[:-1]), []).append(t)
            for t, bs in rows:
                for t2 in by_prefix.get((t[1:], bs[1:]), []):
                    cands.append(t + (t2[-1],))
        out[k] = cands
    return out


def main_mine(args):
    """Level-wise mining benchmark: one step = one ep_mine call."""
    import torch
    import frequent_episode_mining_amd as fem
    from frequent_episode_mining_amd import workloads as W

    t0 = time.time()
    wl = W.make_mining(args.config)
    threshold = wl.threshold if args.threshold is None else args.threshold
    log("workload %s: %s (%.1fs to generate)" % (wl.name, wl.description, time.time() - t0))
    dev = torch.device("cuda:0")
    times, types = fem.to_device(wl.times, wl.types, dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        return fem.mine(times, types, wl.alphabet, wl.bins, max_nodes=wl.max_nodes,
                        threshold=threshold, two_pass=args.two_pass_mining, mode=args.mode,
                        stream=stream, candidates=True)

    mined, cands = step()
    log("levels: frequent %s, candidates %s" % ({k: len(v[3]) for k, v in mined.items()}, cands))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    fem.profile_begin()
    for _ in range(args.steps):
        step()
    prof = fem.profile_end()
    per = {k: prof[k] / args.steps for k in PHASES}
    top = max(per, key=per.get)
    which = PHASES[top]
    log("phases per step: map %.4f (filter %.4f, prune %.4f, ticks %.4f, positions %.4f) closure %.4f "
        "concat %.4f other %.4f ms; %.1f counting calls per step"
        % (prof["map_ms"] / args.steps, per["map_filter_ms"], per["map_prune_ms"], per["map_ticks_ms"],
           per["map_positions_ms"], prof["closure_ms"] / args.steps, prof["concat_ms"] / args.steps,
           prof["other_ms"] / args.steps, prof["calls"] / args.steps))
    fem.profile_begin_kernel(which, 1)
    torch.cuda.synchronize(dev)
    w0 = time.perf_counter()
    for _ in range(args.steps):
        mined, cands = step()
    torch.cuda.synchronize(dev)
    w1 = time.perf_counter()
    kprof = fem.profile_end()
    ms_per_step = (w1 - w0) * 1000.0 / args.steps
    n = wl.n_events
    total_cands = sum(cands.values())
    value = n * total_cands / (ms_per_step / 1000.0)
    kernel_ms = kprof[top] / args.steps
    # work of the dominant kernel: 10 int32 ops per (candidate, relevant event)
    cnt = np.bincount(wl.types, minlength=65536).astype(np.int64)
    rel = int(cnt[np.unique(wl.alphabet)].sum())  # size 1: each type's own events
    for k, lst in mining_candidates(mined, wl.bins).items():
        rel += sum(int(cnt[np.unique(np.array(t))].sum()) for t in lst)
    # (the ticks phase: the tick kernel, and the type-sliced kernel for the
    # two-node candidates)
    names = {"map_filter_ms": "filter_kernel", "map_prune_ms": "list_prune_kernel",
             "map_ticks_ms": "map_ticks_kernel+map_slice_kernel", "map_positions_ms": "map_bits_kernel"}
    achieved = OPS_PER_RELEVANT_PAIR * rel / (kernel_ms / 1000.0) / 1e12 if kernel_ms > 0 else 0.0
    roofline = {"bound": "alu", "achieved": achieved, "peak": ALU_PEAK_TOPS, "unit": "TOP/s",
                "frac": achieved / ALU_PEAK_TOPS, "traffic": None,
                "work": "%d int32 ops x %d (candidate, relevant event) pairs over all sizes"
                        % (OPS_PER_RELEVANT_PAIR, rel),
                "kernel": names[top], "kernel_ms": kernel_ms,
                "launches_per_step": kprof["calls"] / args.steps, "timed_launches": kprof["calls"]}
    log("step %.4f ms; %s kernel %.4f ms per step" % (ms_per_step, which, kernel_ms))

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        threads = min(os.cpu_count() or 1, 16)
        reps, total, ok = 0, 0.0, True
        while True:
            t0 = time.perf_counter()
            want = oracle.mine(wl.times, wl.types, wl.alphabet, wl.bins, wl.max_nodes, threshold,
                               n_threads=threads)
            total += time.perf_counter() - t0
            reps += 1
            ok = ok and sorted(want) == sorted(mined) and all(
                all(np.array_equal(a, b) for a, b in zip(mined[k], want[k])) for k in want)
            if total >= 0.9 * args.cpu_seconds or reps >= 100:
                break
        cpu = {"value": n * total_cands * reps / total, "unit": "episode-events/s",
               "cores": threads, "kind": "oracle",
               "sample": "the whole mining job (%d sizes, %d candidates), %d pass(es), %.2f s"
                         % (len(cands), total_cands, reps, total)}
        parity = "identical frequent sets and counts" if ok else "MISMATCH"
        log("cpu oracle: %s; parity %s" % (cpu["sample"], parity))

    line = {
        "metric": "episode-events/sec (events x candidate episodes counted)",
        "value": value,
        "unit": "episode-events/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "n_events": n,
                   "scheme": "level-wise mining%s, threshold %d, up to %d nodes"
                             % (" (two-pass counting)" if args.two_pass_mining else "", threshold,
                                wl.max_nodes),
                   "frequent": {str(k): int(len(v[3])) for k, v in mined.items()},
                   "candidates": {str(k): int(v) for k, v in cands.items()},
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line))
    if parity == "MISMATCH":
        sys.exit(1)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="longchain",
                    choices=["tiny", "ptpe", "mapconcat", "level2", "longchain", "sym26"],
                    help="a counting workload, or sym26: level-wise mining of a Sym26-shaped stream")
    ap.add_argument("--mode", default="auto", choices=["auto", "ptpe", "mapconcat"])
    ap.add_argument("--segments", type=int, default=-1,
                    help="MapConcatenate segment count (-1: the workload's own, 0: planner)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--scheme", default="alpha", choices=["alpha", "upper", "two-pass", "stream"],
                    help="alpha: exact counts; upper: relaxed episodes (lower bounds 0); "
                         "two-pass: relaxed counts, then exact counts of those >= --threshold; "
                         "stream: the stream pushed in --batches batches to an EpisodeStream")
    ap.add_argument("--batches", type=int, default=10, help="batches of --scheme stream")
    ap.add_argument("--threshold", type=int, default=None,
                    help="support threshold of --scheme two-pass (default 30000) or of mining "
                         "(default: the workload's)")
    ap.add_argument("--two-pass-mining", action="store_true",
                    help="sym26: count every size from 2 on with the two-pass elimination")
    ap.add_argument("--plan", default="",
                    help="comma-separated planner switches (EP_PLAN_* names, e.g. prune,no-reduce); "
                         "they choose kernels, never results")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, 5)
        return

    import frequent_episode_mining_amd as fem
    from frequent_episode_mining_amd import workloads as W

    fem.load_library()
    if args.config in W.MINING:
        return main_mine(args)
    if args.threshold is None:
        args.threshold = 30000
    t0 = time.time()
    wl = W.make(args.config)
    log("workload %s: %s (%.1fs to generate)" % (wl.name, wl.description, time.time() - t0))
    seg = wl.n_segments if args.segments < 0 else args.segments
    mode = args.mode
    if mode == "auto" and args.segments >= 0 and args.segments != 0:
        mode = "mapconcat"
    if mode == "auto" and args.segments < 0 and wl.n_segments:
        mode = "mapconcat"  # the workload names its segment count
    if mode == "auto":
        seg = 0

    dev = torch.device("cuda:0")
    times, types = fem.to_device(wl.times, wl.types, dev)
    table = fem.EpisodeTable(wl.ep_types, wl.t_low, wl.t_high)
    out = torch.empty(wl.n_episodes, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)

    scheme = args.scheme
    kept_box = [0]
    plan = [p for p in args.plan.split(",") if p]

    cuts = np.linspace(0, wl.n_events, max(1, args.batches) + 1).astype(np.int64)

    def step():
        if scheme == "stream":
            st = fem.EpisodeStream(table, mode=mode, n_segments=seg, stream=stream, plan=plan)
            for i in range(cuts.size - 1):
                st.push(times[cuts[i]:cuts[i + 1]], types[cuts[i]:cuts[i + 1]], stream=stream)
            c = st.counts(stream=stream)
            st.close()
            return c, None
        if scheme == "two-pass":
            c, u, kept_box[0] = fem.count_two_pass(times, types, table, threshold=args.threshold,
                                                   mode=mode, n_segments=seg, stream=stream, plan=plan)
            return c, u
        fem.count_episodes(times, types, table, mode=mode, n_segments=seg, out=out, stream=stream,
                           upper_only=(scheme == "upper"), plan=plan)
        return out, None

    if scheme == "stream":
        # the stream reports no plan: the first batch counted alone has the
        # same kernels (the list rule looks at the episodes and the batch size)
        _, st = fem.count_episodes(times[cuts[0]:cuts[1]], types[cuts[0]:cuts[1]], table, mode="mapconcat",
                                   n_segments=seg, stats=True, stream=stream, plan=plan)
        st = dict(st, mode="mapconcat per batch", n_segments=0, repairs=0, fallbacks=0)
    elif scheme == "two-pass":
        _, _, _, st = fem.count_two_pass(times, types, table, threshold=args.threshold, mode=mode,
                                         n_segments=seg, stats=True, stream=stream, plan=plan)
    else:
        _, st = fem.count_episodes(times, types, table, mode=mode, n_segments=seg, stats=True,
                                   out=out, upper_only=(scheme == "upper"), plan=plan)
    log("plan: %s" % st)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)

    # An untimed pass with every phase timed (events around each phase cost
    # the stream a few microseconds each): the breakdown for the log, and which
    # Map-step kernel dominates.
    fem.profile_begin()
    for _ in range(args.steps):
        step()
    prof = fem.profile_end()
    per = {k: prof[k] / args.steps for k in PHASES}
    if not st["kernels"] & 4:
        per["map_filter_ms"] = 0.0  # no filter launched: the interval is two bare events
    if not st["kernels"] & 8:
        per["map_prune_ms"] = 0.0  # no pruning launched: likewise
    top = max(per, key=per.get)
    which = PHASES[top]
    log("phases per step: map %.4f (filter %.4f, prune %.4f, ticks %.4f, positions %.4f) closure %.4f "
        "concat %.4f other %.4f ms"
        % (prof["map_ms"] / args.steps, per["map_filter_ms"], per["map_prune_ms"], per["map_ticks_ms"],
           per["map_positions_ms"], prof["closure_ms"] / args.steps,
           prof["concat_ms"] / args.steps, prof["other_ms"] / args.steps))

    # The timed region: only the dominant kernel's two events, on one call in
    # four (every call for the two-pass scheme: its steps alternate passes).
    every = 1 if scheme in ("two-pass", "stream") else 4
    fem.profile_begin_kernel(which, every)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        res, res_upper = step()
    ev1.record(stream)
    we = time.perf_counter()
    torch.cuda.synchronize(dev)
    w1 = time.perf_counter()
    kprof = fem.profile_end()
    gpu_ms = ev0.elapsed_time(ev1) / args.steps
    wall_ms = (w1 - w0) * 1000.0 / args.steps
    ms_per_step = max(gpu_ms, wall_ms)
    counts = res.cpu().numpy()
    if scheme == "two-pass":
        upper = res_upper.cpu().numpy()
        counts = np.stack([counts, upper])
        log("two-pass: threshold %d, %d of %d episodes counted exactly, %d frequent"
            % (args.threshold, kept_box[0], wl.n_episodes, int((counts[0] >= args.threshold).sum())))
    log("host enqueue %.4f ms per call" % ((we - w0) * 1000.0 / args.steps))
    # the dominant Map-step kernel of this workload, timed alone by the
    # library's events on the stream it runs on, during the timed calls
    if st["kernels"] & 1:
        pos_name = "map_list_kernel" if st["kernels"] & 4 else "map_bits_kernel"
    else:
        pos_name = "map_scan_kernel"
    # (two-node episodes on the type-sliced kernel: it takes the tick kernel's slot)
    names = {"map_filter_ms": "filter_kernel", "map_prune_ms": "list_prune_kernel",
             "map_ticks_ms": "map_slice_kernel" if st["kernels"] & 32 else "map_ticks_kernel",
             "map_positions_ms": pos_name}
    log("step %.4f ms (gpu events %.4f, wall %.4f); %s %.4f ms per launch (%d launches timed)"
        % (ms_per_step, gpu_ms, wall_ms, names[top], kprof[top] / max(kprof["calls"], 1), kprof["calls"]))

    n, S = wl.n_events, wl.n_episodes
    value = n * S / (ms_per_step / 1000.0)

    kernel, kernel_ms = names[top], kprof[top] / max(kprof["calls"], 1)
    map_s = kernel_ms / 1000.0
    rel = relevant_pairs(wl)
    if scheme == "two-pass":
        # both passes' launches per step: all episodes, then the kept ones
        kept_rows = np.flatnonzero(counts[1] >= args.threshold)
        rel = rel + relevant_pairs_rows(wl, kept_rows)
        kernel_ms = kprof[top] / args.steps
        map_s = kernel_ms / 1000.0
    elif scheme == "stream":
        # every batch's launch: the whole stream once (the halo re-counts are extra work)
        kernel_ms = kprof[top] / args.steps
        map_s = kernel_ms / 1000.0
    traffic = stored_traffic(wl.name if scheme == "alpha" else "%s-%s" % (wl.name, scheme), kernel)
    if traffic is not None and scheme == "two-pass":
        traffic *= 2  # the stored figure is per dispatch; a step launches the kernel twice
    if kernel == "list_prune_kernel":
        # every entry read once (the kept ones are written back in place)
        moved = 8.0 * rel
        achieved = moved / map_s / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                    "work": "8 B x %d entries read" % rel}
    elif kernel == "filter_kernel":
        # the algorithmic work is one read of the stream (6 B per event); the
        # {time, levels} entries the filter writes for the list kernel are this
        # design's own intermediate: reported beside it, not counted as work
        moved = 6.0 * n
        achieved = moved / map_s / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                    "work": "6 B x %d events read (one pass over the stream)" % n,
                    "intermediate_bytes_written": 8.0 * rel}
    else:
        achieved = OPS_PER_RELEVANT_PAIR * rel / map_s / 1e12
        roofline = {"bound": "alu", "achieved": achieved, "peak": ALU_PEAK_TOPS, "unit": "TOP/s",
                    "frac": achieved / ALU_PEAK_TOPS, "traffic": traffic,
                    "work": "%d int32 ops x %d (episode, relevant event) pairs"
                            % (OPS_PER_RELEVANT_PAIR, rel)}
    roofline.update({"kernel": kernel, "kernel_ms": kernel_ms,
                     "launches_per_step": kprof["calls"] / args.steps,
                     "timed_launches": kprof["calls"],
                     "map_kernels_ms": {names[k]: v for k, v in per.items()},
                     # the whole call (every kernel, its gaps and the table upload)
                     # against one pass over the stream at HBM peak, and against the
                     # stream read once per episode (what one reader per episode
                     # would move)
                     "hbm_one_pass_frac": 6.0 * n / (ms_per_step / 1000.0) / 1e9 / HBM_PEAK_GBS,
                     "hbm_per_episode_frac": 6.0 * n * S / (ms_per_step / 1000.0) / 1e9 / HBM_PEAK_GBS,
                     "map_step_one_pass_frac": 6.0 * n / (prof["map_ms"] / args.steps / 1000.0)
                                               / 1e9 / HBM_PEAK_GBS})

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        cpu, ok, m = cpu_baseline(wl, counts, args.cpu_seconds, scheme, args.threshold)
        parity = "bit-exact on %d sampled episodes" % m if ok else "MISMATCH"
        log("cpu oracle: %s; parity %s" % (cpu["sample"], parity))
        if not ok:
            print("bench: GPU counts differ from the oracle", file=sys.stderr)

    line = {
        "metric": "episode-events/sec (events x episodes counted)",
        "value": value,
        "unit": "episode-events/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "n_events": n,
                   "n_episodes": S, "n_nodes": wl.n_nodes, "mode": st["mode"],
                   "segments": st["n_segments"], "window_runs": st["max_runs"],
                   "repairs": st["repairs"], "fallbacks": st["fallbacks"],
                   "plan": plan,
                   "scheme": {"alpha": "exact counts",
                              "upper": "relaxed episodes (lower bounds 0)",
                              "two-pass": "two-pass elimination, threshold %d, %d kept"
                                          % (args.threshold, kept_box[0]),
                              "stream": "streaming counts, %d batches" % args.batches}[scheme],
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line))
    if parity == "MISMATCH":
        sys.exit(1)


if __name__ == "__main__":
    main()
