"""Benchmark of the mixer hot path on one MI355X.

One step = one free-running generation of all L positions of the workload
(every red cell, every direct and FFT gray block, graphs as in production),
starting from cleared activations with the seeded first input.  Inputs are
resident in HBM before timing starts.

Prints ONE JSON line with:
  value        mixer tokens/s (positions/s x B) over the K timed steps
  latency_us   per-position latency from device wall-clock stamps (p50/p99/max,
               median per block-size class)
  roofline     FFT gray-block kernels: algorithmic bytes / event-measured kernel
               time over the timed steps, against 8 TB/s HBM
  lazy_gpu     the GPU Lazy baseline (O(n) per position), timed at sampled
               positions and integrated over all L (cost is affine in n)
  cpu_baseline the CPU oracle on a bounded sample, scaled to the full workload

Usage: python bench.py [--gpus 1] [--steps 4] [--warmup 2] [--workload 4]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "mixer tokens/sec + p50/p99 per-token latency; HBM GB/s % of peak (L=2^17)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fft_alg_bytes(w, U):
    """Algorithmic bytes of one FFT gray-block launch of edge U over all layers:
    per (l, c): B*(4U input + 8U accumulator read-modify-write) + 8U spectrum."""
    return w.M * w.D * (w.B * 12 * U + 8 * U)


def kernel_source_hash():
    """Hash of the FFT gray-block kernel sources (the kernels the traffic summary covers,
    with the device helpers they include)."""
    h = hashlib.sha256()
    for f in ("fi_fft_kernels.h", "fi_fft.h", "fi_device.h"):
        with open(os.path.join(ROOT, "long_convolution_sequence_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(w, launches_by_class):
    """Per-launch HBM traffic (read + write bytes) of the FFT gray blocks, from the
    committed PMC summary of each class, weighted like the timed launches; only
    if the summary was taken on the current kernel sources."""
    path = TRAFFIC_PATH
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("kernel_source_hash") != kernel_source_hash() or d.get("workload") != w.name:
        return None
    per = {r["q"]: r["read_bytes"] + r["write_bytes"] for r in d.get("per_class", [])}
    n = sum(launches_by_class.values())
    if n == 0 or any(q not in per for q in launches_by_class):
        return None
    return round(sum(per[q] * k for q, k in launches_by_class.items()) / n)


def cpu_baseline(w, h, target_s=12.0):
    """The CPU oracle (naive fp64 definition) on a bounded sample: a subset of
    (b, c) chains over a prefix of positions, scaled to the whole workload
    (chains are independent; per-position cost grows linearly with n)."""
    import oracle
    from long_convolution_sequence_amd import workloads

    threads = oracle.num_threads()
    nch = max(threads, 8)
    x1 = workloads.x_first(w).reshape(-1)
    rng = np.random.default_rng(0)
    chains = np.sort(rng.choice(w.B * w.D, nch, replace=False))
    cs = (chains % w.D).astype(np.int32)
    def run(steps):
        t0 = time.time()
        oracle.stack(h, cs, x1[chains], steps)
        return time.time() - t0

    steps = 1024                                  # grow the prefix until a run takes >= 1 s,
    dt = run(steps)                               # then size one run to about target_s
    while dt < 1.0 and steps < w.L:
        steps = min(w.L, steps * 2)
        dt = run(steps)
    if dt < target_s and steps < w.L:
        steps = int(min(w.L, steps * np.sqrt(target_s / dt)))
        dt = run(steps)
    # sum_{n<=L} n / sum_{n<=steps} n  and  chains total / sampled
    full = dt * (w.L * (w.L + 1)) / (steps * (steps + 1)) * (w.B * w.D) / nch
    return {
        "value": w.L * w.B / full,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{nch} of {w.B * w.D} (b,c) chains x first {steps} positions x {w.M} layers, "
                  f"{dt:.1f}s measured, scaled by chain count and by the quadratic position "
                  f"cost to all L={w.L} positions (extrapolated)",
    }


TRAFFIC_PATH = os.path.join(ROOT, "profiles", "fft_tile_traffic_L131072.json")
COPY_MIB = 1024


def traffic_run(args):
    """The workload's FFT gray-block classes, each launched once more after a
    warm-up, then a plain device-to-device copy of COPY_MIB MiB (twice): run
    under rocprofv3 --pmc FETCH_SIZE and again under --pmc WRITE_SIZE, the copy
    gives each counter's scale (bytes it reads for known bytes moved)."""
    import torch

    from long_convolution_sequence_amd import fi, workloads

    w = workloads.WORKLOADS[args.workload]
    h = workloads.filters(w)
    ctx = fi.Context(torch.from_numpy(h).cuda(), w.B)
    fft = [q for (q, p, _, _) in ctx.tau_table() if p == fi.PATH_FFT]
    for q in fft:
        log(f"traffic run: class {q} (U={1 << q})")
        ctx.time_block(q, fi.PATH_FFT, reps=1)
    ctx.close()
    src = torch.ones(COPY_MIB << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"traffic run: copied {COPY_MIB} MiB twice; FFT classes {fft}")


def traffic_summary(args):
    """Per-launch HBM traffic of the FFT gray blocks from the two PMC runs of
    --traffic-run (counter_collection CSVs), written to TRAFFIC_PATH."""
    import csv
    import re

    from long_convolution_sequence_amd import workloads

    w = workloads.WORKLOADS[args.workload]
    copy_kib = COPY_MIB * 1024

    def load(path, counter):
        per = {}     # class -> list of KiB per launch (split classes: fwd + inv of one launch)
        copies = []
        rows = list(csv.DictReader(open(path)))
        by_kernel = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            name, v, grid = r["Kernel_Name"], float(r["Counter_Value"]), int(r["Grid_Size"])
            if "copyBuffer" in name:
                copies.append((int(r["Dispatch_Id"]), v))
                continue
            m = re.search(r"k_fft_(tile2|tile|sub_fwd|sub_inv)<(\d+)(?:, *\d+)?>", name)
            if not m:
                continue
            kind, lg = m.group(1), int(m.group(2))
            if kind == "tile":
                q = lg
            elif kind == "tile2":
                q = lg + 1
            else:
                tpb = max(256, (1 << lg) // 16)
                k = grid // (w.M * w.B * w.D * tpb)
                q = lg + k.bit_length() - 1
            by_kernel.setdefault((q, kind), []).append(v)
        for (q, kind), vs in by_kernel.items():
            per.setdefault(q, 0.0)
            per[q] += sum(vs) / len(vs)
        # the calibration copies are the last two copy dispatches
        last = [v for _, v in sorted(copies)[-2:]]
        return per, sum(last) / len(last)

    fetch, fetch_copy = load(args.traffic_summary[0], "FETCH_SIZE")
    write, write_copy = load(args.traffic_summary[1], "WRITE_SIZE")
    f_scale = copy_kib / fetch_copy
    w_scale = copy_kib / write_copy
    classes = sorted(set(fetch) & set(write))
    rows = []
    for q in classes:
        U = 1 << q
        rd = fetch[q] * f_scale * 1024
        wr = write[q] * w_scale * 1024
        alg = fft_alg_bytes(w, U)
        rows.append({"q": q, "U": U, "read_bytes": round(rd), "write_bytes": round(wr),
                     "alg_bytes": alg, "ratio": round((rd + wr) / alg, 3)})
    out = {
        "workload": w.name,
        "kernel_source_hash": kernel_source_hash(),
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "calibration": f"device-to-device copy of {COPY_MIB} MiB: FETCH_SIZE read {fetch_copy:.0f} KiB, "
                       f"WRITE_SIZE {write_copy:.0f} KiB per dispatch",
        "per_class": rows,
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o pmc -- python3 bench.py --traffic-run",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o pmc -- python3 bench.py --traffic-run",
            "python3 bench.py --traffic-summary <fetch csv> <write csv>",
        ],
    }
    with open(TRAFFIC_PATH, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def hyena_run(w, positions, warm=512):
    """One free-running generation of the Hyena-style block workload (projection,
    gate, mixer, GELU MLP, RMSNorm, tanh feedback), end to end, and the split of
    its time between the mixer and the block: the block kernels of one position
    are timed alone with HIP events (fi_time_hyena_block), the mixer's share is
    the rest of the generation."""
    import torch

    from long_convolution_sequence_amd import fi, workloads

    h = workloads.filters(w)
    bits = workloads.hyena_weights(w)
    x1 = torch.from_numpy(workloads.x_first(w)).cuda()
    hc = fi.Context(torch.from_numpy(h).cuda(), w.B, map=fi.MAP_HYENA)
    del h
    hc.set_block_weights(bits["W"], bits["W1"], bits["W2"])
    hc.set_input(x1)
    hc.generate(min(positions, warm), want_y=False)            # warm-up (graphs, caches)
    hc.reset()
    hc.set_input(x1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hc.generate(positions, want_y=False)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st = hc.stamps(1, positions).astype(np.float64)
    lat = np.diff(st) / 100.0
    block_us = hc.time_hyena_block(reps=20)
    paths = [p for (_, p, _, _) in hc.tau_table()]
    hc.close()
    del hc
    torch.cuda.empty_cache()
    block_s = positions * block_us * 1e-6
    return {
        "workload": w.name, "positions": positions,
        "e2e_s": round(dt, 4), "e2e_tokens_per_s": round(positions * w.B / dt, 1),
        "block_us_per_position": round(block_us, 2),
        "block_share": round(min(1.0, block_s / dt), 4),
        "mixer_s": round(max(0.0, dt - block_s), 4),
        "mixer_tokens_per_s": round(positions * w.B / max(dt - block_s, 1e-9), 1),
        "latency_us": {"p50": round(float(np.percentile(lat, 50)), 2),
                       "p99": round(float(np.percentile(lat, 99)), 2),
                       "max": round(float(lat.max()), 1)},
        "block_paths": ["fft" if p == fi.PATH_FFT else "direct" for p in paths],
        "note": "free-running generation from position 0 (graphs per block-size class); block time = "
                "positions x the event-timed block kernels of one position (projections with the red "
                "cells, GELU MLP, RMSNorm, output), mixer time = the rest (gray blocks and launches)",
    }


def pareto(w, h, split, reps=8):
    """Per block size, the device time of one launch of each gray-block path at the
    real shape (the pages' runtime-per-tile-size comparison): the direct kernel
    (one launch per position, red cells included) where it exists (U <= 128),
    the FFT kernels where they exist (U >= 4)."""
    import torch

    from long_convolution_sequence_amd import fi

    pc = fi.Context(torch.from_numpy(h).cuda(), w.B, tau_split=split, use_graphs=False)
    rows = []
    for q in range(w.P):
        row = {"U": 1 << q}
        if q <= 7:
            row["direct_us"] = round(pc.time_block(q, fi.PATH_DIRECT, reps=reps), 2)
        if q >= 2:
            row["fft_us"] = round(pc.time_block(q, fi.PATH_FFT, reps=2 if q >= 14 else reps), 2)
        rows.append(row)
    pc.close()
    del pc
    torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-lazy", action="store_true")
    ap.add_argument("--no-defer-leg", action="store_true", help="skip the generation with deferred split blocks")
    ap.add_argument("--no-prefill-leg", action="store_true", help="skip the prefill timing")
    ap.add_argument("--no-dd-leg", action="store_true", help="skip the data-dependent-filter timing")
    ap.add_argument("--no-pareto-leg", action="store_true", help="skip the per-size path timing")
    ap.add_argument("--no-hyena-leg", action="store_true", help="skip the Hyena-style block workload leg")
    ap.add_argument("--no-chunk-leg", action="store_true",
                    help="skip the generation with chunks twice as long (throughput against p99 latency)")
    ap.add_argument("--hyena-positions", type=int, default=4096,
                    help="positions of the Hyena-style block leg (the whole L with --workload 5)")
    ap.add_argument("--positions", type=int, default=0, help="profile aid: generate only a prefix")
    ap.add_argument("--tau-split", type=int, default=-1,
                    help="first FFT block class (log2 U) instead of the calibrated choice; chunks are that long")
    ap.add_argument("--traffic-run", action="store_true",
                    help="launch each FFT class once and a calibration copy (run under rocprofv3 --pmc)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the FFT traffic summary from the two PMC runs")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the mixer shards over channels with no communication, see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    if args.traffic_run:
        traffic_run(args)
        return

    import torch

    from long_convolution_sequence_amd import fi, workloads

    w = workloads.WORKLOADS[args.workload]
    L = args.positions or w.L
    if w.block == "hyena":
        # the Hyena-style block workload end to end (its own line)
        hy = hyena_run(w, L)
        log(f"bench: {w.name}: {hy['e2e_tokens_per_s']:,.0f} tokens/s end to end, block share {hy['block_share']}")
        out = {"metric": "end-to-end tokens/sec + mixer/block time split (Hyena-style block, L=2^15)",
               "value": hy["e2e_tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": 1, "warmup": 1,
               "ms_per_step": round(hy["e2e_s"] * 1e3, 3), "higher_is_better": True, "scaling": "weak",
               "vs_baseline": None, "dtype": "f32 (bf16 weights)",
               "data": "synthetic (seeded random filters, block weights and first input, recipe in DESIGN.md)",
               "config": {"workload": w.name, "M": w.M, "B": w.B, "D": w.D, "L": L}, "hyena": hy}
        print(json.dumps(out), flush=True)
        return
    log(f"bench: {w.name}, generating inputs")
    h = workloads.filters(w)
    hdev = torch.from_numpy(h).cuda()
    x1 = torch.from_numpy(workloads.x_first(w)).cuda()
    # the production path: graphs of whole chunks and of their FFT gray blocks,
    # no per-kernel events
    # made with defer_wide = 2 so that the deferral leg below can defer the
    # two-half class too (its offset spectra live in the workspace); the timed
    # steps run with deferral off
    ctx = fi.Context(hdev, w.B, tau_split=args.tau_split, defer_wide=0 if args.no_defer_leg else 2)
    ctx.set_defer_wide(0)
    tau = ctx.tau_table()
    split = next((q for (q, pth, _, _) in tau if pth == fi.PATH_FFT), w.P)
    calib = [{"first_fft_U": 1 << g, "chunk_and_fft_us": round(uc, 2), "modeled_run_ms": round(ur * 1e-3, 3)}
             for (g, uc, ur) in ctx.chunk_table() if ur >= 0]
    log("bench: block paths", [(q, "fft" if p == fi.PATH_FFT else "direct") for (q, p, _, _) in tau])

    def one_step(c):
        c.reset()
        c.set_input(x1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        c.generate(L, want_y=False)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    for i in range(args.warmup):
        dt = one_step(ctx)
        log(f"bench: warmup {i + 1}/{args.warmup}: {dt:.3f}s")
    times, lat = [], []
    for i in range(args.steps):
        dt = one_step(ctx)
        times.append(dt)
        st = ctx.stamps(1, L).astype(np.float64)
        lat.append(np.diff(st) / 100.0)              # 100 MHz ticks -> us; positions 2..L
        log(f"bench: step {i + 1}/{args.steps}: {dt:.3f}s ({L * w.B / dt:,.0f} tokens/s)")
    total = float(np.sum(times))
    value = L * w.B * args.steps / total
    lat = np.concatenate(lat)
    npos = np.tile(np.arange(2, L + 1), args.steps)
    cls = np.array([(int(n) & -int(n)).bit_length() - 1 if n < w.L else w.P for n in range(2, L + 1)])
    cls = np.tile(cls, args.steps)
    per_class = {int(q): round(float(np.median(lat[cls == q])), 2) for q in np.unique(cls)}

    # Kernel durations for the roofline: the same generation, with every chunk
    # and FFT gray-block launch bracketed by HIP events that the dispatch
    # itself stamps (direct launches: events cannot be stamped inside graphs).
    # The kernels are the same; only the launches between them differ.
    ev_steps = max(2, min(args.steps, 4))
    ectx = fi.Context(hdev, w.B, time_blocks=True, tau_split=split)
    one_step(ectx)
    ectx.block_times(clear=True)
    ectx.chunk_times(clear=True)
    ev_times = []
    chunk_ms, chunk_n = 0.0, 0
    blk_ms = np.zeros(w.P)
    blk_n = np.zeros(w.P, dtype=np.int64)
    for i in range(ev_steps):
        ev_times.append(one_step(ectx))
        for q, ms, cnt in ectx.block_times(clear=True):
            blk_ms[q] += ms
            blk_n[q] += cnt
        cms, cn = ectx.chunk_times(clear=True)
        chunk_ms += cms
        chunk_n += cn
    ev_total = float(np.sum(ev_times))
    log(f"bench: {ev_steps} event-timed generations: {L * w.B * ev_steps / ev_total:,.0f} tokens/s")
    ectx.close()
    del ectx, hdev
    torch.cuda.empty_cache()

    # FFT gray-block roofline over the event-timed generations
    rows = []
    tot_bytes = tot_ms = 0.0
    for q in range(w.P):
        if blk_n[q] == 0:
            continue
        U = 1 << q
        by = fft_alg_bytes(w, U)
        avg_ms = blk_ms[q] / blk_n[q]
        rows.append({"U": U, "launches": int(blk_n[q]), "avg_us": round(avg_ms * 1e3, 2),
                     "alg_bytes": by, "GBps": round(by / (avg_ms * 1e-3) / 1e9, 1)})
        tot_bytes += by * blk_n[q]
        tot_ms += blk_ms[q]
    launches = int(blk_n.sum())
    achieved = tot_bytes / (tot_ms * 1e-3) / 1e9 if tot_ms > 0 else 0.0
    G = 1 << split if split < w.P else L                                  # chunks end at FFT positions
    chunk = None
    if chunk_n:
        avg_us = chunk_ms * 1e3 / chunk_n
        # per-position latency inside chunks (timed steps), by the position's place
        # in its chunk (r = 2 .. G-1; r = 1 follows the FFT block before the chunk,
        # r = G ends with the FFT block after it)
        r = (npos - 1) % G + 1
        win = max(1, G // 8)
        by_place, mean_place = {}, {}
        for a in range(0, G, win):
            sel = (r > max(a, 1)) & (r <= min(a + win, G - 1))
            if sel.any():
                by_place[f"{max(a, 1) + 1}-{min(a + win, G - 1)}"] = round(float(np.median(lat[sel])), 3)
                mean_place[f"{max(a, 1) + 1}-{min(a + win, G - 1)}"] = round(float(np.mean(lat[sel])), 3)
        first = r == 1
        in_chunk = (r >= 2) & (r <= G - 1)
        # algorithmic bytes of a chunk launch: every direct gray block of edge U < G
        # inside the chunk (per (l, c): B*12U + 4(2U-1)) and the red cells (12 bytes
        # per (l, b, c) and position)
        lg = G.bit_length() - 1
        per_lc = sum((G >> (q + 1)) * (w.B * 12 * (1 << q) + 4 * (2 * (1 << q) - 1)) for q in range(lg))
        chunk_bytes = w.M * w.D * per_lc + 12 * w.M * w.B * w.D * G
        chunk = {"kernel": "k_chunk (red cells and direct gray blocks of a chunk of positions)",
                 "alg_bytes_per_launch": chunk_bytes,
                 "hbm_frac_by_alg_bytes": round(chunk_bytes / (avg_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                 "launches": int(chunk_n), "positions_per_launch": G,
                 "avg_launch_us": round(avg_us, 2), "us_per_position": round(avg_us / G, 4),
                 "median_us_by_place_in_chunk": by_place,
                 "mean_us_by_place_in_chunk": mean_place,
                 "first_position_median_us": round(float(np.median(lat[first])), 2) if first.any() else None,
                 "sum_of_mean_position_us_2_to_G-1": round(float(np.mean(lat[in_chunk])) * (G - 2), 1),
                 "share_of_event_timed_step": round(chunk_ms * 1e-3 / ev_total, 4),
                 "fft_share_of_event_timed_step": round(tot_ms * 1e-3 / ev_total, 4),
                 "bound": "latency: the serial red-cell chain (M layers of fma + tanh per position) "
                          "and one workgroup barrier per position, not bytes or flops"}

    # one more generation with the later sub-blocks of split gray blocks
    # deferred to the context's second stream (large-block latency smoothing)
    defer = None
    if not args.no_defer_leg:
        top = w.P - 1
        dcls = cls[:L - 1]

        def deferred_generation(level):
            ctx.set_defer_wide(level)
            dt = one_step(ctx)
            dl = np.diff(ctx.stamps(1, L).astype(np.float64)) / 100.0
            ctx.set_defer_wide(0)
            lat_us = {"p50": round(float(np.percentile(dl, 50)), 2),
                      "p99": round(float(np.percentile(dl, 99)), 2),
                      "max": round(float(dl.max()), 1)}
            for q in (top - 1, top):
                lat_us[f"class_{q}_median"] = round(float(np.median(dl[dcls == q])), 1)
            return {"tokens_per_s": round(L * w.B / dt, 1), "latency_us": lat_us}

        defer = deferred_generation(1)
        defer["note"] = ("one generation with fi_options.defer_wide = 1: a split gray block computes its "
                         "first output sub-block before the next position and the rest on a second "
                         "stream; not part of the timed steps above")
        defer["undeferred_class_medians_us"] = {f"class_{q}": per_class.get(q) for q in (top - 1, top)}
        two = deferred_generation(2)
        two["note"] = ("one generation with fi_options.defer_wide = 2: the two-half class as well, run as 4 "
                       "sub-blocks of half the one-workgroup width with sub-blocks 1..3 on the second stream")
        defer["level_2"] = two
        log(f"bench: deferral: class {top - 1}/{top} medians {defer['latency_us'][f'class_{top - 1}_median']}/"
            f"{defer['latency_us'][f'class_{top}_median']} us (level 1), "
            f"{two['latency_us'][f'class_{top - 1}_median']}/{two['latency_us'][f'class_{top}_median']} us (level 2)")
    # one generation with chunks twice as long (one more direct class): the
    # calibration picks the chunk length for throughput, but the first position
    # of a chunk and the one whose FFT block ends it take the boundary's cost,
    # two of every G positions, which sets the p99 once 2/G passes 1%
    longer = None
    G2 = 1 << (split + 1)
    if not args.no_chunk_leg and args.tau_split < 0 and split + 1 < w.P and G2 <= 256:
        hd2 = torch.from_numpy(h).cuda()
        lctx = fi.Context(hd2, w.B, tau_split=split + 1)
        del hd2
        one_step(lctx)
        dt = one_step(lctx)
        ll = np.diff(lctx.stamps(1, L).astype(np.float64)) / 100.0
        lctx.close()
        del lctx
        torch.cuda.empty_cache()
        longer = {"chunk_positions": G2, "tokens_per_s": round(L * w.B / dt, 1),
                  "latency_us": {"p50": round(float(np.percentile(ll, 50)), 2),
                                 "p99": round(float(np.percentile(ll, 99)), 2),
                                 "max": round(float(ll.max()), 1)},
                  "note": f"one generation (after one warm-up) with the first FFT class pinned to 2^{split + 1}: "
                          f"chunks of {G2} positions instead of the calibrated {1 << split}; not part of the "
                          f"timed steps above"}
        log(f"bench: chunks of {G2}: {longer['tokens_per_s']:,.0f} tokens/s, p99 {longer['latency_us']['p99']} us")
    traffic = measured_traffic(w, {q: int(blk_n[q]) for q in range(w.P) if blk_n[q] > 0})
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "kernel": "FFT gray blocks (k_fft_tile / k_fft_sub_fwd+inv), all classes",
        "alg_bytes_per_launch": round(tot_bytes / max(launches, 1)),
        "avg_launch_us": round(tot_ms * 1e3 / max(launches, 1), 2),
        "per_class": rows,
        "measured": f"kernel durations from {ev_steps} generations run right after the timed steps, every FFT "
                    f"gray-block launch bracketed by HIP events stamped by the dispatch on the context's stream "
                    f"(direct launches; the timed steps replay the same kernels from graphs)",
        "event_timed_tokens_per_s": round(L * w.B * ev_steps / ev_total, 1),
    }
    ctx.close()
    del ctx
    torch.cuda.empty_cache()

    par = None
    if not args.no_pareto_leg:
        par = pareto(w, h, split)
        log("bench: per-size path times " + ", ".join(
            f"U={r['U']}: " + "/".join(f"{r[k]}" for k in ("direct_us", "fft_us") if k in r) for r in par))

    hyena = None
    if not args.no_hyena_leg:
        hyena = hyena_run(workloads.WORKLOADS[5], args.hyena_positions)
        log(f"bench: Hyena-style block workload, {args.hyena_positions} positions: "
            f"{hyena['e2e_tokens_per_s']:,.0f} tokens/s end to end, block share {hyena['block_share']}")

    lazy = ablations = None
    if not args.no_lazy:
        # the baselines use no gray blocks: skip calibration and graphs
        bl = fi.Context(torch.from_numpy(h).cuda(), w.B, use_graphs=False, tau_split=0)
        pts = sorted({max(1, int(w.L * k / 8)) for k in range(1, 9)} | {1, 64})
        fits = {}
        for name, kind in (("lazy", fi.BASE_LAZY), ("lazy_np", fi.BASE_LAZY_NP), ("eager", fi.BASE_EAGER),
                           ("eager_np", fi.BASE_EAGER_NP)):
            tus = [bl.baseline_time(kind, n, reps=3 if (n > 1024) == name.startswith("lazy") else 10)
                   for n in pts]
            # per-position cost is affine in the work: n for Lazy, L - n for Eager
            work = np.array([n if name.startswith("lazy") else w.L - n for n in pts], dtype=np.float64)
            A = np.vstack([np.ones(len(pts)), work]).T
            a, b = np.linalg.lstsq(A, np.array(tus), rcond=None)[0]
            total_s = (a * w.L + b * w.L * (w.L + 1) / 2 - (0 if name.startswith("lazy") else b * w.L)) * 1e-6
            resid = np.abs(A @ np.array([a, b]) - np.array(tus)) / np.array(tus)
            fits[name] = {"tokens_per_s": w.L * w.B / total_s, "total_s_extrapolated": round(total_s, 2),
                          "sample_us": {str(n): round(t, 2) for n, t in zip(pts, tus)},
                          "fit_us": [round(float(a), 3), float(b)],
                          "fit_max_rel_residual": round(float(resid.max()), 4)}
        bl.close()
        del bl
        lazy = dict(fits["lazy"])
        lazy["speedup_vs_lazy"] = round(value / lazy["tokens_per_s"], 1)
        lazy["note"] = ("Lazy per-position device time measured at the sampled positions with HIP events "
                        "and integrated over n = 1..L with an affine fit (fit_max_rel_residual: the fit's "
                        "largest relative miss at the sampled positions); a full Lazy generation of this "
                        "workload would take total_s_extrapolated seconds")
        ablations = {k: {"tokens_per_s": round(v["tokens_per_s"], 2),
                         "total_s_extrapolated": v["total_s_extrapolated"], "fit_us": v["fit_us"],
                         "fit_max_rel_residual": v["fit_max_rel_residual"]}
                     for k, v in fits.items()}
        # the tiled path without chunks (one position per launch), with and without graphs
        for name, graphs in (("tiled_per_position_graphs", True), ("tiled_per_position_no_graphs", False)):
            pc = fi.Context(torch.from_numpy(h).cuda(), w.B, chunk_direct=False, use_graphs=graphs)
            pc.set_input(x1)
            pc.generate(min(L, 4096), want_y=False)          # warm-up (graphs, caches)
            pc.reset()
            pc.set_input(x1)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            pc.generate(L, want_y=False)
            torch.cuda.synchronize()
            ablations[name] = {"tokens_per_s": round(L * w.B / (time.perf_counter() - t0), 1)}
            pc.close()
            del pc
        ablations["note"] = ("the pages' ablations on this workload: Lazy / Eager and their non-layer-"
                             "parallel forms (NP: the per-row work launched layer by layer), each timed at "
                             "sampled positions and integrated with an affine fit in its per-position work; "
                             "the tiled path with one launch (or graph) per position instead of chunks, "
                             "with and without graphs, one timed generation each")
        log("bench: ablations " + ", ".join(f"{k} {v['tokens_per_s']:,.0f}" for k, v in ablations.items()
                                            if isinstance(v, dict)))

    prefill = None
    if not args.no_prefill_leg:
        # prompts of P positions: eager (all positions of a layer at once) against P
        # teacher-forced positions (chunks); each timed warm, on device events
        prefill = {}
        for P in sorted({min(32768, w.L // 4), min(65536, w.L // 2)}):
            xp = torch.from_numpy(np.random.default_rng(5).standard_normal((P, w.B, w.D)).astype(np.float32)).cuda()
            row = {}
            for name, eager in (("eager", True), ("steps", False)):
                pf = fi.Context(torch.from_numpy(h).cuda(), w.B, eager_prefill=eager, tau_split=split)
                ms = []
                for _ in range(3):
                    pf.reset()
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    pf.prefill(xp, want_y=False)
                    b.record()
                    torch.cuda.synchronize()
                    ms.append(a.elapsed_time(b))
                pf.close()
                del pf
                row[f"{name}_ms"] = round(float(np.median(ms[1:])), 3)
                row[f"{name}_tokens_per_s"] = round(P * w.B / (np.median(ms[1:]) * 1e-3), 1)
            prefill[f"P={P}"] = row
            del xp
            log(f"bench: prefill P={P}: eager {row['eager_ms']} ms, steps {row['steps_ms']} ms")
        prefill["note"] = ("fi_prefill of a seeded N(0,1) prompt at position 0, eager (layer by layer, all "
                           "positions at once; the gray blocks after n <= P batched per class, the widest "
                           "after the layers) against P teacher-forced positions (chunks); median of two warm "
                           "runs, HIP events on the stream")

    dd = None
    if not args.no_dd_leg:
        # data-dependent filters (taps arriving with the data), one layer of the workload's
        # channels over L_dd positions, against the fixed-filter path with one launch per
        # position at the same shape (both one position at a time, no chunks)
        Ld = min(16384, w.L)
        rng = np.random.default_rng(9)
        xd = torch.from_numpy(rng.standard_normal((Ld, w.B, w.D)).astype(np.float32)).cuda()
        hd = torch.from_numpy((rng.standard_normal((Ld, w.B, w.D)) *
                               np.exp(-np.arange(Ld) / 2048.0)[:, None, None]).astype(np.float32)).cuda()
        yd = torch.empty_like(xd)
        ddc = fi.DDContext(w.B, w.D, Ld)
        ms = []
        for _ in range(2):
            ddc.reset()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            ddc.run(xd, hd, yd)
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        ddc.close()
        del ddc
        hf = torch.from_numpy(np.ascontiguousarray(h[:1, :, :Ld])).cuda()
        fx = fi.Context(hf, w.B, chunk_direct=False)
        fx.set_input(xd[0])
        fx.generate(Ld, want_y=False)      # warm
        fx.reset()
        fx.set_input(xd[0])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fx.generate(Ld, want_y=False)
        b.record()
        torch.cuda.synchronize()
        fixed_ms = a.elapsed_time(b)
        fx.close()
        del fx
        dd = {"L": Ld, "B": w.B, "D": w.D, "ms": round(ms[-1], 3),
              "tokens_per_s": round(Ld * w.B / (ms[-1] * 1e-3), 1),
              "fixed_filter_per_position_tokens_per_s": round(Ld * w.B / (fixed_ms * 1e-3), 1),
              "note": ("fi_dd_run over L positions of one layer (x and taps h seeded, given per position), "
                       "warm, HIP events; beside it the fixed-filter path at the same shape with one launch "
                       "per position (chunks off), one warm generation")}
        log(f"bench: data-dependent filters L={Ld}: {dd['tokens_per_s']:,.0f} tokens/s; fixed filters per "
            f"position {dd['fixed_filter_per_position_tokens_per_s']:,.0f}")
        # the workload's whole stack with data-dependent taps (fi_dd_stack_*): every layer's taps
        # per position, tanh between layers, over Ls positions
        Ls = min(4096, w.L)
        hs = torch.from_numpy((rng.standard_normal((Ls, w.M, w.B, w.D)) / np.sqrt(64.0) *
                               np.exp(-np.arange(Ls) / 2048.0)[:, None, None, None]).astype(np.float32)).cuda()
        ys = torch.empty_like(hs)
        sdc = fi.DDContext(w.B, w.D, Ls, layers=w.M)
        sms = []
        for _ in range(2):
            sdc.reset()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            sdc.run(xd[:Ls], hs, ys)
            b.record()
            torch.cuda.synchronize()
            sms.append(a.elapsed_time(b))
        sdc.close()
        del sdc, hs, ys
        dd["stack"] = {"M": w.M, "L": Ls, "ms": round(sms[-1], 3),
                       "tokens_per_s": round(Ls * w.B / (sms[-1] * 1e-3), 1),
                       "note": "fi_dd_stack_* over L positions of all the workload's layers (layer 0's input and "
                               "every layer's taps given per position, tanh between layers), warm, HIP events"}
        log(f"bench: data-dependent stack M={w.M} L={Ls}: {dd['stack']['tokens_per_s']:,.0f} tokens/s")

    cpu = None if args.no_cpu_baseline else cpu_baseline(w, h)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded random filters and first input, recipe in DESIGN.md)",
        "config": {"workload": w.name, "M": w.M, "B": w.B, "D": w.D, "L": L,
                   "block_paths": ["fft" if p == fi.PATH_FFT else "direct" for (_, p, _, _) in tau]},
        "split_calibration": {"per_candidate": calib,
                              "note": "fi_init timed one chunk of 2^g positions and the class-g FFT block "
                                      "after it per candidate g (the hybrid rule on the chunk path); the "
                                      "cheapest modeled run sets the split"} if calib else None,
        "latency_us": {"p50": round(float(np.percentile(lat, 50)), 2),
                       "p99": round(float(np.percentile(lat, 99)), 2),
                       "max": round(float(lat.max()), 1),
                       "per_class_median": per_class},
        "roofline": roofline,
        "chunk_kernel": chunk,
        "defer_wide": defer,
        "longer_chunks": longer,
        "lazy_gpu": lazy,
        "ablations": ablations,
        "prefill": prefill,
        "data_dependent": dd,
        "pareto": {"per_size": par,
                   "note": "device time of one gray-block launch per block size at this shape, each path where "
                           "it exists (direct: the per-position kernel with the red cells; fft: the transform "
                           "kernels alone); inside chunks the direct blocks below the split run as per-target "
                           "sums instead (chunk_kernel)"} if par else None,
        "hyena_block": hyena,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
