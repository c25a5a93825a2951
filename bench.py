#!/usr/bin/env python3
"""Benchmark: microseconds per SAGA + Atop-N decode-attention step and achieved
HBM bandwidth at 128K context on one MI355X.

A step is one decode token through all layers of the workload: for each layer,
the score/compare/compact pass over the key cache (with the exact threshold
refresh on every R-th step, found from the previous refresh's survivors as a
pivot) and the sparse softmax + gather-PV.  Inputs are
seeded synthetic tensors already resident in HBM.  The dense full-attention
GQA kernel runs on its own cache in the same process, and the fp64 CPU oracle
is timed on a bounded sample on the host cores.  Besides the mean over the
timed steps (`value`), per-step p10/p50/p90 and the medians of refresh and
non-refresh steps are reported (`per_step_us`), and the dominant kernel's rate
is given against both the 8 TB/s spec and the library's plain streaming-read
probe over the same caches (`roofline.probe_read_gbps`, `frac_of_probe`).
Before the W warmup steps the step loop runs untimed for about 50 ms, so the
timed steps see the GPU in the steady state of a running decode loop rather
than just out of the idle time of setup.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "µs per decode-attention step and achieved HBM GB/s at 128K ctx, 1 MI355X"
PEAK_HBM = 8.0e12  # MI355X HBM3E, bytes/s
MALL_BYTES = 256 << 20  # MI355X Infinity Cache: caches larger than this stream from HBM
ROTATE_K_BYTES = 1 << 30  # single-layer workloads rotate over >= 1 GiB of key caches
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
DOMINANT = "saga::k_select"  # the streaming score/compare/compact kernel (any instantiation)


def traffic_file(workload: str) -> str:
    """Counter summary of one workload (name, with any size overrides)."""
    return os.path.join(PROFILES, "traffic_" + workload.replace(" ", "_").replace("=", "") + ".json")


# The sources the decode-step kernels are built from (the key-merge sources,
# merge.hip and merge_kernels.hpp, do not touch them).
DECODE_SOURCES = ("saga.hip", "saga_device.hpp", "saga_kernels.hpp")


def kernel_source_hash() -> str:
    """sha256 over the decode path's HIP sources, so counter figures taken for other
    code are not reused."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_asymmetric_head_amd", "csrc")
    for f in sorted(DECODE_SOURCES):
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def _kernel_key(name: str) -> str:
    """rocprofv3's kernel name without the return type and argument list."""
    n = name.replace("void ", "", 1)
    return n[:n.index("(")] if "(" in n else n


def summarize_pmc(fetch_csv: str, write_csv: str, copy_mib: int, out: str, workload: str,
                  shape: dict, dominant: str | None = None) -> dict:
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) of
    `bench.py --calibrate-copy MIB` into HBM bytes per launch of every library kernel,
    each counter scaled by what it reads for the calibration copy of known size.  The
    summary names the workload and shape it was taken on and the kernel sources' hash;
    `measured_traffic` reports it only for that same workload, shape and code."""
    import csv
    import statistics

    def per_kernel(path):
        vals = {}
        for r in csv.DictReader(open(path)):
            vals.setdefault(_kernel_key(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return vals

    known_kib = copy_mib * 1024.0
    kernels: dict = {}
    scales = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        v = per_kernel(path)
        copy = [x for k, xs in v.items() if "copyBuffer" in k for x in xs if x > 0.25 * known_kib]
        if not copy:
            raise SystemExit(f"{path}: calibration copy not found")
        factor = known_kib / statistics.median(copy)
        scales[name] = {"copy_counter_kib": statistics.median(copy), "scale": round(factor, 4)}
        for k, xs in v.items():
            if not k.startswith("saga::"):
                continue
            e = kernels.setdefault(k, {})
            e[name] = {"counter_kib_per_launch": statistics.median(xs), "launches": len(xs)}
    for k, e in kernels.items():
        e["bytes_per_launch"] = round(sum(
            e[c]["counter_kib_per_launch"] * scales[c]["scale"] for c in e if c in scales) * 1024.0)
    dom = dominant or max((k for k in kernels if k.startswith(DOMINANT)),
                          key=lambda k: kernels[k].get("FETCH_SIZE", {}).get("launches", 0),
                          default=None)
    if dom is None:
        raise SystemExit(f"{fetch_csv}: no {DOMINANT} launches found")
    summary = {"workload": workload, "shape": shape, "dominant": dom,
               "traffic_bytes_per_launch": kernels[dom]["bytes_per_launch"],
               "kernels": kernels, "scales": scales,
               "calibration": f"__amd_rocclr_copyBuffer of {copy_mib} MiB (torch D2D copy)",
               "kernel_source_sha256": kernel_source_hash()}
    with open(out, "w") as f:
        json.dump(summary, f, indent=1)
        f.write("\n")
    return summary


def measured_traffic(workload: str, shape: dict, path: str | None = None):
    """The committed counter summary of this workload, or None when there is none,
    or it was taken on another shape or on other kernel sources."""
    try:
        t = json.load(open(path or traffic_file(workload)))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    if t.get("workload") != workload or t.get("shape") != shape:
        return None
    return t


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="llama32-1b-128k-16L")
    ap.add_argument("--B", type=int, default=0, help="override the workload's batch size")
    ap.add_argument("--l-kv", type=int, default=0, help="override the workload's context length")
    ap.add_argument("--R", type=int, default=0, help="override the workload's refresh period")
    ap.add_argument("--N", type=int, default=0, help="override the workload's N")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of HIP graphs")
    ap.add_argument("--no-read-sweep", action="store_true",
                    help="skip the search for the fastest cold read of the caches")
    ap.add_argument("--cpu-sample-layers", type=int, default=16)
    ap.add_argument("--kernel-timing-steps", type=int, default=8)
    ap.add_argument("--no-merge", action="store_true",
                    help="skip the GQA -> SAGA key-merge (conversion) timing")
    ap.add_argument("--merge-only", action="store_true",
                    help="time only the GQA -> SAGA key merge and print its JSON")
    ap.add_argument("--merge-reps", type=int, default=20)
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the workload's per-kernel counter traffic summary and exit")
    ap.add_argument("--caches", type=int, default=0,
                    help="independent seeded caches per pass (default: the workload's layers, "
                         "or for a one-layer workload enough caches for 1 GiB of keys)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run 4 plain device-to-device copies of MIB MiB (a reference "
                         "kernel of known traffic for hardware counter runs)")
    return ap.parse_args()


def merge_bench(torch, reps: int, warmup: int = 2) -> dict:
    """Whole-call time of the GQA -> SAGA key merge (eqs. 13-15, Theorem 4.2) on
    one attention layer of each converted model's shape, 16384 calibration tokens,
    inputs resident in HBM; HIP events on the stream the library launches on."""
    from sparse_asymmetric_head_amd import workload as wl
    from sparse_asymmetric_head_amd.merge import KeyMerge

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    res = {}
    for cfg in map(wl.merge_config, wl.MERGE_BENCH):
        n, h_q, h_kt, d, dm = cfg.n, cfg.h_q, cfg.h_kt, cfg.d, cfg.d_model
        X, Q, W = wl.make_merge_inputs(cfg, 1, dev)
        m = KeyMerge(n, h_q, h_kt, d, dm, device=dev)
        torch.cuda.synchronize()
        times = []
        with torch.cuda.stream(stream):
            for i in range(warmup + reps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                m(X, Q, W, stream=stream)
                e1.record(stream)
                stream.synchronize()
                if i >= warmup:
                    times.append(e0.elapsed_time(e1) * 1e3)
        times.sort()
        us = times[len(times) // 2]
        P = h_kt * (h_kt - 1) // 2
        proj_flop = 2 * n * dm * h_kt * d
        gram_flop = 2 * (n * h_q + n * P) * d * d
        in_bytes = 2 * (n * dm + n * h_q * d + h_kt * d * dm)
        res[cfg.name] = {"n": n, "h_q": h_q, "h_kt": h_kt, "d": d, "d_model": dm,
                         "us_per_layer": round(us, 1), "us_p10": round(times[len(times) // 10], 1),
                         "pairs": [tuple(p) for p in m.pairs.cpu().tolist()],
                         "projection_gflop": round(proj_flop / 1e9, 2),
                         "gram_gflop": round(gram_flop / 1e9, 2),
                         "input_mb": round(in_bytes / 1e6, 1)}
        log(f"key merge {cfg.name}: {us:.1f} us per layer (p10 {times[len(times) // 10]:.1f})")
        del X, Q, W, m
    return res


def resolve_workload(args):
    """(cfg, config index, workload name with its overrides, caches per pass, shape)."""
    from sparse_asymmetric_head_amd import workload as wl

    cfg = next((c for c in wl.CONFIGS if c.name == args.config), None)
    if cfg is None:
        return None
    ci = wl.config_index(cfg)
    over = {k: v for k, v in (("B", args.B), ("l_kv", args.l_kv), ("R", args.R), ("N", args.N))
            if v > 0}
    if over:  # the same seeded recipe at another size or refresh period (a sweep point)
        cfg = cfg.with_(**over)
    k_bytes = cfg.B * cfg.h_k * cfg.l_kv * cfg.d * 2
    caches = rotation_caches(cfg.layers, k_bytes, args.caches)
    name = cfg.name + "".join(f" {k}={v}" for k, v in over.items())
    if caches != cfg.layers:
        name += f" caches={caches}"
    shape = {"B": cfg.B, "h_q": cfg.h_q, "h_k": cfg.h_k, "h_v": cfg.h_v, "d": cfg.d,
             "l_kv": cfg.l_kv, "N": cfg.N, "R": cfg.R, "caches": caches}
    return cfg, ci, name, caches, shape


def rotation_caches(layers: int, k_bytes: int, forced: int = 0) -> int:
    """Independent caches one timed pass runs over: a multi-layer workload runs its
    layers; a one-layer workload rotates over enough seeded caches that a pass reads at
    least 1 GiB of keys, so no step finds its cache in the 256 MB Infinity Cache."""
    if forced > 0:
        return forced
    if layers > 1:
        return layers
    return max(1, min(1024, -(-ROTATE_K_BYTES // k_bytes)))


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the SAGA decode step here runs on a single "
              "MI355X with no collectives; run with --gpus 1.", file=sys.stderr)
        return 2
    res = None if args.merge_only else resolve_workload(args)
    if res is None and not args.merge_only:
        print(f"unknown config {args.config}", file=sys.stderr)
        return 2
    if args.summarize_pmc:
        cfg, ci, wname, L, shape = res
        print(json.dumps(summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1],
                                       args.calibrate_copy or 256, traffic_file(wname), wname,
                                       shape)))
        return 0

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    from sparse_asymmetric_head_amd import saga
    from sparse_asymmetric_head_amd import workload as wl

    saga.lib()  # fails loudly when the HIP library is missing
    if args.merge_only:
        print(json.dumps({"gqa_to_saga_merge": merge_bench(torch, args.merge_reps)}), flush=True)
        return 0
    cfg, ci, wname, L, shape = res
    B, h_q, h_k, h_v, d, l_kv, N, R, T = (cfg.B, cfg.h_q, cfg.h_k, cfg.h_v, cfg.d, cfg.l_kv,
                                           cfg.N, cfg.R, cfg.steps)
    # a pass runs every cache once (one decode token through all layers, or one
    # layer-step on each rotated cache); a workload step is cfg.layers of them
    steps_per_pass = L / cfg.layers
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration: 4 copies of {args.calibrate_copy} MiB "
            f"({n} bytes read and {n} written per copy)")
        del src, dst
    log(f"workload {wname}: B={B} h_q={h_q} h_k={h_k} h_v={h_v} d={d} l_kv={l_kv} N={N} "
        f"R={R} layers={cfg.layers} caches per pass={L}")

    # ------------------------------------------------------------ inputs
    layers = [wl.make_layer(cfg, l, device=dev, cfg_index=ci) for l in range(L)]
    Qall = torch.stack([x["Q"] for x in layers], dim=1).contiguous()  # [T][L][B][h_q][d]
    Ks = [x["K"] for x in layers]
    Vs = [x["V"] for x in layers]
    torch.cuda.synchronize()
    log("inputs generated")

    ws = saga.alloc_workspace(saga.saga_workspace_bytes(B, h_q, h_k, h_v, d, l_kv, N), dev)
    taus = torch.zeros(L, B, h_q, dtype=torch.float32, device=dev)
    pivots = torch.full((L, B, h_q, N), -1, dtype=torch.int32, device=dev)
    Os = torch.empty(L, B, h_q, d, dtype=torch.float32, device=dev)
    cnts = torch.empty(L, B, h_q, dtype=torch.int32, device=dev)
    qbuf = torch.empty(L, B, h_q, d, dtype=torch.bfloat16, device=dev)

    # refresh modes of saga_decode_step_pivot: 0 compare with tau, 1 full
    # exact refresh (records the pivot), 2 exact refresh from the pivot
    def layer_pass(mode: int, q):
        for l in range(L):
            saga.saga_decode_step_pivot(q[l], Ks[l], Vs[l], N, taus[l], pivots[l], mode,
                                        Os[l], cnts[l], ws)

    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        layer_pass(1, Qall[0])  # eager first call: loads the kernels; first refresh of every layer
        layer_pass(0, Qall[0])
    stream.synchronize()
    # One graph per (query step, refresh) pair, each reading that step's
    # resident queries: a step then replays one graph and copies nothing.
    graphs = {}
    if not args.no_graph:
        for i in range(T):
            for refresh in ((i % R == 0,) if T % R == 0 else (True, False)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    layer_pass(2 if refresh else 0, Qall[i])
                graphs[(i, refresh)] = g
        log(f"graphs captured ({len(graphs)})")

    def step(t: int):
        refresh = (t % R) == 0
        if graphs:
            graphs[(t % T, refresh)].replay()
        else:
            layer_pass(2 if refresh else 0, Qall[t % T])

    sel_counts = []
    with torch.cuda.stream(stream):
        # Settle: untimed steps until the GPU has run this loop for ~50 ms.
        # After the idle time of setup, the first ~100 steps run a few
        # percent slower than the steady state a decode loop sits in; the
        # warmup steps and the timed steps below follow as the contract has
        # them (every step of the trajectory does its full work).
        t_settle = time.perf_counter() + 0.05
        t = 0
        while time.perf_counter() < t_settle:
            for _ in range(4):
                step(t)
                t += 1
            stream.synchronize()
        for t in range(args.warmup):
            step(t)
        stream.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t_wall0 = time.perf_counter()
        ev0.record(stream)
        for t in range(args.warmup, args.warmup + args.steps):
            step(t)
        ev1.record(stream)
        stream.synchronize()
        t_wall1 = time.perf_counter()
        gpu_ms = ev0.elapsed_time(ev1)
        wall_ms = (t_wall1 - t_wall0) * 1e3
        sel_counts.append(cnts.float().mean().item())
        # A second pass over the same steps with one event between consecutive
        # steps gives the per-step distribution (refresh and non-refresh steps
        # apart); the events cost a little, so `value` comes from the pass above.
        # The warmup steps run again first, so the second pass starts from the
        # same state (the exact refresh at step 0) as the timed one.
        for t in range(args.warmup):
            step(t)
        stream.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        evs[0].record(stream)
        for i, t in enumerate(range(args.warmup, args.warmup + args.steps)):
            step(t)
            evs[i + 1].record(stream)
        stream.synchronize()
        # per workload step: a pass runs steps_per_pass of them (one, unless a
        # one-layer workload rotates over several caches)
        step_us = [evs[i].elapsed_time(evs[i + 1]) * 1e3 / steps_per_pass
                   for i in range(args.steps)]
    pass_us = max(gpu_ms, wall_ms) / args.steps * 1e3
    us_per_step = pass_us / steps_per_pass
    ms_per_step = us_per_step / 1e3
    ref_us = [u for i, u in enumerate(step_us) if (args.warmup + i) % R == 0]
    non_us = [u for i, u in enumerate(step_us) if (args.warmup + i) % R != 0]

    def pct(xs, q):
        xs = sorted(xs)
        return xs[min(len(xs) - 1, max(0, round(q * (len(xs) - 1))))] if xs else None

    per_step = {"p10": pct(step_us, 0.1), "p50": pct(step_us, 0.5), "p90": pct(step_us, 0.9),
                "non_refresh_p50": pct(non_us, 0.5),
                "refresh_p50": pct(ref_us, 0.5), "refresh_steps": len(ref_us)}
    per_step = {k: (round(v, 2) if isinstance(v, float) else v) for k, v in per_step.items()}
    log(f"timed {args.steps} passes of {steps_per_pass:g} steps: {us_per_step:.1f} us/step "
        f"(events {gpu_ms:.3f} ms, "
        f"wall {wall_ms:.3f} ms); per step p10/p50/p90 {per_step['p10']}/{per_step['p50']}/"
        f"{per_step['p90']} us, non-refresh p50 {per_step['non_refresh_p50']}, refresh p50 "
        f"{per_step['refresh_p50']}")

    # ------------------------------------------------------------ kernel timing pass
    # The dominant kernel (the streaming score/compare/compact pass) timed
    # with HIP events on the stream it runs on: a graph of its launches over
    # all layers (non-refresh), replayed back to back; per-launch time =
    # elapsed / launches.  (Events around single launches would add several
    # microseconds of event overhead to each.)
    reps = max(1, args.kernel_timing_steps)
    with torch.cuda.stream(stream):
        qbuf.copy_(Qall[(args.warmup + args.steps) % T])

        inner = max(1, -(-64 // L))  # >= 64 launches per graph: amortise the graph launch

        def select_pass():
            for _ in range(inner):
                for l in range(L):
                    saga.saga_select(qbuf[l], Ks[l], h_v, N, taus[l], False, ws, stream)

        select_pass()
        stream.synchronize()
        sg = None
        if not args.no_graph:
            sg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(sg, stream=stream):
                select_pass()
        run_sel = sg.replay if sg is not None else select_pass
        run_sel()
        stream.synchronize()
        k0 = torch.cuda.Event(enable_timing=True)
        k1 = torch.cuda.Event(enable_timing=True)
        k0.record(stream)
        for _ in range(reps):
            run_sel()
        k1.record(stream)
        stream.synchronize()
    sel_us = k0.elapsed_time(k1) * 1e3 / (reps * L * inner)
    mean_count = sum(sel_counts) / len(sel_counts)

    # ------------------------------------------------------------ achievable read
    # The library's plain streaming-read probe over the same key caches, same
    # protocol: the achievable-read reference for the streaming kernel.
    sink = torch.zeros(saga.PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
    with torch.cuda.stream(stream):

        def probe_pass():
            for _ in range(inner):
                for l in range(L):
                    saga.saga_read_probe(Ks[l], sink, stream)

        probe_pass()
        stream.synchronize()
        pg = None
        if not args.no_graph:
            pg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(pg, stream=stream):
                probe_pass()
        run_probe = pg.replay if pg is not None else probe_pass
        run_probe()
        stream.synchronize()
        k0.record(stream)
        for _ in range(reps):
            run_probe()
        k1.record(stream)
        stream.synchronize()
    probe_us = k0.elapsed_time(k1) * 1e3 / (reps * L * inner)
    probe_gbps = B * h_k * l_kv * d * 2 / (probe_us * 1e-6) / 1e9
    log(f"read probe over the same caches: {probe_us:.2f} us/launch -> {probe_gbps:.0f} GB/s")

    # The fastest cold read of the same caches among the library's probe shapes
    # (workgroups x waves x loads in flight per lane, contiguous ranges or
    # interleaved runs): the best read pattern this GPU offers for this buffer size.
    best_read = None
    if not args.no_read_sweep:
        for blocks in (256, 512, 1024):
            for waves, loads in ((4, 4), (4, 8), (4, 16), (8, 4), (8, 8)):
                for chunked in (True, False):
                    def shape_pass():
                        for _ in range(inner):
                            for l in range(L):
                                saga.saga_read_probe_shape(Ks[l], sink, blocks, waves, loads,
                                                           chunked, stream)
                    with torch.cuda.stream(stream):
                        shape_pass()
                        stream.synchronize()
                        sg = None
                        if not args.no_graph:
                            sg = torch.cuda.CUDAGraph()
                            with torch.cuda.graph(sg, stream=stream):
                                shape_pass()
                        run_s = sg.replay if sg is not None else shape_pass
                        run_s()
                        stream.synchronize()
                        k0.record(stream)
                        for _ in range(reps):
                            run_s()
                        k1.record(stream)
                        stream.synchronize()
                    us = k0.elapsed_time(k1) * 1e3 / (reps * L * inner)
                    if best_read is None or us < best_read["us"]:
                        best_read = {"us": round(us, 3), "blocks": blocks, "waves": waves,
                                     "loads_per_lane": loads,
                                     "pattern": "contiguous ranges" if chunked else "interleaved runs"}
        best_read["gbps"] = round(B * h_k * l_kv * d * 2 / (best_read["us"] * 1e-6) / 1e9, 1)
        log(f"best cold read of the same caches: {best_read['us']:.2f} us/launch -> "
            f"{best_read['gbps']:.0f} GB/s ({best_read['blocks']} x {best_read['waves']} waves x "
            f"{best_read['loads_per_lane']} loads, {best_read['pattern']})")

    k_bytes = B * h_k * l_kv * d * 2
    q_bytes = B * h_q * d * 2
    tau_bytes = B * h_q * 4
    o_bytes = B * h_q * d * 4
    v_bytes = B * h_q * mean_count * d * 2
    select_alg = k_bytes + q_bytes + tau_bytes
    pass_alg = L * (k_bytes + q_bytes + tau_bytes + o_bytes + v_bytes)
    achieved = select_alg / (sel_us * 1e-6)
    log(f"select kernel {sel_us:.2f} us/launch -> {achieved / 1e9:.0f} GB/s")

    # ------------------------------------------------------------ SAGA full attention
    # The decoupled heads without the sparsity (every position), on the same
    # caches: K read once per key head, V once per value head.
    full = None
    if not args.no_dense:
        fws = torch.empty(saga.saga_full_attention_workspace_bytes(B, h_q, h_k, h_v, d, l_kv),
                          dtype=torch.uint8, device=dev)
        fO = torch.empty(L, B, h_q, d, dtype=torch.float32, device=dev)

        def full_pass():
            for l in range(L):
                saga.saga_full_attention(qbuf[l], Ks[l], Vs[l], fO[l], fws)

        with torch.cuda.stream(stream):
            full_pass()
            stream.synchronize()
            fg = None
            if not args.no_graph:
                fg = torch.cuda.CUDAGraph()
                with torch.cuda.graph(fg, stream=stream):
                    full_pass()
            run_full = fg.replay if fg is not None else full_pass
            for _ in range(args.warmup):
                run_full()
            stream.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            w0 = time.perf_counter()
            e0.record(stream)
            for _ in range(args.steps):
                run_full()
            e1.record(stream)
            stream.synchronize()
            w1 = time.perf_counter()
        full_us = max(e0.elapsed_time(e1), (w1 - w0) * 1e3) / args.steps * 1e3 / steps_per_pass
        full_bytes = cfg.layers * (B * (h_k + h_v) * l_kv * d * 2 + q_bytes + o_bytes)
        full = {"us_per_step": round(full_us, 2),
                "hbm_gbps": round(full_bytes / (full_us * 1e-6) / 1e9, 1),
                "speedup_saga_sparse_vs_full": round(full_us / us_per_step, 3)}
        log(f"SAGA full attention (h_k={h_k}, h_v={h_v}): {full_us:.1f} us/step, "
            f"{full['hbm_gbps']:.0f} GB/s")
        del fws, fO

    # ------------------------------------------------------------ dense baseline
    dense = None
    if cfg.dense_h_kv and not args.no_dense:
        del layers
        dl = [wl.make_dense_layer(cfg, l, device=dev, cfg_index=ci) for l in range(L)]
        hk = cfg.dense_h_kv
        dws = torch.empty(saga.saga_dense_workspace_bytes(B, h_q, hk, d, l_kv), dtype=torch.uint8,
                          device=dev)
        dO = torch.empty(L, B, h_q, d, dtype=torch.float32, device=dev)

        def dense_pass():
            for l in range(L):
                saga.saga_dense_gqa_baseline(dl[l]["Q"], dl[l]["K"], dl[l]["V"], dO[l], dws)

        with torch.cuda.stream(stream):
            dense_pass()
            stream.synchronize()
            dg = None
            if not args.no_graph:
                dg = torch.cuda.CUDAGraph()
                with torch.cuda.graph(dg, stream=stream):
                    dense_pass()
            run = dg.replay if dg is not None else dense_pass
            for _ in range(args.warmup):
                run()
            stream.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            w0 = time.perf_counter()
            e0.record(stream)
            for _ in range(args.steps):
                run()
            e1.record(stream)
            stream.synchronize()
            w1 = time.perf_counter()
        dense_us = max(e0.elapsed_time(e1), (w1 - w0) * 1e3) / args.steps * 1e3 / steps_per_pass
        dense_bytes = cfg.layers * (2 * B * hk * l_kv * d * 2 + q_bytes + o_bytes)
        dense = {"h_kv": hk, "us_per_step": round(dense_us, 2),
                 "hbm_gbps": round(dense_bytes / (dense_us * 1e-6) / 1e9, 1),
                 "speedup_saga_vs_dense": round(dense_us / us_per_step, 3)}
        if full is not None:
            full["speedup_vs_dense_gqa"] = round(dense_us / full["us_per_step"], 3)
        log(f"dense GQA h_kv={hk}: {dense_us:.1f} us/step, speedup {dense_us / us_per_step:.2f}x")
        del dl

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        lib = oracle.load()
        S = max(1, min(args.cpu_sample_layers, L))
        # the oracle refreshes at every step t with t % R == 0: at least two refreshes
        # and about 10-30 s of oracle work over the sample
        steps = min(4 * R, max(R + 1, 64))
        n_ref = -(-steps // R)
        n_norm = steps - n_ref
        t_one = t_all = 0.0
        for l in range(S):
            x = wl.make_layer(cfg, l, device=dev, cfg_index=ci, steps=steps)
            Qh, Kh, Vh = (oracle._u16(x[k]) for k in ("Q", "K", "V"))
            del x
            c0 = time.perf_counter()
            oracle.trajectory(Qh[:1], Kh, Vh, h_k, h_v, N, R, lib=lib)
            c1 = time.perf_counter()
            oracle.trajectory(Qh, Kh, Vh, h_k, h_v, N, R, lib=lib)
            c2 = time.perf_counter()
            t_one += c1 - c0
            t_all += c2 - c1
        t_ref = t_one / S
        # the full trajectory holds n_ref refresh steps and n_norm non-refresh ones
        t_norm = max((t_all / S - n_ref * t_ref) / n_norm, 0.0) if n_norm else 0.0
        cpu_us = cfg.layers * (t_ref + (R - 1) * t_norm) / R * 1e6
        # the same oracle on one core: one layer's refresh step and one plain step
        cores = oracle.num_threads(lib)
        oracle.set_num_threads(1, lib)
        x = wl.make_layer(cfg, 0, device=dev, cfg_index=ci, steps=2)
        Qh, Kh, Vh = (oracle._u16(x[k]) for k in ("Q", "K", "V"))
        del x
        c0 = time.perf_counter()
        oracle.trajectory(Qh[:1], Kh, Vh, h_k, h_v, N, R, lib=lib)
        c1 = time.perf_counter()
        oracle.trajectory(Qh[:2], Kh, Vh, h_k, h_v, N, max(R, 2), lib=lib)
        c2 = time.perf_counter()
        oracle.set_num_threads(cores, lib)
        one_ref, one_norm = c1 - c0, max((c2 - c1) - (c1 - c0), 0.0)
        one_us = cfg.layers * (one_ref + (R - 1) * one_norm) / R * 1e6
        cpu_model = ""
        try:
            with open("/proc/cpuinfo") as f:
                cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")),
                                 "")
        except OSError:
            pass
        cpu = {"value": round(cpu_us, 1), "unit": "us/step", "cores": cores,
               "kind": "oracle",
               "single_core_value": round(one_us, 1),
               "host": {"cpu_model": cpu_model, "logical_cpus": os.cpu_count()},
               "sample": (f"{S} of {L} caches x {steps + 1} oracle layer-steps each (one refresh "
                          f"step alone, then {steps} steps with {n_ref} refreshes, at multiples "
                          f"of {R}) of "
                          f"{cfg.name}; per-layer costs amortised over R={R} and scaled to "
                          f"{cfg.layers} layers (refresh {t_ref:.3f} s, non-refresh {t_norm:.3f} s per "
                          f"layer-step, {t_one + t_all:.1f} s of oracle time); single_core_value "
                          f"from layer 0's refresh step and one plain step on one thread "
                          f"(refresh {one_ref:.3f} s, non-refresh {one_norm:.3f} s), scaled alike")}
        log(f"cpu oracle: {cpu_us / 1e3:.1f} ms/step on {cpu['cores']} threads, "
            f"{one_us / 1e3:.1f} ms/step on one ({cpu_model})")

    traffic = measured_traffic(wname, shape)
    merge = None
    if not args.no_merge:
        merge = merge_bench(torch, args.merge_reps)

    out = {
        "metric": METRIC,
        "value": round(us_per_step, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": round(args.steps * steps_per_pass),
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wname,
                   "B": B, "h_q": h_q, "h_k": h_k, "h_v": h_v, "d": d,
                   "l_kv": l_kv, "N": N, "R": R, "layers": cfg.layers, "global_batch": B,
                   "seq_len": l_kv, "parallelism": "single-gpu"},
        # every pass reads L independent caches; beyond the 256 MB Infinity Cache none
        # of them is still on chip when its turn comes again
        "rotation": {"caches_per_pass": L, "passes": args.steps,
                     "k_bytes_per_pass": L * k_bytes,
                     "kv_bytes_resident": L * B * (h_k + h_v) * l_kv * d * 2,
                     "cold": L * B * (h_k + h_v) * l_kv * d * 2 > MALL_BYTES},
        "hbm_gbps": round(pass_alg / (pass_us * 1e-6) / 1e9, 1),
        "us_per_layer_step": round(pass_us / L, 3),
        "mean_survivors_per_row": round(mean_count, 1),
        "roofline": {"bound": "hbm", "kernel": "k_select (score + compare + compact)",
                     "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM, 4),
                     "traffic": traffic["traffic_bytes_per_launch"] if traffic else None,
                     "traffic_unit": "HBM bytes per launch",
                     "traffic_source": os.path.relpath(traffic_file(wname), ROOT) if traffic else None,
                     "kernel_us": round(sel_us, 3), "bytes_per_launch": select_alg,
                     "probe_read_gbps": round(probe_gbps, 1),
                     "frac_of_probe": round(achieved / 1e9 / probe_gbps, 4),
                     "best_read": best_read,
                     "frac_of_best_read": (round(achieved / 1e9 / best_read["gbps"], 4)
                                           if best_read else None)},
        "per_step_us": per_step,
        "kernel_traffic": ({k: v["bytes_per_launch"] for k, v in traffic["kernels"].items()}
                           if traffic else None),
        "dense_gqa": dense,
        "saga_full_attention": full,
        "gqa_to_saga_merge": merge,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
