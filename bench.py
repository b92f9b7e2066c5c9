#!/usr/bin/env python3
"""Decode benchmark of the int4 KV-cache attention path on one MI355X.

Metric: sdpa_int4 decode microseconds per layer-step and the achieved HBM
bandwidth of the split kernel, on the Llama-3.1-70B-shaped layer at 128K
context (64 query heads / 8 KV heads, head_dim 128, bf16 inputs), cycling
over 80 distinct caches (12.5 GiB, far larger than the 256 MB last-level
cache, so every step streams from HBM).

A step is one pass of the whole hot path over every layer: the split pass,
which also quantises the new token into the layer's cache (the block whose
chunk holds it), then the LSE combine.  The step is
captured once in a HIP graph and replayed.  Inputs are synthetic and seeded
(int4_kv_cache_quant_amd.synth); they are resident in HBM before timing.

Prints one JSON line.  The CPU oracle is timed on the host on one full
layer-step (all query heads of layer 0), which doubles as a parity check of
the GPU outputs of that layer.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sdpa_int4 decode µs/layer-step + achieved HBM GB/s (% peak) at 128K ctx"
HBM_PEAK_GBPS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
CSRC = "int4_kv_cache_quant_amd/csrc/"
KERNEL_SOURCES = {  # the sources a split kernel's traffic summary is tagged with
    "split_mfma": [CSRC + "sdpa_mfma.hip", CSRC + "mfma_common.hpp", CSRC + "srft.hpp", CSRC + "common.hpp"],
    "split_vec": [CSRC + "sdpa_vec.hip", CSRC + "common.hpp"],
    "split_bits_mfma": [CSRC + "bits_mfma.hip", CSRC + "bits_layout.hpp", CSRC + "mfma_common.hpp",
                        CSRC + "srft.hpp", CSRC + "common.hpp"],
    "split_bits": [CSRC + "bits.hip", CSRC + "bits_layout.hpp", CSRC + "common.hpp"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(kernel):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(kernel, workload_name, bits):
    tag = "" if bits == 4 else f"-{bits}bit"
    return os.path.join(PROFILE_DIR, f"traffic_{kernel}_{workload_name}{tag}.json")


def traffic_from_profile(kernel, workload_name, bits=4):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None
    when the kernel source changed since they were taken."""
    path = traffic_path(kernel, workload_name, bits)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != source_sha(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def counter_per_dispatch(run_dir, counter):
    """{dispatch id: (kernel name, summed value)} from a rocprofv3 CSV counter run."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name, val = out.get(r["Dispatch_Id"], (r["Kernel_Name"], 0.0))
                out[r["Dispatch_Id"]] = (name, val + float(r["Counter_Value"]))
    return out


def traffic_summary(fetch_dir, write_dir, workload, calib_mib, commands, kernel="split_mfma", bits=4):
    """Calibrated HBM bytes per split launch from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch) of
    `bench.py --no-graph --copy-calibration-mib N`: each counter is scaled by
    what it reads for the plain elementwise copy of N MiB (N MiB read and N
    MiB written).  Writes profiles/traffic_<kernel>_<workload>[-<b>bit].json."""
    import numpy as np
    from int4_kv_cache_quant_amd import synth
    w = synth.WORKLOADS[workload]
    known_kib = calib_mib * 1024.0
    rec = {"workload": w.name, "calibration_copy_mib": calib_mib, "commands": commands}
    for counter, run_dir, key in (("FETCH_SIZE", fetch_dir, "fetch"), ("WRITE_SIZE", write_dir, "write")):
        per = counter_per_dispatch(run_dir, counter)
        calib = sorted((v for n, v in per.values() if "elementwise" in n), reverse=True)[:5]
        split = [v for n, v in per.values() if kernel + "_kernel" in n]
        if len(calib) < 5 or not split:
            raise SystemExit(f"{run_dir}: no calibration copy or split dispatches for {counter}")
        factor = known_kib / float(np.mean(calib))
        rec[f"{key}_kib_per_launch_raw"] = float(np.mean(split))
        rec[f"{key}_calibration_kib_raw"] = float(np.mean(calib))
        rec[f"{key}_factor"] = factor
        rec[f"{key}_bytes_per_launch"] = float(np.mean(split)) * factor * 1024.0
        rec[f"{key}_launches"] = len(split)
    unit = w.Hkv * 2 * (w.D * bits // 8 + 4 * (w.D // 32))
    lens_sum = int(synth.lens(w, 0).astype(np.int64).sum())
    rec["algorithmic_bytes_per_launch"] = lens_sum * unit + w.B * w.Hq * w.D * 2
    rec["hbm_bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    rec["kernel"] = kernel
    rec["code_bits"] = bits
    rec["kernel_source_sha"] = source_sha(kernel)
    path = traffic_path(kernel, w.name, bits)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3, help="workload number (3 = 70B layer at 128K)")
    ap.add_argument("--also", default="1,2,4,5",
                    help="other workloads timed in the same run (step and split only), comma-separated; "
                         "'' for none")
    ap.add_argument("--layers", type=int, default=None, help="distinct caches (default: the workload's)")
    ap.add_argument("--chunk", type=int, default=0, help="force the split chunk (0 = planner default)")
    ap.add_argument("--splits", type=int, default=0,
                    help="force the split count (0 = planner default; below max_len / chunk the pieces "
                         "interleave)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a graph")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling probe")
    ap.add_argument("--chan-scale", action="store_true",
                    help="give K a per-channel scale (seeded; 1/multiplier on the outlier channels)")
    ap.add_argument("--v-rotate", action="store_true",
                    help="rotate V too (seeded signs); outputs are brought back by the inverse rotation")
    ap.add_argument("--srft", action="store_true",
                    help="rotate K by the sign-randomised FFT (seeded signs); a workload that rotates K "
                         "switches from the Walsh-Hadamard rotation to this one")
    ap.add_argument("--srht", action="store_true",
                    help="rotate K by the sign-randomised Walsh-Hadamard transform (seeded signs) on a "
                         "workload that does not rotate it")
    ap.add_argument("--code-bits", type=int, default=4, choices=(2, 3, 4),
                    help="code width of the caches; 2 and 3 take the b-bit path (no rotation or channel "
                         "scale)")
    ap.add_argument("--cpu-threads", type=int, default=None,
                    help="threads of the multi-threaded oracle leg (default: the cores this process may "
                         "use, at most 16)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device-to-device copy of this many MiB (5 times), "
                         "whose counter readings calibrate FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_RUN_DIR", "WRITE_RUN_DIR"),
                    help="write the calibrated HBM traffic of the split kernel from two rocprofv3 "
                         "--pmc runs (FETCH_SIZE, WRITE_SIZE) into profiles/, then exit")
    ap.add_argument("--pmc-commands", default="", help="the profiling commands, recorded with the summary")
    ap.add_argument("--traffic-kernel", default="split_mfma", choices=sorted(KERNEL_SOURCES),
                    help="the split kernel whose dispatches --traffic-summary reads")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args.traffic_summary[0], args.traffic_summary[1], args.workload,
                        args.copy_calibration_mib or 1024, args.pmc_commands, args.traffic_kernel,
                        args.code_bits)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures a single GPU: --gpus {args.gpus} / WORLD_SIZE {world} is not "
              "supported (the decode path has no multi-GPU component; see the sharding notes "
              "in the design document).", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    import int4_kv_cache_quant_amd as otq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    otq.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads and writes n * 4 bytes
        torch.cuda.synchronize()
        log(f"bench: copy calibration {args.copy_calibration_mib} MiB x 5 done")
        del src, dst

    rec = bench_workload(args.workload, args, primary=True)
    others = []
    for tok in [t for t in args.also.split(",") if t.strip()]:
        wn = int(tok)
        if wn == args.workload:
            continue
        torch.cuda.empty_cache()
        others.append(bench_workload(wn, args, primary=False))
    rec["other_workloads"] = others
    print(json.dumps(rec), flush=True)


def stream_ceiling(torch, otq, dev, nbytes, copies, steps):
    """The streaming-read rate of this GPU for reads of nbytes per launch:
    the probe kernel over `copies` distinct buffers (as the split pass cycles
    over distinct caches), replayed in a graph; the best of a few grid sizes."""
    nbytes = (nbytes + 15) // 16 * 16
    bufs = [torch.full((nbytes // 4,), i + 1, dtype=torch.int32, device=dev) for i in range(copies)]
    best = None
    sweep = {}
    for blocks in (512, 1024, 2048, 4096, 8192):
        sink = torch.empty(blocks, dtype=torch.int32, device=dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for b in bufs:
                otq.otq_stream_read_probe(b, sink, nbytes=nbytes, blocks=blocks)
        g.replay()
        torch.cuda.synchronize()
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            g.replay()
        e.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(e) * 1000.0 / (steps * copies)
        gbps = nbytes / (us * 1e-6) / 1e9
        log(f"bench: stream ceiling {nbytes / 2**20:.1f} MiB x {copies}, {blocks} blocks: {us:.2f} us, "
            f"{gbps:.0f} GB/s")
        sweep[blocks] = round(gbps, 1)
        if best is None or gbps > best["GBps"]:
            best = {"GBps": round(gbps, 1), "us_per_launch": round(us, 3), "blocks": blocks}
        del g, sink
    del bufs
    torch.cuda.empty_cache()
    best.update({"kernel": "stream_read (otq_stream_read_probe)", "bytes_per_launch": int(nbytes),
                 "buffers": copies, "frac_of_peak": round(best["GBps"] / HBM_PEAK_GBPS, 4),
                 "GBps_by_blocks": sweep})
    return best


def oracle_cache(oracle, w, host_kv0, rot_norm, rot_kind, bits, threads):
    """Layer 0's K/V quantised by the oracle (not timed)."""
    kb, vb, sg, lam0, vsg0 = host_kv0
    kc, ks = oracle.quantize(kb, w.dtype, signs=sg, rot_norm=rot_norm, threads=threads,
                             chan_scale=lam0, rot_kind=rot_kind, code_bits=bits)
    vc, vs = oracle.quantize(vb, w.dtype, signs=vsg0, rot_norm=rot_norm, threads=threads,
                             rot_kind=rot_kind, code_bits=bits)
    return kc, ks, vc, vs


def oracle_leg(oracle, w, host_kv0, qc, q0, rot_norm, rot_kind, bits, threads, budget_s, max_reps):
    """The oracle's fp64 layer-step of layer 0 on `threads` threads, repeated
    until budget_s of wall time (at least once, at most max_reps times)."""
    _, _, sg, lam0, vsg0 = host_kv0
    kc, ks, vc, vs = qc
    lens0 = synth_lens(w)
    reps = 0
    t = time.perf_counter()
    while True:
        ref = oracle.sdpa(q0, w.dtype, kc, ks, vc, vs, lens0, w.scale, signs=sg, rot_norm=rot_norm,
                          threads=threads, chan_scale=lam0, v_signs=vsg0, rot_kind=rot_kind, code_bits=bits)
        reps += 1
        if time.perf_counter() - t >= budget_s or reps >= max_reps:
            break
    return ref, (time.perf_counter() - t) / reps, reps


def synth_lens(w):
    from int4_kv_cache_quant_amd import synth
    return synth.lens(w, 0)


def bench_workload(wnum, args, primary):
    """Build the workload's caches, time the step, and (for the primary
    workload) the per-kernel durations, bulk append, streaming ceiling and
    the CPU oracle legs.  Returns the record."""
    import numpy as np
    import torch

    import int4_kv_cache_quant_amd as otq
    from int4_kv_cache_quant_amd import synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[wnum]
    L = w.layers if (args.layers is None or not primary) else args.layers
    log(f"bench: workload {wnum} {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} "
        f"T={w.T} layers={L}")

    # ---------------------------------------------------------------- setup
    rot_kind = "srft" if args.srft else "srht"
    bits = args.code_bits
    extra_rot = primary and (args.srft or args.srht)
    chan = primary and args.chan_scale
    vrot = primary and args.v_rotate
    wbits = bits  # b-bit caches take the rotations and the channel scale too
    if args.srft and args.srht:
        sys.exit("bench.py: --srft and --srht name two different K rotations")
    t_setup = time.time()
    caches, k_new, v_new, qs, lens_l, pos_l = [], [], [], [], [], []
    host_kv0 = None
    for l in range(L):
        signs = torch.from_numpy(synth.rot_signs(w, l)).to(dev) if (w.rotate or extra_rot) else None
        lam = torch.from_numpy(synth.chan_scale(w, l)).to(dev) if chan else None
        vsg = torch.from_numpy(synth.v_rot_signs(w, l)).to(dev) if vrot else None
        cache = otq.Int4KVCache(w.B, w.Hkv, w.D, w.capacity, device=dev, rot_signs=signs,
                                chan_scale=lam, v_rot_signs=vsg, rot_kind=rot_kind, code_bits=wbits)
        k = synth.kv(w, l, "k", device=dev)
        v = synth.kv(w, l, "v", device=dev)
        lens = synth.lens(w, l)
        lens_t = torch.from_numpy(lens).to(dev)
        for t0 in range(0, w.T, 16384):
            t1 = min(w.T, t0 + 16384)
            pos = torch.full((w.B,), t0, dtype=torch.int32, device=dev)
            cache.append(k[:, :, t0:t1].contiguous(), v[:, :, t0:t1].contiguous(), pos)
        idx = (lens_t.long() - 1).clamp(min=0)
        ar = torch.arange(w.B, device=dev)
        k_new.append(k[ar, :, idx].contiguous())  # [B, Hkv, D]: the token at lens - 1
        v_new.append(v[ar, :, idx].contiguous())
        if l == 0 and primary and not args.no_cpu:
            host_kv0 = (synth.bits(k), synth.bits(v), None if signs is None else signs.cpu().numpy(),
                        None if lam is None else lam.cpu().numpy(),
                        None if vsg is None else vsg.cpu().numpy())
        del k, v
        caches.append(cache)
        qs.append(synth.query(w, l, device=dev))
        lens_l.append(lens_t)
        pos_l.append((lens_t - 1).clamp(min=0).to(torch.int32))
        if l % 10 == 9 or l == L - 1:
            torch.cuda.synchronize()
            log(f"bench: built {l + 1}/{L} caches ({time.time() - t_setup:.1f}s)")
    max_len = int(max(int(x.max()) for x in lens_l))
    plan = caches[0].plan(w.Hq, max_len, chunk=args.chunk if primary else 0,
                          splits=args.splits if primary else 0)
    ws = caches[0].workspace(w.Hq, max_len, plan)
    outs = [torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev) for _ in range(L)]
    torch.cuda.synchronize()
    cache_bytes = sum(c.nbytes for c in caches)
    log(f"bench: setup {time.time() - t_setup:.1f}s, cache {cache_bytes / 2**30:.2f} GiB, "
        f"plan chunk={plan.chunk} splits={plan.num_splits} variant={plan.variant}")

    def append(l):  # the separate append kernel (timed for reference; the 4-bit step fuses it)
        otq.otq_quantize_append(k_new[l][:, :, None], v_new[l][:, :, None], caches[l].desc, pos_l[l])

    def split(l):
        otq.otq_sdpa_int4_split(qs[l], caches[l].desc, lens_l[l], max_len, w.scale, ws, plan)

    def combine(l):
        otq.otq_sdpa_lse_combine(w.Hq, caches[l].desc, lens_l[l], max_len, ws, plan, outs[l])

    def fused(l):  # split over the cached tokens, then the combine that appends the new token
        otq.otq_sdpa_int4_decode_append(qs[l], k_new[l], v_new[l], caches[l].desc, lens_l[l],
                                        max_len, w.scale, outs[l], ws, plan=plan)

    def step():
        for l in range(L):
            fused(l)

    # ---------------------------------------------------------------- timed steps
    graph = None
    if not args.no_graph:
        step()  # warm the launch path once before capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
    run = graph.replay if graph is not None else step
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    us_layer_step = ms_per_step * 1000.0 / L
    log(f"bench: {args.steps} steps, {ms_per_step:.3f} ms/step (events), {wall * 1e3 / args.steps:.3f} "
        f"ms/step (wall), {us_layer_step:.2f} us/layer-step")

    # ---------------------------------------------------------------- per-kernel durations
    def kernel_avg_us(fn, passes=3):
        """Eager fallback: HIP events around every launch."""
        evs = []
        for _ in range(passes):
            for l in range(L):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn(l)
                b.record()
                evs.append((a, b))
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1000.0

    def graph_avg_us(fn):
        """Average duration of one launch of fn, timed with HIP events over
        replays of a graph holding one launch per layer (back to back, as in
        the step; the same stream as the kernels)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for l in range(L):
                fn(l)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1000.0 / (args.steps * L)

    timer = kernel_avg_us if graph is None else graph_avg_us
    split_us = timer(split)
    combine_us = timer(combine) if primary else None
    append_us = timer(append) if primary else None
    torch.cuda.synchronize()
    sdpa_graph_us = None
    if graph is not None and primary:
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2):
            for l in range(L):
                split(l)
                combine(l)
        for _ in range(2):
            g2.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            g2.replay()
        b.record()
        torch.cuda.synchronize()
        sdpa_graph_us = a.elapsed_time(b) * 1000.0 / (args.steps * L)
    log(f"bench: split {split_us:.2f} us, combine {combine_us} us, append (unfused kernel) {append_us} us, "
        f"sdpa (split+combine, graph) {sdpa_graph_us} us per layer")

    # algorithmic bytes: packed codes + fp32 scales of every attended token, q read; out write
    lens_sum = [int(x.long().sum()) for x in lens_l]
    unit = w.Hkv * 2 * (w.D * wbits // 8 + 4 * (w.D // 32))     # bytes per attended token (K+V)
    split_bytes = float(np.mean([s * unit for s in lens_sum])) + w.B * w.Hq * w.D * 2
    layer_bytes = split_bytes + w.B * w.Hq * w.D * 4
    achieved = split_bytes / (split_us * 1e-6) / 1e9
    step_gbps = layer_bytes / (us_layer_step * 1e-6) / 1e9
    if wbits != 4:
        kname = "split_bits_mfma" if plan.variant == 2 else "split_bits"
    else:
        kname = "split_mfma" if plan.variant == 2 else "split_vec"
    if not primary:
        del caches, outs, ws, qs, k_new, v_new
        torch.cuda.empty_cache()
        rec = {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D,
               "context": w.T, "layers": L, "code_bits": wbits, "chunk": plan.chunk,
               "num_splits": plan.num_splits, "kernel": kname,
               "us_layer_step": round(us_layer_step, 3), "split_us": round(split_us, 3),
               "split_GBps": round(achieved, 1), "split_frac": round(achieved / HBM_PEAK_GBPS, 4),
               "step_GBps": round(step_gbps, 1), "step_frac": round(step_gbps / HBM_PEAK_GBPS, 4),
               "algorithmic_bytes_per_split_launch": int(split_bytes)}
        if not args.no_ceiling:  # the streaming rate at this workload's bytes per launch
            c = stream_ceiling(torch, otq, dev, int(split_bytes), min(L, 16), max(4, args.steps // 2))
            rec.update({"stream_ceiling_GBps": c["GBps"], "stream_ceiling_blocks": c["blocks"],
                        "split_frac_of_ceiling": round(achieved / c["GBps"], 4),
                        "step_frac_of_ceiling": round(step_gbps / c["GBps"], 4)})
        return rec

    # ---------------------------------------------------------------- bulk append (cache build)
    # Chunks of the workload's K/V quantised into a scratch cache of the same
    # shape, each chunk a distinct input, so that a pass over them (inputs and
    # outputs) is larger than the last-level cache and the rate is HBM's.
    n_bulk = min(16384, w.capacity)
    n_chunks = max(1, min(8, w.capacity // n_bulk))
    bulk_in = [(synth.kv(w, i, "k", T=n_bulk, device=dev), synth.kv(w, i, "v", T=n_bulk, device=dev))
               for i in range(n_chunks)]
    scratch = otq.Int4KVCache(w.B, w.Hkv, w.D, w.capacity, device=dev, rot_signs=caches[0].rot_signs,
                              chan_scale=caches[0].chan_scale, v_rot_signs=caches[0].v_rot_signs,
                              rot_kind=rot_kind, code_bits=wbits)
    bulk_pos = [torch.full((w.B,), i * n_bulk, dtype=torch.int32, device=dev) for i in range(n_chunks)]

    def bulk_pass():
        for i in range(n_chunks):
            scratch.append(bulk_in[i][0], bulk_in[i][1], bulk_pos[i])

    bulk_pass()
    torch.cuda.synchronize()
    reps = 5
    if graph is not None:
        gb = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gb):
            bulk_pass()
        gb.replay()
    bulk_run = gb.replay if graph is not None else bulk_pass
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        bulk_run()
    b.record()
    torch.cuda.synchronize()
    bulk_us = a.elapsed_time(b) * 1000.0 / (reps * n_chunks)
    bulk_bytes = w.B * w.Hkv * n_bulk * (2 * w.D * 2 + 2 * (w.D * wbits // 8 + 4 * (w.D // 32)))
    log(f"bench: bulk append of {n_bulk} tokens x {w.B * w.Hkv} heads: {bulk_us:.2f} us, "
        f"{bulk_bytes / (bulk_us * 1e-6) / 1e9:.0f} GB/s")
    del bulk_in, scratch
    if graph is not None:
        del gb
    torch.cuda.empty_cache()

    ceiling = None
    if not args.no_ceiling:
        ceiling = stream_ceiling(torch, otq, dev, int(split_bytes), min(L, 16), max(4, args.steps // 2))
        ceiling["split_frac_of_ceiling"] = round(achieved / ceiling["GBps"], 4)
        ceiling["step_frac_of_ceiling"] = round(step_gbps / ceiling["GBps"], 4)

    traffic = traffic_from_profile(kname, w.name, wbits)

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    check = None
    if host_kv0 is not None:
        import oracle
        try:
            share = len(os.sched_getaffinity(0))
        except AttributeError:
            share = os.cpu_count() or 1
        threads = args.cpu_threads or min(16, share)
        q0 = synth.bits(qs[0])
        rot_norm = caches[0].rot_norm
        t = time.time()
        qc = oracle_cache(oracle, w, host_kv0, rot_norm, rot_kind, wbits, threads)
        log(f"bench: oracle quantised layer 0 in {time.time() - t:.1f}s on {threads} threads")
        tok = int(np.asarray(synth.lens(w, 0), dtype=np.int64).sum())
        legs = []
        ref = None
        for nt, budget, max_reps in ((1, 10.0, 50), (threads, 10.0, 200)):
            ref_n, sdpa_s, nrep = oracle_leg(oracle, w, host_kv0, qc, q0, rot_norm, rot_kind, wbits,
                                             nt, budget, max_reps)
            ref = ref_n if ref is None else ref
            log(f"bench: oracle on {nt} thread(s): layer-step {sdpa_s:.3f}s ({nrep} runs)")
            legs.append({"threads": nt, "us_layer_step": round(sdpa_s * 1e6, 1), "runs": nrep})
        got = outs[0].cpu().numpy().astype(np.float64)
        err = got - ref
        check = {"layer": 0, "rows": int(w.B * w.Hq), "max_abs": float(np.abs(err).max()),
                 "rel_l2": float(np.linalg.norm(err) / np.linalg.norm(ref)),
                 "codes_note": "outputs of the last timed step vs the fp64 oracle"}
        multi = legs[1]
        cpu = {"value": multi["us_layer_step"], "unit": "us/layer-step", "cores": multi["threads"],
               "kind": "oracle",
               "sample": f"one full layer-step of layer 0 (all {w.B * w.Hq} query rows, {tok} cached "
                         f"tokens per KV head), fp64 attention in plain C over the oracle's quantised "
                         f"cache, timed {multi['runs']} times; mean per layer-step",
               "single_thread_us_layer_step": legs[0]["us_layer_step"],
               "legs": legs, "host_cpu_count": os.cpu_count(), "host_cpu_share": share}
        log(f"bench: GPU vs oracle max_abs={check['max_abs']:.2e} rel_l2={check['rel_l2']:.2e}")

    codes = "int4 codes" if wbits == 4 else f"{wbits}-bit codes"
    dtype = (f"f16 mfma operands, f32 accumulate ({codes}, f32 scales)" if plan.variant == 2
             else f"f32 vector arithmetic ({codes}, f32 scales)")
    step_desc = (f"per layer: the split pass over the cached tokens, then the combine pass that quantises "
                 f"the new token into the cache ({codes}) and merges it (otq_sdpa_int4_decode_append)")
    return {
        "metric": METRIC,
        "value": round(us_layer_step, 3),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
            "head_dim": w.D, "context": w.T, "layers": L, "input_dtype": w.dtype,
            "cache_gib": round(cache_bytes / 2**30, 3), "chunk": plan.chunk,
            "num_splits": plan.num_splits, "variant": "mfma" if plan.variant == 2 else "vector",
            "graph": graph is not None, "k_chan_scale": bool(chan),
            "v_rotated": bool(vrot),
            "k_rotation": ("none" if not (w.rotate or extra_rot) else rot_kind),
            "code_bits": wbits,
            "step": step_desc,
        },
        "kernels_us": {
            "split": round(split_us, 3),
            # after a split the partials come from the memory side, not from
            # a warm L2 as in a graph of combines alone: time it in place
            "combine_after_split": None if sdpa_graph_us is None else round(sdpa_graph_us - split_us, 3),
            "append_combine_after_split": round(us_layer_step - split_us, 3),
            "combine_back_to_back": round(combine_us, 3),
            "append_unfused_kernel": round(append_us, 3),
            "sdpa_per_layer_graph": None if sdpa_graph_us is None else round(sdpa_graph_us, 3)},
        "sdpa_GBps": round(layer_bytes / ((sdpa_graph_us or (split_us + combine_us)) * 1e-6) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": kname,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(split_bytes),
                     "note": "achieved = algorithmic bytes of one split launch / its mean duration"},
        "step_roofline": {"achieved": round(step_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": round(step_gbps / HBM_PEAK_GBPS, 4),
                          "algorithmic_bytes_per_layer_step": int(layer_bytes),
                          "note": "whole layer-step (split + combine + append) over µs per layer-step"},
        "stream_ceiling": ceiling,
        "append_bulk": {"kernel": "quantize_tile" if wbits == 4 else "quantize_bits", "tokens_per_sequence": n_bulk,
                        "sequences": w.B, "kv_heads": w.Hkv, "us": round(bulk_us, 3),
                        "algorithmic_bytes": int(bulk_bytes),
                        "GBps": round(bulk_bytes / (bulk_us * 1e-6) / 1e9, 1),
                        "frac": round(bulk_bytes / (bulk_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)},
        "cpu_baseline": cpu,
        "check": check,
    }


if __name__ == "__main__":
    main()
