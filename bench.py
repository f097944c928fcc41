#!/usr/bin/env python3
"""Benchmark: exact top-k -> top-p sampling on one MI355X.

One step = one call of topk_topp_sample over the whole heterogeneous batch
(B=256 rows, V=151,936 fp32 probabilities; 64 greedy rows, 64 top-p-only rows,
128 rows with k in [20, 1024]), tokens only (renorm_out = NULL), inputs
already resident in HBM.  Timed steps rotate over several copies of the
input so that the 256 MiB Infinity Cache cannot serve a repeated read, and
advance the Philox offset by one per call.

Prints one JSON line: rows/s for the whole job, the kernel's achieved HBM
bandwidth against the 8 TB/s peak (algorithmic bytes = B*V*4 + 12*B per
launch divided by the kernel's average duration: one pair of HIP events on the
launch stream brackets the timed region, which holds exactly one kernel launch
per step), and the CPU oracle timed on the host cores as a baseline.

Before the timed region the script replays the same calls from a captured HIP
graph and times the library's plain read of the same bytes (both reported in
the line); after it, it repeats the timed loop for a median and checks the
tokens of one call against the oracle.
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

PEAK_HBM_GBPS = 8000.0
METRIC = "rows/s and achieved HBM GB/s (% of peak) at B=256, V=151,936 top-k+top-p"
KERNEL_SRC = os.path.join(ROOT, "top_exact_sampling_amd", "csrc", "tes_sampler.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tes_main_kernel_hetero_b256_v151936_traffic.txt")


ROW_MIX = {
    1: "k=50, p=0.9 on all rows",
    2: "k~U{1..1024}, p~U[0.5,1.0]",
    3: "64 greedy (k=1), 64 top-p only (k=V, p~U[0.8,0.99]), "
       "128 k~U{20..1024} with p~U[0.7,1.0]",
    4: "k~U{1..1024}, p~U[0.5,1.0]; 10 all-zero rows, 10 NaN/negative/-0.0 rows, "
       "10 rows with 2-5 +inf",
    5: "top-p only: k=V, p=0.95",
}
INPUT = {
    1: "fp32 probs, softmax of 2*N(0,1) logits with 3 tokens boosted +10",
    2: "fp32 probs, softmax of 2*N(0,1) logits with 1-8 tokens boosted U[8,15]",
    3: "fp32 probs, softmax of 2*N(0,1) logits with 1-8 tokens boosted U[8,15]",
    4: "fp32 probs of the same recipe quantised to multiples of 2^-20 and renormalised",
    5: "fp32 probs, softmax of 0.5*N(0,1) logits (high entropy)",
}


def source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    t = {}
    try:
        with open(TRAFFIC_FILE) as f:
            for ln in f:
                if ":" in ln and not ln.startswith((" ", "#")):
                    k, v = ln.split(":", 1)
                    t[k.strip()] = v.strip()
    except OSError:
        return None
    if t.get("kernel_source_sha256_16") != source_hash():
        return None
    try:
        return int(t["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name, B, call, min_wall=10.0, max_reps=40, single_wall=3.0):
    """The oracle as it stands, on every host core this process may use (rows
    split statically across threads), plus a one-thread figure on a bounded
    prefix of the same batch.  call(lo, hi, n_threads, offset) runs the
    oracle on rows (or requests) [lo, hi)."""
    cores = len(os.sched_getaffinity(0))
    reps, t0 = 0, time.perf_counter()
    while True:
        call(0, B, cores, reps)
        reps += 1
        wall = time.perf_counter() - t0
        if wall >= min_wall or reps >= max_reps:
            break
    # One thread: rows in batch order until ~single_wall seconds have passed.
    rows1, t1 = 0, time.perf_counter()
    while rows1 < B:
        n = min(8, B - rows1)
        call(rows1, rows1 + n, 1, 0)
        rows1 += n
        if time.perf_counter() - t1 >= single_wall:
            break
    wall1 = time.perf_counter() - t1
    return {
        "value": round(reps * B / wall, 1),
        "unit": "rows/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d full passes over all %d rows of %s (stable sort per row, %d host threads, "
                  "%.1f s)" % (reps, B, name, cores, wall),
        "cpu_model": cpu_model(),
        "single_thread_rows_per_s": round(rows1 / wall1, 1),
        "single_thread_sample": "first %d rows of the batch on one thread (%.1f s)" % (rows1, wall1),
    }


def graph_timing(step, copies, stream, calls=20, replays=50):
    """Average duration of one call when `calls` calls (rotating over the
    input copies) are captured in one HIP graph and replayed."""
    import torch

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        step(0, side)  # the library's first use of this stream, outside capture
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream()
        for i in range(calls):
            step(i, cap)
    g.replay()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()  # replays run on the current stream
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for _ in range(replays):
        g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * calls)


def read_timing(tes, probs, nbytes, dev, stream, steps):
    """Average duration of a plain read of one input copy (reference stream
    kernel of the library), rotating over the copies like the timed calls."""
    import torch

    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def rd(i):
        rc = tes.sampler_read_probe(probs[i % len(probs)].data_ptr(), nbytes, sink.data_ptr(),
                                    dev.index or 0, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError("sampler_read_probe failed: %d" % rc)

    for i in range(10):
        rd(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        rd(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Defaults: ~20 ms of warm-up (the GPU reaches its steady clocks; 20 calls
    # measured ~1.5 us per call slower) and ~40 ms timed.
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--copies", type=int, default=4, help="rotating input copies (> MALL)")
    ap.add_argument("--workload", type=int, default=None, choices=[1, 2, 3, 4, 5],
                    help="input recipe (workloads.py); 3, the heterogeneous B=256, V=151,936 "
                         "batch, is the headline (5 for --mode spec)")
    ap.add_argument("--mode", choices=["probs", "logits", "spec"], default="probs",
                    help="probs: topk_topp_sample (the headline); logits: "
                         "topk_topp_sample_logits on the recipe's logits with per-row "
                         "temperature and min-p; spec: spec_verify_sample, requests of 7 drafts "
                         "and 8 target rows over the recipe's rows")
    ap.add_argument("--input-dtype", choices=["fp32", "bf16"], default="fp32",
                    help="row format: fp32 (the headline) or bf16 (topk_topp_sample_bf16, "
                         "the same rows rounded to bf16)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-parity", action="store_true", help="skip the oracle check")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one device copy of this size (counter calibration)")
    ap.add_argument("--renorm", action="store_true",
                    help="also write renorm_out (dense [B][V] fp32) in every timed call")
    ap.add_argument("--slab", type=int, default=0, metavar="CAP",
                    help="--mode probs: call topk_topp_sample_slab instead, exporting each "
                         "row's sorted support (rows with k_eff <= CAP, 1..1024) in every "
                         "timed call")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed repetitions of --steps calls; the first is the timed region of "
                         "the line, the median over all is reported beside it")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this sampler has no multi-GPU path "
              "(rows are independent; see the sharding note in the design document). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import top_exact_sampling_amd as tes
    import workloads

    if args.workload is None:
        args.workload = 5 if args.mode == "spec" else 3
    import oracle

    bf16 = args.input_dtype == "bf16"
    if bf16 and args.mode != "probs":
        raise SystemExit("--input-dtype bf16 applies to --mode probs only")
    if args.slab and (args.mode != "probs" or bf16 or not 1 <= args.slab <= 1024):
        raise SystemExit("--slab CAP (1..1024) applies to --mode probs with fp32 rows only")
    if args.mode == "spec":
        sw = workloads.make_spec(args.workload)
        w = workloads.make(args.workload)  # the target rows (same inputs)
        B = sw.target.shape[0]
        w.probs, w.top_k, w.top_p = sw.target, sw.top_k, sw.top_p
    elif args.mode == "logits":
        w = workloads.make_logits(args.workload)
    else:
        w = workloads.make(args.workload)
    B, V = w.B, w.V
    if bf16:
        # The same rows rounded to bf16; the oracle reads their exact fp32
        # widening, which is what a bf16 entry means to the sampler.
        t16 = torch.from_numpy(w.probs).to(torch.bfloat16)
        w.probs = (t16.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16) \
            .view(np.float32)
    esize = 2 if bf16 else 4
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sampler = tes.Sampler(0, max_batch=B, max_vocab=V)
    # Rotating copies: at least twice the 256 MiB Infinity Cache in total
    # (fewer for the large batches, whose single copy already exceeds it).
    copies = max(1, min(args.copies, -(-2 * (256 << 20) // (B * V * esize))))
    args.copies = copies
    if bf16:
        probs = [t16.to(dev) for _ in range(copies)]
    else:
        probs = [torch.from_numpy(w.probs).to(dev) for _ in range(copies)]
    top_k = torch.from_numpy(w.top_k).to(dev)
    top_p = torch.from_numpy(w.top_p).to(dev)
    out = torch.empty(B, dtype=torch.int32, device=dev)
    ren = torch.empty((B, V), dtype=torch.float32, device=dev) if args.renorm else None
    stream = torch.cuda.current_stream(dev)
    orc = oracle.load()

    # Call i draws with Philox offset w.offset + i, as a decode loop advances
    # it, so that draw-dependent paths are sampled rather than one fixed draw.
    if args.mode == "probs" and args.slab:
        s_idx = torch.empty((B, args.slab), dtype=torch.int32, device=dev)
        s_ren = torch.empty((B, args.slab), dtype=torch.float32, device=dev)
        s_len = torch.empty(B, dtype=torch.int32, device=dev)
        s_route = torch.empty(B, dtype=torch.int32, device=dev)

        def step(i, st=None):
            rc = tes.topk_topp_sample_slab(
                sampler.handle, probs[i % args.copies].data_ptr(), B, V, top_k.data_ptr(),
                top_p.data_ptr(), w.seed, w.offset + i, out.data_ptr(),
                ren.data_ptr() if ren is not None else None, s_idx.data_ptr(), s_ren.data_ptr(),
                args.slab, s_len.data_ptr(), s_route.data_ptr(),
                (stream if st is None else st).cuda_stream)
            if rc != 0:
                raise RuntimeError("topk_topp_sample_slab failed: %d" % rc)

        def oracle_call(lo, hi, nt, off):
            return orc.sample(w.probs[lo:hi], w.top_k[lo:hi], w.top_p[lo:hi], w.seed,
                              w.offset + off, n_threads=nt)[0]
    elif args.mode == "probs":
        def step(i, st=None):
            sampler.sample(probs[i % args.copies], top_k, top_p, w.seed, w.offset + i,
                           out_tokens=out, renorm_out=ren, stream=stream if st is None else st)

        def oracle_call(lo, hi, nt, off):
            return orc.sample(w.probs[lo:hi], w.top_k[lo:hi], w.top_p[lo:hi], w.seed,
                              w.offset + off, n_threads=nt)[0]
    elif args.mode == "logits":
        tau = torch.from_numpy(w.temperature).to(dev)
        mp = torch.from_numpy(w.min_p).to(dev)

        def step(i, st=None):
            sampler.sample_logits(probs[i % args.copies], top_k, top_p, w.seed, w.offset + i,
                                  temperature=tau, min_p=mp, out_tokens=out, renorm_out=ren,
                                  stream=stream if st is None else st)

        def oracle_call(lo, hi, nt, off):
            return orc.sample_logits(w.probs[lo:hi], w.top_k[lo:hi], w.top_p[lo:hi],
                                     w.temperature[lo:hi], w.min_p[lo:hi], w.seed,
                                     w.offset + off, n_threads=nt)[0]
    else:
        if args.renorm:
            raise SystemExit("--renorm does not apply to --mode spec")
        Lt = sw.Lt
        N = B // Lt
        L = sw.draft_tokens.shape[1]
        draft = torch.from_numpy(sw.draft).to(dev)
        dtok = torch.from_numpy(sw.draft_tokens).to(dev)
        sout = torch.empty((N, L + 1), dtype=torch.int32, device=dev)
        sacc = torch.empty(N, dtype=torch.int32, device=dev)

        def step(i, st=None):
            rc = tes.spec_verify_sample(sampler.handle, probs[i % args.copies].data_ptr(), N, Lt,
                                        V, top_k.data_ptr(), top_p.data_ptr(), draft.data_ptr(),
                                        L, dtok.data_ptr(), None, w.seed, w.offset + i,
                                        sout.data_ptr(), sacc.data_ptr(),
                                        (stream if st is None else st).cuda_stream)
            if rc != 0:
                raise RuntimeError("spec_verify_sample failed: %d" % rc)

        def oracle_call(lo, hi, nt, off):
            r0, r1 = lo // Lt * Lt, -(-hi // Lt) * Lt
            n0, n1 = r0 // Lt, r1 // Lt
            return orc.spec_verify(sw.target[r0:r1], Lt, sw.top_k[r0:r1], sw.top_p[r0:r1],
                                   sw.draft[n0 * L:n1 * L], sw.draft_tokens[n0:n1], None, w.seed,
                                   w.offset + off, n_threads=nt)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # Two reference measurements come first: the same calls replayed from one
    # captured HIP graph (launch overhead removed), and a plain read of the
    # same bytes by the library's reference stream kernel, on the same stream
    # and input copies.  (Run before the timed region, they also bring the GPU
    # to the clocks it keeps in a decode loop.)
    graph_ms = graph_timing(step, args.copies, stream)
    read_ms = read_timing(tes, probs, B * V * esize, dev, stream, max(args.steps, 200))

    # Timed region: exactly `steps` calls, back to back on the launch stream,
    # bracketed by one pair of HIP events on that stream (each call is one
    # sampler launch, plus one each for renorm_out and the slab export, so
    # the events give the call's average duration).  Further repetitions of the same loop follow; their
    # median is reported beside the first.
    def timed_loop(first):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(args.steps):
            step(first + i)
        ev1.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, ev0.elapsed_time(ev1) / args.steps

    wall, kern_ms = timed_loop(0)
    ms_per_step = wall * 1e3 / args.steps
    reps_ms = [kern_ms] + [timed_loop(args.steps * (j + 1))[1]
                           for j in range(max(0, args.repeats - 1))]
    kern_med = sorted(reps_ms)[len(reps_ms) // 2]

    # Algorithmic bytes: the rows once, top_k, top_p and the token (and the
    # temperature and min-p of logit rows), plus the dense renorm_out write
    # when requested.  Speculative verification: the target rows once, the
    # drafts' 4-byte lookups, and for each request with a rejection its
    # draft row and target row once more (the correction's residual); the
    # rejections are counted on the call checked below.
    per_row = {"probs": 12, "logits": 20, "spec": 12}[args.mode]
    alg_bytes = B * V * esize + per_row * B + (B * V * 4 if args.renorm else 0)
    # The slab export writes an index and a weight per slot, a length and a route per row.
    alg_bytes += B * (args.slab * 8 + 8) if args.slab else 0
    parity = None
    step(0)
    torch.cuda.synchronize()
    if args.mode == "spec":
        oout, oacc = oracle_call(0, B, len(os.sched_getaffinity(0)), 0)
        rejected = int((oacc < L).sum())
        alg_bytes += N * L * 12 + rejected * 2 * V * 4
        if not args.no_parity:
            same = np.array_equal(sout.cpu().numpy(), oout) and np.array_equal(sacc.cpu().numpy(),
                                                                               oacc)
            parity = "bit-exact" if same else "MISMATCH"
    elif not args.no_parity:
        otok = oracle_call(0, B, len(os.sched_getaffinity(0)), 0)
        gtok = out.cpu().numpy()
        parity = "bit-exact" if np.array_equal(gtok, otok) else \
            "MISMATCH on %d rows" % int((gtok != otok).sum())
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9

    traffic = traffic_from_profile() if (args.workload == 3 and not bf16 and not args.renorm
                                         and args.mode == "probs" and not args.slab) else None
    line = {
        "metric": METRIC,
        "value": round(B / (ms_per_step * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.input_dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "B": B,
            "V": V,
            "mode": args.mode,
            "row_mix": ROW_MIX[args.workload] + (
                "; temperature ~U[0.5,1.5] (5% 0, 5% 1), min_p 0 on half the rows else "
                "~U[0.005,0.3]" if args.mode == "logits" else "") + (
                "; %d requests of %d drafts, %d target rows each, draft rows "
                "softmax(log p + 0.5 N(0,1))" % (B // sw.Lt, sw.Lt - 1, sw.Lt)
                if args.mode == "spec" else ""),
            "input": (INPUT[args.workload] + (", rounded to bf16" if bf16 else "")) if
            args.mode != "logits" else "fp32 logits of the same recipe, before the softmax",
            "input_dtype": args.input_dtype,
            "renorm_out": "dense [B][V] fp32" if args.renorm else None,
            "slab_export_cap": args.slab or None,
            "arithmetic": "u32 keys, u64 fixed-point masses, u128 products (integer decisions)",
            "input_sha256": workloads.sha256_of(w) if args.mode != "spec" else
            workloads.sha256_of(w) + "+draft",
            "input_copies_rotated": args.copies,
            "kernel_ms_hip_events": round(kern_ms, 5),
            "kernel_ms_repeats": [round(x, 5) for x in reps_ms],
            "kernel_ms_median": round(kern_med, 5),
            "kernel_ms_graph_replay": round(graph_ms, 5),
            "plain_read_ms_same_bytes": round(read_ms, 5),
            "plain_read_GBps": round(B * V * esize / (read_ms * 1e-3) / 1e9, 1),
            "frac_of_plain_read": round(read_ms / kern_ms, 4),
            "parity_vs_oracle": parity,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "traffic_source": ("rocprofv3 FETCH_SIZE + WRITE_SIZE summary committed under "
                               "profiles/ for this kernel source hash") if traffic else None,
        },
        "cpu_baseline": None if args.no_cpu else cpu_baseline(w.name, B, oracle_call),
    }
    sampler.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
