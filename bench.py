#!/usr/bin/env python3
"""Benchmark of the Q4 linear layer on one MI355X.

Workload: the Qwen2.5-7B-shaped projection set (q 3584x3584, k and v
512x3584, gate and up 18944x3584, down 3584x18944), Q4 weights (blocks of 32,
fp16 scales), bf16 activations, at every decode row count M = 1..8.  One
step = the six projections at each M = 1..8 (48 calls through the library's
crossover dispatcher), each M on its own weight copy taken from a rotation
pool larger than the 256 MB Infinity Cache, so weights stream from HBM (no
copy is read twice within 1.5 GiB of weight traffic).  Inputs are seeded
synthetic data of those shapes (no trained weights); every input is resident
in HBM before the timed region.

Printed JSON line: value = achieved algorithmic HBM GB/s over the whole step
(codes + scales + activations + outputs per call, divided by step time),
with the dominant kernel's roofline and the fp64 CPU oracle timed on the
host as a baseline.  The GEMV->GEMM crossover (on the layer set and per
matrix) and the per-M bandwidth are reported under "detail".

Timing: each step's 48 launches are captured once in a HIP graph (one graph
per offset into the pool); the timed region replays them between two events on the
launch stream, after a barrier-free torch.cuda.synchronize() on both sides.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, 8 TB/s


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "q4_gemv_7b_layer_set_m1-8_traffic.md")
KERNEL_SOURCES = ("bit_quantized_matmul_q4_amd/csrc/q4_kernels.hip", "bit_quantized_matmul_q4_amd/csrc/q4_device.hpp",
                  "bit_quantized_matmul_q4_amd/csrc/q4_plan.hpp", "bit_quantized_matmul_q4_amd/build.py")


def measured_traffic():
    """HBM bytes per launch from the committed byte-counter summary, or None
    when it is missing or was taken on other kernel sources."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and not line.startswith("|"))
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("kernel_source_sha256", "").strip() != h.hexdigest():
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def log(msg: str) -> None:
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--pool-gib", type=float, default=1.5, help="rotation pool of weight copies (GiB)")
    ap.add_argument("--no-crossover", action="store_true", help="skip the GEMV/GEMM crossover sweep")
    ap.add_argument("--no-stream", action="store_true", help="skip the 28-layer decode weight stream")
    ap.add_argument("--no-fused", action="store_true", help="skip the fused-launch step")
    ap.add_argument("--no-schemes", action="store_true", help="skip the pages' switching schemes comparison")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the 0.5B-shaped layer set and the single 896 x 896 matvec")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-per-launch", action="store_true",
                    help="skip the per-matrix launch timings (per-M and per-matrix GB/s)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget for the CPU oracle sample")
    ap.add_argument("--kernel", default="auto", choices=["auto", "gemv", "gemm"])
    ap.add_argument("--detail-json", default=None, help="also write the full results here")
    ap.add_argument("--eager-step", action="store_true",
                    help="run one step's launches eagerly (no graphs) and exit: for hardware-counter passes")
    ap.add_argument("--eager-m", default=None, metavar="M,M,...",
                    help="row counts of the eager step (default 1..8), e.g. 124 with --kernel gemm")
    ap.add_argument("--eager-reps", type=int, default=1, help="repeat the eager step (weights from the pool)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run 8 plain device copies of MIB MiB each and exit: calibrates byte counters")
    return ap.parse_args()


def main() -> int:
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import bit_quantized_matmul_q4_amd as q4
    import synth
    from bit_quantized_matmul_q4_amd import build as hip_build

    if args.copy_calibration:
        dev = torch.device("cuda:0")
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 8 copies of %d bytes (each reads and writes %d bytes)" % (n, n))
        return 0

    if not os.path.exists(hip_build.LIB):
        hip_build.build_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mats = synth.SET_7B
    Ms = list(range(1, 9))
    set_bytes = sum(sum(q4.packed_sizes(m.N, m.K)) for m in mats)
    P = max(2, int(np.ceil(args.pool_gib * (1 << 30) / set_bytes)))
    log("device %s, rotation pool %d copies of the layer set (%.2f GiB)"
        % (torch.cuda.get_device_name(dev), P, P * set_bytes / (1 << 30)))

    # ---- inputs, resident in HBM: weights drawn directly in the packed form.
    # Each copy of the set is held as the fused buffers (q|k|v, gate|up,
    # down); the six projections are views into them.
    base = []
    for mi, m in enumerate(mats):
        wq_t, sc_t = synth.packed_weight(m.N, m.K, 3, mi)
        base.append(q4.Q4Weight(torch.from_numpy(wq_t).to(dev),
                                torch.from_numpy(sc_t.view(np.int16)).to(dev).view(torch.float16), m.N, m.K))
    fuse_groups = ((0, 1, 2), (3, 4), (5,))  # q|k|v, gate|up, down

    def fused_copy():
        fused = [q4.concat_n([base[i] for i in grp]) for grp in fuse_groups]
        views = []
        for f, grp in zip(fused, fuse_groups):
            views += q4.split_n(f, [mats[i].N for i in grp])
        return fused, views

    fpool, pool = [], []
    for _ in range(P):
        f, v = fused_copy()
        fpool.append(f)
        pool.append(v)
    fmats = [(sum(mats[i].N for i in grp), mats[grp[0]].K) for grp in fuse_groups]
    Mmax = 128
    xs = {}
    for K in sorted({m.K for m in mats}):
        xb = synth.activations(Mmax, K, "bf16", 3, 100 + K)
        xs[K] = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    ys = {(mi, M): torch.empty((M, m.N), dtype=torch.float32, device=dev)
          for mi, m in enumerate(mats) for M in range(1, Mmax + 1)
          if M <= 20 or M in (24, 28, 32, 33, 36, 40, 44, 48, 64, 85, 96, 124, 128)}
    torch.cuda.synchronize()

    yf = {(j, M): torch.empty((M, fmats[j][0]), dtype=torch.float32, device=dev)
          for j in range(len(fmats)) for M in (1, 2, 3, 4, 5, 6, 7, 8, 16, 64)}

    def call(mi, M, p, kernel):
        q4.linear(xs[mats[mi].K][:M], pool[p][mi], out=ys[(mi, M)], kernel=kernel)

    def call_fused(j, M, w):
        q4.linear(xs[fmats[j][1]][:M], w, out=yf[(j, M)])

    def capture(fn):
        # warm the launch path (and any workspace) once outside capture
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    def time_graphs(graphs, reps):
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(reps):
            graphs[i % len(graphs)].replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps  # ms

    def step_bytes(M_list):
        return sum(synth.algorithmic_bytes(M, m.N, m.K) for M in M_list for m in mats)

    if args.eager_step:
        eMs = [int(v) for v in args.eager_m.split(",")] if args.eager_m else Ms
        for r in range(args.eager_reps):
            for M in eMs:
                for mi in range(len(mats)):
                    call(mi, M, r % P, args.kernel)
        torch.cuda.synchronize()
        flops = sum(2 * M * m.N * m.K for M in eMs for m in mats)
        log("eager step x %d: %d launches each, %d algorithmic bytes, %d useful flops per step"
            % (args.eager_reps, len(eMs) * len(mats), step_bytes(eMs), flops))
        return 0

    # ---- the step: 6 projections x M = 1..8, one graph per pool offset.
    # Row count j of step graph p reads copy (p * 8 + j) mod P: each M reads
    # a copy of its own, so no weight is reread out of the Infinity Cache
    # (one copy for all eight M would reread it seven times within 1 GB).
    def copy_of(p, j):
        return (p * len(Ms) + j) % P

    log("capturing %d step graphs" % P)
    step_graphs = [capture(lambda p=p: [call(mi, M, copy_of(p, j), args.kernel)
                                        for j, M in enumerate(Ms) for mi in range(len(mats))])
                   for p in range(P)]
    for i in range(args.warmup):
        step_graphs[i % P].replay()
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    ms_step = time_graphs(step_graphs, args.steps)
    bytes_step = step_bytes(Ms)
    value = bytes_step / (ms_step * 1e-3) / 1e9
    rows_per_s = sum(Ms) / (ms_step * 1e-3)
    log("step %.3f us, %.1f GB/s (%.1f%% of 8 TB/s)" % (ms_step * 1e3, value, 100 * value / PEAK_HBM_GBS))
    # roofline of the dominant kernel: every launch of the step runs the
    # matrix-vector kernel, so its average launch duration over the timed
    # region is the step time over the 48 launches (inter-launch gaps
    # inside the graph included)
    n_launch = len(Ms) * len(mats)
    launch_ms = ms_step / n_launch
    achieved = bytes_step / n_launch / (launch_ms * 1e-3) / 1e9

    # ---- per-launch durations of the dominant kernel and per-M bandwidth:
    # back-to-back launches of one shape, one graph, each launch on another
    # copy of the matrix.  The copies span at least the pool's size per
    # matrix (the step pool's copies plus clones), so that every launch
    # streams its weights from HBM: the step pool alone holds 14 copies of
    # q_proj (100 MB), which the Infinity Cache would keep.
    # The per-matrix crossover (M* of each projection alone) is taken on the
    # same pools, with each kernel forced.
    per_launch = {}
    per_m = per_matrix_m8 = per_launch_us = None
    xM = list(range(1, 21)) + [24, 28, 32, 48, 64, 96, 128]
    per_matrix_x = {}
    if not args.no_per_launch:
        pool_bytes = args.pool_gib * (1 << 30)
        for mi, m in enumerate(mats):
            wbytes = sum(q4.packed_sizes(m.N, m.K))
            extra = [q4.Q4Weight(base[mi].codes.clone(), base[mi].scales.clone(), m.N, m.K)
                     for _ in range(max(0, int(np.ceil(pool_bytes / wbytes)) - P))]
            mpool = [pool[p][mi] for p in range(P)] + extra
            for M in Ms:
                g = capture(lambda M=M, mi=mi, mpool=mpool: [q4.linear(xs[m.K][:M], w, out=ys[(mi, M)],
                                                                       kernel=args.kernel) for w in mpool])
                g.replay()  # untimed first replay
                # best of three: the first timing after the previous matrix's
                # clones were freed has been seen up to 5x slower, once
                per_launch[(mi, M)] = min(time_graphs([g], 1) for _ in range(3)) / len(mpool)  # ms per launch
                del g
            if not args.no_crossover:
                rows = []
                for M in xM:
                    t = {}
                    for kern in ("gemv", "gemm"):
                        g = capture(lambda M=M, mi=mi, mpool=mpool, kern=kern: [
                            q4.linear(xs[m.K][:M], w, out=ys[(mi, M)], kernel=kern) for w in mpool])
                        g.replay()
                        t[kern] = min(time_graphs([g], 1) for _ in range(2)) / len(mpool) * 1e3  # us
                        del g
                    rows.append([M, round(t["gemv"], 2), round(t["gemm"], 2)])
                mstar_m = None
                for r in reversed(rows):
                    if r[2] >= r[1]:
                        break
                    mstar_m = r[0]
                per_matrix_x[m.name] = {"M_star": mstar_m, "rows_M_gemv_us_gemm_us": rows}
                log("%s: matrix-matrix faster from M* = %s" % (m.name, mstar_m))
            del extra, mpool
            torch.cuda.empty_cache()
        per_m = {}
        for M in Ms:
            t = sum(per_launch[(mi, M)] for mi in range(len(mats)))
            per_m[str(M)] = round(step_bytes([M]) / (t * 1e-3) / 1e9, 1)
        per_matrix_m8 = {mats[mi].name: round(synth.algorithmic_bytes(8, mats[mi].N, mats[mi].K)
                                              / (per_launch[(mi, 8)] * 1e-3) / 1e9, 1) for mi in range(len(mats))}
        per_launch_us = {m.name: {str(M): round(per_launch[(mi, M)] * 1e3, 2) for M in Ms}
                         for mi, m in enumerate(mats)}
        log("per-M GB/s %s" % per_m)
        log("per-matrix GB/s at M=8 %s" % per_matrix_m8)

    # ---- the same step with fused launches: q|k|v (N = 4608) and gate|up
    # (N = 37888) as one call each, down on its own (24 calls); x is read
    # once per fused call, so the step's algorithmic bytes are a little lower
    fused_step = None
    if not args.no_fused:
        fgraphs = [capture(lambda p=p: [call_fused(j, M, fpool[copy_of(p, i)][j])
                                        for i, M in enumerate(Ms) for j in range(len(fmats))])
                   for p in range(P)]
        for i in range(args.warmup):
            fgraphs[i % P].replay()
        ms_fused = time_graphs(fgraphs, args.steps)
        fbytes = sum(synth.algorithmic_bytes(M, N, K) for M in Ms for (N, K) in fmats)
        fused_step = {"calls_per_step": len(Ms) * len(fmats), "us_per_step": round(ms_fused * 1e3, 2),
                      "gbs": round(fbytes / (ms_fused * 1e-3) / 1e9, 1),
                      "pct_of_peak": round(100 * fbytes / (ms_fused * 1e-3) / 1e9 / PEAK_HBM_GBS, 1),
                      "rows_per_s": round(sum(Ms) / (ms_fused * 1e-3), 1),
                      "matrices": ["q|k|v %dx%d" % fmats[0], "gate|up %dx%d" % fmats[1], "down %dx%d" % fmats[2]]}
        log("fused step %.2f us, %.1f GB/s" % (ms_fused * 1e3, fused_step["gbs"]))
        del fgraphs

    # ---- the whole 7B decode weight stream: 28 distinct copies of the layer
    # set plus the LM head, per M, as one graph (unfused and fused calls)
    stream = None
    if not args.no_stream:
        from synth import LM_HEAD_7B, N_LAYERS_7B
        layers = [fused_copy() for _ in range(N_LAYERS_7B)]
        wq_t, sc_t = synth.packed_weight(LM_HEAD_7B.N, LM_HEAD_7B.K, 5, 6)
        head = q4.Q4Weight(torch.from_numpy(wq_t).to(dev),
                           torch.from_numpy(sc_t.view(np.int16)).to(dev).view(torch.float16),
                           LM_HEAD_7B.N, LM_HEAD_7B.K)
        del wq_t, sc_t
        stream = {}
        for M in (1, 4, 16, 64):
            yh = torch.empty((M, LM_HEAD_7B.N), dtype=torch.float32, device=dev)

            def run(fused, M=M, yh=yh):
                for f, v in layers:
                    if fused:
                        for j in range(len(fmats)):
                            call_fused(j, M, f[j])
                    else:
                        for mi in range(len(mats)):
                            q4.linear(xs[mats[mi].K][:M], v[mi], out=ys[(mi, M)])
                q4.linear(xs[LM_HEAD_7B.K][:M], head, out=yh)
            nbytes = N_LAYERS_7B * step_bytes([M]) + synth.algorithmic_bytes(M, LM_HEAD_7B.N, LM_HEAD_7B.K)
            rec = {}
            for fused in (False, True):
                g = capture(lambda fused=fused: run(fused))
                ms = time_graphs([g], 5)
                del g
                rec["fused" if fused else "unfused"] = {
                    "us": round(ms * 1e3, 1), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                    "rows_per_s": round(M / (ms * 1e-3), 1)}
            stream[str(M)] = rec
            log("decode stream M=%d: %s" % (M, rec))
        del layers, head
        torch.cuda.empty_cache()

    # ---- the small workloads: the single 896 x 896 matvec at M = 1 and the
    # Qwen2.5-0.5B-shaped layer set at M = 1, 2, 4, fp16 activations; each
    # call on its own weight copy from a pool of about half the step pool's
    # size, so the weights stream from HBM
    small = None
    if not args.no_small:
        small = {}
        for wl in (1, 2):
            spec = synth.WORKLOADS[wl]
            smats = spec["matrices"]
            sbytes = sum(sum(q4.packed_sizes(m.N, m.K)) for m in smats)
            SP = max(2, int(np.ceil(args.pool_gib * (1 << 30) / 2 / sbytes)))
            sbase = []
            for mi, m in enumerate(smats):
                wq_t, sc_t = synth.packed_weight(m.N, m.K, wl, mi)
                sbase.append(q4.Q4Weight(torch.from_numpy(wq_t).to(dev),
                                         torch.from_numpy(sc_t.view(np.int16)).to(dev).view(torch.float16), m.N, m.K))
            spool = [[q4.Q4Weight(w.codes.clone(), w.scales.clone(), w.N, w.K) for w in sbase] for _ in range(SP)]
            Mx = max(spec["Ms"])
            sx = {}
            for K in sorted({m.K for m in smats}):
                xb = synth.activations(Mx, K, spec["x"], wl, 100 + K)
                sx[K] = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.float16)
            rec = {}
            for M in spec["Ms"]:
                ysm = [torch.empty((M, m.N), dtype=torch.float32, device=dev) for m in smats]
                g = capture(lambda M=M, ysm=ysm: [q4.linear(sx[m.K][:M], spool[p][mi], out=ysm[mi])
                                                  for p in range(SP) for mi, m in enumerate(smats)])
                g.replay()
                ms = min(time_graphs([g], 1) for _ in range(3)) / SP  # per pass over the set
                del g
                nb = sum(synth.algorithmic_bytes(M, m.N, m.K) for m in smats)
                rec[str(M)] = {"us": round(ms * 1e3, 2), "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
                               "rows_per_s": round(M / (ms * 1e-3), 1)}
            small[spec["name"]] = {"matrices": ["%s %dx%d" % (m.name, m.N, m.K) for m in smats],
                                   "x": spec["x"], "weight_copies": SP, "per_M": rec}
            log("%s: %s" % (spec["name"], rec))
            del spool, sbase, sx
            torch.cuda.empty_cache()

    # ---- the pages' kernel-switching schemes as comparators, on the layer
    # set at the pages' row counts: 1..5 (one row per request) and the
    # continuous-batching iterations 8, 19, 44, 85 tokens and the 124-row
    # mixed batch.  Schemes: this library's rule (M <= T: one multi-row
    # matrix-vector call, else matrix-matrix); one row -> matrix-vector, more
    # -> matrix-matrix; up to 4 rows -> one matrix-vector call per row
    # (written straight into its row of y), more -> matrix-matrix; every row
    # through the matrix-vector kernel.  All four must give the same bits.
    schemes = None
    if not args.no_schemes:
        T = q4.get_crossover()

        def scheme_calls(name, M, p):
            for mi, m in enumerate(mats):
                x, w, y = xs[m.K][:M], pool[p][mi], ys[(mi, M)]
                if name == "library" or name == "all_gemv":
                    kern = "gemv" if (name == "all_gemv" or M <= T) else "gemm"
                    q4.linear(x, w, out=y, kernel=kern)
                elif name == "one_row_gemv" or M > 4:
                    q4.linear(x, w, out=y, kernel="gemv" if M == 1 else "gemm")
                else:  # row by row
                    for r in range(M):
                        q4.linear(x[r:r + 1], w, out=y[r:r + 1], kernel="gemv")

        names = ("library", "one_row_gemv", "row_by_row_le4", "all_gemv")
        schemes = {"T": T, "rows": {}, "bits_identical": True}
        for M in (1, 2, 3, 4, 5, 8, 19, 44, 85, 124):
            rec, outs = {}, {}
            for name in names:
                g = capture(lambda name=name, M=M: [scheme_calls(name, M, p % P) for p in range(4)])
                rec[name] = round(time_graphs([g], 3) / 4 * 1e3, 2)  # us per layer set
                del g
                scheme_calls(name, M, 0)
                torch.cuda.synchronize()
                outs[name] = [ys[(mi, M)].clone() for mi in range(len(mats))]
            for name in names[1:]:
                for a, b in zip(outs["library"], outs[name]):
                    if not torch.equal(a.view(torch.int32), b.view(torch.int32)):
                        schemes["bits_identical"] = False
            schemes["rows"][str(M)] = rec
            log("schemes M=%d: %s" % (M, rec))
        del outs

    # ---- GEMV -> GEMM crossover on the layer set
    crossover = None
    if not args.no_crossover:
        cM = list(range(1, 21)) + [24, 28, 32, 33, 36, 40, 44, 48, 64, 96, 124, 128]
        table = []
        for M in cM:
            t = {}
            for kernel in ("gemv", "gemm"):
                g = capture(lambda M=M, kernel=kernel: [call(mi, M, p % P, kernel)
                                                        for p in range(4) for mi in range(len(mats))])
                g.replay()  # untimed first replay
                # best of three timings: a single disturbed timing must not move M*
                t[kernel] = min(time_graphs([g], 3) for _ in range(3)) / 4 * 1e3  # us per layer set
            table.append({"M": M, "gemv_us": round(t["gemv"], 2), "gemm_us": round(t["gemm"], 2),
                          "gemm_over_gemv": round(t["gemm"] / t["gemv"], 3)})
        # M*: the first sampled M from which the matrix-matrix kernel stays faster
        mstar = None
        for r in reversed(table):
            if r["gemm_us"] >= r["gemv_us"]:
                break
            mstar = r["M"]
        crossover = {"layer_set_table": table, "M_star": mstar,
                     "T_rule": (mstar - 1) if mstar else None,
                     "library_T": q4.get_crossover(),
                     "per_matrix": per_matrix_x or None}
        log("crossover M* = %s" % mstar)

    # ---- CPU baseline: the fp64 oracle on a bounded sample of the same step
    cpu = None
    if not args.no_cpu:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        os.environ.setdefault("OMP_NUM_THREADS", str(threads))
        oracle.load_library()
        done_bytes, done_rows, t_cpu, calls, passes = 0, 0, 0.0, 0, 0
        x_host = {K: xs[K][:8].view(torch.int16).cpu().numpy().view(np.uint16) for K in xs}
        w_host = [(base[mi].codes.cpu().numpy(), base[mi].scales.view(torch.int16).cpu().numpy().view(np.uint16))
                  for mi in range(len(mats))]
        # whole steps (the 48 calls in order) until the time budget is used;
        # a step cut short by the budget still counts the calls it made
        while t_cpu < args.cpu_seconds:
            for M in Ms:
                for mi, m in enumerate(mats):
                    if t_cpu >= args.cpu_seconds and calls % len(mats) == 0:
                        break
                    t0 = time.perf_counter()
                    oracle.linear_tiled(x_host[m.K][:M], True, w_host[mi][0], w_host[mi][1], m.N, m.K)
                    t_cpu += time.perf_counter() - t0
                    done_bytes += synth.algorithmic_bytes(M, m.N, m.K)
                    done_rows += M
                    calls += 1
            passes += 1
        cpu = {"value": round(done_bytes / t_cpu / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": "%d calls of the step (%d pass(es) over its 48 calls, M = 1..8 x 6 matrices), %.1f s"
                         % (calls, passes, t_cpu),
               "rows_per_s": round(done_rows / t_cpu, 2)}
        log("cpu oracle %.3f GB/s on %d threads" % (cpu["value"], threads))

    out = {
        "metric": "achieved HBM GB/s (% of peak) for Q4 linear at M=1..8, 7B shapes; crossover M",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Q4 codes uniform 0..15, fp16 scales |N(0,0.02)|, x ~ N(0,1) bf16)",
        "config": {"workload": "qwen2.5-7b_layer_set_M1-8",
                   "matrices": ["%s %dx%d" % (m.name, m.N, m.K) for m in mats],
                   "M": Ms, "calls_per_step": len(Ms) * len(mats), "kernel": args.kernel,
                   "rotation_pool_copies": P, "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 1),
                   "rows_per_s": round(rows_per_s, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "q4_gemv (split and segment forms), bf16", "launches_per_step": n_launch,
                     "avg_bytes_per_launch": int(bytes_step / n_launch),
                     "avg_launch_us": round(launch_ms * 1e3, 3)},
        "cpu_baseline": cpu,
        "detail": {"per_m_gbs": per_m, "per_matrix_gbs_m8": per_matrix_m8, "per_launch_us": per_launch_us, "fused_step": fused_step,
                   "decode_stream_7b": stream, "small_workloads": small, "switching_schemes": schemes, "crossover": crossover},
    }
    line = json.dumps(out)
    if args.detail_json:
        with open(args.detail_json, "w") as f:
            f.write(json.dumps(out, indent=1) + "\n")
    print(line)
    sys.stdout.flush()
    return 0


if __name__ == "__main__":
    sys.exit(main())
