#!/usr/bin/env python3
"""Benchmark of the Q4 linear layer on one MI355X.

Headline workload: the Qwen2.5-7B-shaped projection set (q 3584x3584, k and v
512x3584, gate and up 18944x3584, down 3584x18944), Q4 weights (blocks of 32,
fp16 scales), bf16 activations, at every decode row count M = 1..8.  One step
= the six projections at each M = 1..8 (48 calls through the library's
crossover dispatcher), each M on its own weight copy taken from a rotation
pool larger than the 256 MB Infinity Cache, so weights stream from HBM (no
copy is read twice within 1.5 GiB of weight traffic).  Inputs are seeded
synthetic data of those shapes (no trained weights); every input is resident
in HBM before the timed region.

Printed JSON line: value = achieved algorithmic HBM GB/s over the whole step
(codes + scales + activations + outputs per call, divided by step time);
roofline = the matrix-vector kernel (every launch of the step), its achieved
bandwidth from the measured launch durations of each (matrix, M) of the step
(back-to-back launches of one shape in a graph, timed with events on the
launch stream); cpu_baseline = the fp64 oracle timed on the host.  "detail" carries: a plain >= 2 GiB read timed in the same run
(the calibration every record's GB/s is also compared with), one record per
(workload, matrix, M, kernel) with time, bytes, GB/s, % of 8 TB/s, % of the
calibration read, rows/s, TFLOP/s, MFMA %, the oracle's max normalised
error on sampled outputs and the bit-invariance result; the grouped step
(q|k|v|gate|up in one launch, down in another), the fused-N step, the 7B
decode weight stream (28 layers + LM head), the 124-row mixed batch, the
0.5B-shaped and single-matvec workloads, GPT-2-small-shaped projections, the
pages' switching schemes and the GEMV -> GEMM crossover.

Timing: each step's 48 launches are captured once in a HIP graph (one graph
per offset into the pool); the timed region replays them between two events
on the launch stream, after a torch.cuda.synchronize() on both sides.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import ctypes.util
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E peak, 8 TB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 / fp16 matrix-core peak
CALIB_BYTES = 2 << 30        # the calibration read: 2 GiB

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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--pool-gib", type=float, default=1.5, help="rotation pool of weight copies (GiB)")
    ap.add_argument("--headline-only", action="store_true",
                    help="the headline step and its roofline only (no detail sections, no CPU leg): for profiling")
    ap.add_argument("--no-crossover", action="store_true", help="skip the GEMV/GEMM crossover sweep")
    ap.add_argument("--no-stream", action="store_true", help="skip the 28-layer decode weight stream")
    ap.add_argument("--no-fused", action="store_true", help="skip the fused-launch step")
    ap.add_argument("--no-grouped", action="store_true", help="skip the grouped-launch step")
    ap.add_argument("--no-schemes", action="store_true", help="skip the pages' switching schemes comparison")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the 0.5B-shaped layer set and the single 896 x 896 matvec")
    ap.add_argument("--no-gpt2", action="store_true", help="skip the GPT-2-small-shaped projections")
    ap.add_argument("--no-mixed", action="store_true", help="skip the 124-row mixed batch")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg (baseline and error checks)")
    ap.add_argument("--no-per-launch", action="store_true",
                    help="skip the per-matrix launch timings (per-M and per-matrix GB/s)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the CPU oracle's headline sample")
    ap.add_argument("--kernel", default="auto", choices=["auto", "gemv", "gemm"])
    ap.add_argument("--detail-json", default=None, help="also write the full results here")
    ap.add_argument("--records-csv", default=None, help="also write the per-record table here")
    ap.add_argument("--eager-step", action="store_true",
                    help="run one step's launches eagerly (no graphs) and exit: for hardware-counter passes")
    ap.add_argument("--eager-m", default=None, metavar="M,M,...",
                    help="row counts of the eager step (default 1..8), e.g. 124 with --kernel gemm")
    ap.add_argument("--eager-reps", type=int, default=1, help="repeat the eager step (weights from the pool)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run 8 plain device copies of MIB MiB each and exit: calibrates byte counters")
    a = ap.parse_args()
    if a.headline_only:
        for f in ("no_crossover", "no_stream", "no_fused", "no_grouped", "no_schemes", "no_small", "no_gpt2",
                  "no_mixed", "no_cpu", "no_per_launch"):
            setattr(a, f, True)
    return a


class Records:
    """One record per (workload, matrix, M, kernel), plus the sampled GPU
    outputs the CPU leg checks against the oracle."""

    def __init__(self, calib_gbs):
        self.calib = calib_gbs
        self.rows = []
        self.samples = []

    def add(self, workload, matrix, M, kernel, us, nbytes, flops, x="bf16", bits_invariant=None, mfma=False,
            calls=1):
        gbs = nbytes / (us * 1e-6) / 1e9
        tflops = flops / (us * 1e-6) / 1e12
        rec = {"workload": workload, "matrix": matrix, "M": M, "kernel": kernel, "x": x, "calls": calls,
               "us": round(us, 3), "bytes": int(nbytes), "gbs": round(gbs, 1),
               "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
               "pct_calibration": round(100 * gbs / self.calib, 2) if self.calib else None,
               "rows_per_s": round(M / (us * 1e-6), 1), "tflops": round(tflops, 3),
               "mfma_pct": round(100 * tflops / PEAK_BF16_TFLOPS, 2) if mfma else None,
               "max_norm_err": None, "bits_invariant": bits_invariant}
        self.rows.append(rec)
        return len(self.rows) - 1

    def sample(self, idx, y, x_bits, bf16, wq_t, sc_t, N, K, rng, n=192):
        """Keep n sampled outputs of y (with the four corners) for record(s)
        idx; the oracle checks them in the CPU leg."""
        import numpy as np
        M = y.shape[0]
        ms = np.concatenate([rng.integers(0, M, n), [0, M - 1, 0, M - 1]])
        ns = np.concatenate([rng.integers(0, N, n), [0, 0, N - 1, N - 1]])
        yh = y.cpu().numpy()
        self.samples.append({"records": list(idx) if isinstance(idx, (list, tuple)) else [idx], "x": x_bits[:M],
                             "bf16": bf16, "wq": wq_t, "sc": sc_t, "N": N, "K": K, "ms": ms, "ns": ns,
                             "vals": yh[ms, ns]})


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
    if not os.path.exists(hip_build.PROBE_LIB):
        hip_build.build_probe()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mats = synth.SET_7B
    Ms = list(range(1, 9))
    set_bytes = sum(sum(q4.packed_sizes(m.N, m.K)) for m in mats)
    P = max(2, int(np.ceil(args.pool_gib * (1 << 30) / set_bytes)))
    log("device %s, rotation pool %d copies of the layer set (%.2f GiB)"
        % (torch.cuda.get_device_name(dev), P, P * set_bytes / (1 << 30)))

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

    def best_per_call(fn, calls, tries=3):
        """Best of `tries` timings of one graph of `calls` back-to-back calls (us per call)."""
        g = capture(fn)
        g.replay()  # untimed first replay
        us = min(time_graphs([g], 1) for _ in range(tries)) / calls * 1e3
        del g
        return us

    # ---- the calibration read: a plain streaming read of 2 GiB, in this run
    plib = ctypes.CDLL(hip_build.PROBE_LIB)
    plib.q4probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    plib.q4probe_read.restype = ctypes.c_int
    calib = None
    if not (args.headline_only or args.eager_step):
        cbuf = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        best = (1e30, 0)
        for blocks in (256, 1024, 2048):
            def rd(blocks=blocks):
                st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                assert plib.q4probe_read(cbuf.data_ptr(), CALIB_BYTES, sink.data_ptr(), blocks, st) == 0
            us = best_per_call(rd, 1, tries=5)
            best = min(best, (us, blocks))
        calib = {"bytes": CALIB_BYTES, "us": round(best[0], 2), "gbs": round(CALIB_BYTES / (best[0] * 1e-6) / 1e9, 1),
                 "workgroups": best[1], "kernel": "probe_read (16-byte non-temporal loads, grid-stride)"}
        calib["pct_peak"] = round(100 * calib["gbs"] / PEAK_HBM_GBS, 1)
        del cbuf
        torch.cuda.empty_cache()
        log("calibration read: %.1f GB/s (%.1f%% of 8 TB/s)" % (calib["gbs"], calib["pct_peak"]))
    records = Records(calib["gbs"] if calib else None)

    # ---- issue overlap of the matrix core and the VALU (probe_issue): per
    # iteration a wave runs 4 independent bf16 block dots (mode 1), 16
    # independent fp32 FMAs (mode 2) or both (mode 3); cycles per iteration
    # of one SIMD at 2.4 GHz, 1 and 4 waves per SIMD.  Both together taking
    # about the sum of the two alone means their issue does not overlap,
    # which bounds the matrix-matrix kernel (its per-block fmaf and
    # subtraction are VALU work on top of every block dot).
    issue = None
    if not (args.headline_only or args.eager_step):
        plib.q4probe_issue.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        plib.q4probe_issue.restype = ctypes.c_int
        iters = 4000
        issue = {"iterations": iters, "work_per_wave_iteration": "4 v_mfma_f32_16x16x32_bf16 + 16 v_fma_f32",
                 "cycles_per_iteration_per_simd": {}}
        for wps in (1, 4):
            pout = torch.empty(256 * wps * 256, dtype=torch.float32, device=dev)
            row = {}
            for mode, name in ((1, "mfma_only"), (2, "valu_only"), (3, "both")):
                def run(mode=mode, wps=wps, pout=pout):
                    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                    assert plib.q4probe_issue(mode, pout.data_ptr(), 256 * wps, iters, st) == 0
                us = best_per_call(run, 1, tries=3)
                row[name] = round(us * 1e-6 * 2.4e9 / iters, 1)
            issue["cycles_per_iteration_per_simd"]["%d_waves_per_simd" % wps] = row
            del pout
        log("issue overlap (cycles per iteration per SIMD): %s" % issue["cycles_per_iteration_per_simd"])

    # ---- the fixed cost of a launch: a graph of 48 back-to-back empty kernels
    # (1 and 256 workgroups), us per launch.  The step's 48 launches pay it
    # before any work.
    launch_floor = None
    if not (args.headline_only or args.eager_step):
        plib.q4probe_empty.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        plib.q4probe_empty.restype = ctypes.c_int
        esink = torch.zeros(256, dtype=torch.int32, device=dev)
        launch_floor = {}
        for nb in (1, 256):
            def empties(nb=nb):
                st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                for _ in range(48):
                    assert plib.q4probe_empty(esink.data_ptr(), nb, 0, st) == 0
            launch_floor["%d_workgroups_us" % nb] = round(best_per_call(empties, 48, tries=5), 3)
        launch_floor["step_launches"] = 48
        launch_floor["us_per_step"] = round(48 * launch_floor["1_workgroups_us"], 1)
        log("empty-kernel launch floor: %s" % launch_floor)

    # ---- reads with the matrix-vector kernels' own streaming structure
    # (probe_ring_read: each wave streams a contiguous run of 1 KB quads
    # through a register ring, nothing computed), each launch on another
    # region of a 1.5 GiB buffer: the floor of a kernel built that way, next
    # to the per-launch times of the kernels that have that structure.
    read_structure = None
    if not (args.headline_only or args.eager_step):
        vp, ci = ctypes.c_void_p, ctypes.c_int
        plib.q4probe_ring_read.argtypes = [vp, ci, ci, ci, ci, vp, vp]
        plib.q4probe_ring_read.restype = ci
        rbytes = 3 << 29
        rbuf = torch.empty(rbytes, dtype=torch.uint8, device=dev)
        rsink = torch.zeros(4, dtype=torch.int32, device=dev)
        read_structure = {}
        for name, W, Q, wpg, D in (("down_proj split form: 224 workgroups x 8 waves, 19 quads a wave, 4-deep", 1792, 19, 8, 4),
                                   ("gate_proj segment form: 237 workgroups x 16 waves, 10 quads a wave, 2-deep", 3792, 10, 16, 2),
                                   ("gate_proj segment form with a 4-deep ring", 3792, 10, 16, 4)):
            nb = W * Q * 1024
            calls = rbytes // nb
            def rr(W=W, Q=Q, wpg=wpg, D=D, nb=nb, calls=calls):
                st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                for i in range(calls):
                    assert plib.q4probe_ring_read(rbuf.data_ptr() + i * nb, Q, W, wpg, D, rsink.data_ptr(), st) == 0
            us = best_per_call(rr, calls, tries=3)
            read_structure[name] = {"bytes": nb, "us": round(us, 2), "gbs": round(nb / (us * 1e-6) / 1e9, 1)}
        del rbuf
        torch.cuda.empty_cache()
        log("read structure floors: %s" % {k: v["us"] for k, v in read_structure.items()})

    # ---- inputs, resident in HBM: weights drawn directly in the packed form.
    # Each copy of the set is held as the fused buffers (q|k|v, gate|up,
    # down); the six projections are views into them.
    base, base_host = [], []
    for mi, m in enumerate(mats):
        wq_t, sc_t = synth.packed_weight(m.N, m.K, 3, mi)
        base_host.append((wq_t, sc_t))
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
    xs, xh = {}, {}
    for K in sorted({m.K for m in mats}):
        xh[K] = synth.activations(Mmax, K, "bf16", 3, 100 + K)
        xs[K] = torch.from_numpy(xh[K].view(np.int16)).to(dev).view(torch.bfloat16)
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

    def call_grouped(M, views):
        q4.linear_grouped(xs[3584][:M], views[:5], outs=[ys[(mi, M)] for mi in range(5)], workspace=True)
        q4.linear(xs[18944][:M], views[5], out=ys[(5, M)])

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
    n_launch = len(Ms) * len(mats)
    log("step %.3f us, %.1f GB/s (%.1f%% of 8 TB/s)" % (ms_step * 1e3, value, 100 * value / PEAK_HBM_GBS))
    del step_graphs

    # ---- per-launch times of each (matrix, M) and per-M bandwidth:
    # back-to-back launches of one shape, one graph, each launch on another
    # copy of the matrix.  The copies span at least the pool's size per
    # matrix (the step pool's copies plus clones), so that every launch
    # streams its weights from HBM.  The per-matrix crossover (M* of each
    # projection alone) is taken on the same pools, with each kernel forced.
    rng = np.random.default_rng(7)
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
            # bits: each row of every M equals that row at M = 8, and the
            # matrix-matrix kernel's rows equal the matrix-vector kernel's
            y8 = q4.linear(xs[m.K][:8], base[mi], kernel="gemv").cpu().numpy().view(np.uint32)
            inv = bool(np.array_equal(q4.linear(xs[m.K][:8], base[mi], kernel="gemm").cpu().numpy().view(np.uint32), y8))
            for M in Ms:
                inv = inv and bool(np.array_equal(q4.linear(xs[m.K][:M], base[mi]).cpu().numpy().view(np.uint32),
                                                  y8[:M]))
            for M in Ms:
                us = best_per_call(lambda M=M, mi=mi, mpool=mpool: [
                    q4.linear(xs[m.K][:M], w, out=ys[(mi, M)], kernel=args.kernel) for w in mpool], len(mpool))
                per_launch[(mi, M)] = us * 1e-3  # ms
                idx = records.add("qwen2.5-7b_layer_set", m.name, M, args.kernel, us,
                                  synth.algorithmic_bytes(M, m.N, m.K), 2 * M * m.N * m.K, bits_invariant=inv)
                records.sample(idx, q4.linear(xs[m.K][:M], base[mi], kernel=args.kernel), xh[m.K], True,
                               base_host[mi][0], base_host[mi][1], m.N, m.K, rng)
            if not args.no_crossover:
                rows = []
                for M in xM:
                    t = {}
                    for kern in ("gemv", "gemm"):
                        t[kern] = best_per_call(lambda M=M, mi=mi, mpool=mpool, kern=kern: [
                            q4.linear(xs[m.K][:M], w, out=ys[(mi, M)], kernel=kern) for w in mpool], len(mpool), 2)
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
            records.add("qwen2.5-7b_layer_set", "layer_set", M, args.kernel, t * 1e3, step_bytes([M]),
                        sum(2 * M * mm.N * mm.K for mm in mats), calls=len(mats))
        per_matrix_m8 = {mats[mi].name: round(synth.algorithmic_bytes(8, mats[mi].N, mats[mi].K)
                                              / (per_launch[(mi, 8)] * 1e-3) / 1e9, 1) for mi in range(len(mats))}
        per_launch_us = {m.name: {str(M): round(per_launch[(mi, M)] * 1e3, 2) for M in Ms}
                         for mi, m in enumerate(mats)}
        log("per-M GB/s %s" % per_m)
        log("per-matrix GB/s at M=8 %s" % per_matrix_m8)

    # ---- roofline of the dominant kernel (every launch of the step runs the
    # matrix-vector kernel): achieved = the step's algorithmic bytes over the
    # sum of its 48 launches' measured durations, each (matrix, M) timed as
    # back-to-back launches of that one shape in a graph on the launch stream
    # (above); without those timings, the timed region's average per launch
    if per_launch:
        disp_us = sum(per_launch[(mi, M)] for M in Ms for mi in range(len(mats))) * 1e3 / n_launch
        disp_src = "per-(matrix, M) launch durations, back-to-back launches of each shape in a graph"
    else:
        disp_us = ms_step * 1e3 / n_launch
        disp_src = "timed region / launches"
    achieved = bytes_step / n_launch / (disp_us * 1e-6) / 1e9
    log("roofline: %.3f us average launch duration -> %.1f GB/s" % (disp_us, achieved))

    # ---- the grouped step: per M, q|k|v|gate|up in one q4_linear_grouped
    # launch (they share x) and down in another: 16 launches a step.  x is
    # read once per grouped launch, so the step's algorithmic bytes count it
    # once for the five.
    grouped_step = None
    if not args.no_grouped:
        ggraphs = [capture(lambda p=p: [call_grouped(M, pool[copy_of(p, j)]) for j, M in enumerate(Ms)])
                   for p in range(P)]
        for i in range(args.warmup):
            ggraphs[i % P].replay()
        ms_g = time_graphs(ggraphs, args.steps)
        del ggraphs
        gbytes = bytes_step - sum(4 * 2 * M * 3584 for M in Ms)
        same = True
        for M in Ms:
            call_grouped(M, pool[0])
            yg = [ys[(mi, M)].clone() for mi in range(6)]
            for mi in range(6):
                call(mi, M, 0, "auto")
                same = same and torch.equal(yg[mi].view(torch.int32), ys[(mi, M)].view(torch.int32))
        per_m_g = {}
        for j, M in enumerate(Ms):
            us = best_per_call(lambda M=M: [call_grouped(M, pool[p]) for p in range(P)], P)
            nb = step_bytes([M]) - 4 * 2 * M * 3584
            per_m_g[str(M)] = {"us": round(us, 2), "gbs": round(nb / (us * 1e-6) / 1e9, 1)}
            records.add("qwen2.5-7b_layer_set_grouped", "q|k|v|gate|up + down", M, "auto", us, nb,
                        sum(2 * M * mm.N * mm.K for mm in mats), calls=2, bits_invariant=same)
        grouped_step = {"calls_per_step": 2 * len(Ms), "us_per_step": round(ms_g * 1e3, 2),
                        "gbs": round(gbytes / (ms_g * 1e-3) / 1e9, 1),
                        "pct_of_peak": round(100 * gbytes / (ms_g * 1e-3) / 1e9 / PEAK_HBM_GBS, 1),
                        "pct_of_calibration": round(100 * gbytes / (ms_g * 1e-3) / 1e9 / calib["gbs"], 1) if calib else None,
                        "rows_per_s": round(sum(Ms) / (ms_g * 1e-3), 1), "bits_identical_to_separate_calls": same,
                        "per_M": per_m_g}
        log("grouped step %.2f us, %.1f GB/s" % (ms_g * 1e3, grouped_step["gbs"]))

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

    # ---- the 124-row mixed batch (120 prefill + 4 verify rows) on the 7B
    # set: the matrix-matrix kernel (above the crossover), per matrix on the
    # pool, with its K-split workspace; MFMA utilisation = useful TFLOP/s
    # over the 2.5 PFLOP/s dense bf16 peak
    mixed = None
    if not args.no_mixed:
        M = 124
        mixed = {"per_matrix": {}}
        tot_us = 0.0
        for mi, m in enumerate(mats):
            wsb = q4.workspace_bytes(M, m.N, m.K, "auto")
            wsp = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
            us = best_per_call(lambda mi=mi, m=m, wsp=wsp: [
                q4.linear(xs[m.K][:M], pool[p][mi], out=ys[(mi, M)], workspace=wsp) for p in range(P)], P)
            tot_us += us
            idx = records.add("qwen2.5-7b_mixed_124", m.name, M, "auto", us, synth.algorithmic_bytes(M, m.N, m.K),
                              2 * M * m.N * m.K, mfma=True)
            y = q4.linear(xs[m.K][:M], base[mi], workspace=wsp)
            y4 = q4.linear(xs[m.K][120:124].contiguous(), base[mi])
            records.rows[idx]["bits_invariant"] = bool(torch.equal(y[120:124].view(torch.int32), y4.view(torch.int32)))
            records.sample(idx, y, xh[m.K], True, base_host[mi][0], base_host[mi][1], m.N, m.K, rng)
            mixed["per_matrix"][m.name] = round(us, 2)
            del wsp
        nb = step_bytes([M])
        fl = sum(2 * M * mm.N * mm.K for mm in mats)
        records.add("qwen2.5-7b_mixed_124", "layer_set", M, "auto", tot_us, nb, fl, mfma=True, calls=len(mats))
        mixed.update({"layer_set_us": round(tot_us, 2), "tflops": round(fl / (tot_us * 1e-6) / 1e12, 1),
                      "mfma_pct": round(100 * fl / (tot_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 2),
                      "gbs": round(nb / (tot_us * 1e-6) / 1e9, 1)})
        log("mixed 124 rows: %s" % mixed)

    # ---- the whole 7B decode weight stream: 28 distinct copies of the layer
    # set plus the LM head, per M, as one graph (separate, fused and grouped
    # calls)
    stream = None
    if not args.no_stream:
        from synth import LM_HEAD_7B, N_LAYERS_7B
        layers = [fused_copy() for _ in range(N_LAYERS_7B)]
        hq, hs = synth.packed_weight(LM_HEAD_7B.N, LM_HEAD_7B.K, 5, 6)
        head = q4.Q4Weight(torch.from_numpy(hq).to(dev),
                           torch.from_numpy(hs.view(np.int16)).to(dev).view(torch.float16),
                           LM_HEAD_7B.N, LM_HEAD_7B.K)
        stream = {}
        for M in (1, 4, 16, 64):
            yh = torch.empty((M, LM_HEAD_7B.N), dtype=torch.float32, device=dev)

            def run(mode, M=M, yh=yh):
                for f, v in layers:
                    if mode == "fused":
                        for j in range(len(fmats)):
                            call_fused(j, M, f[j])
                    elif mode == "grouped":
                        call_grouped(M, v)
                    else:
                        for mi in range(len(mats)):
                            q4.linear(xs[mats[mi].K][:M], v[mi], out=ys[(mi, M)])
                q4.linear(xs[LM_HEAD_7B.K][:M], head, out=yh)
            nbytes = N_LAYERS_7B * step_bytes([M]) + synth.algorithmic_bytes(M, LM_HEAD_7B.N, LM_HEAD_7B.K)
            rec = {}
            for mode in ("separate", "fused", "grouped"):
                g = capture(lambda mode=mode: run(mode))
                ms = time_graphs([g], 5)
                del g
                rec[mode] = {"us": round(ms * 1e3, 1), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                             "rows_per_s": round(M / (ms * 1e-3), 1)}
                records.add("qwen2.5-7b_decode_weight_stream", "28 layers + lm_head (%s)" % mode, M, "auto",
                            ms * 1e3, nbytes, 2 * M * (N_LAYERS_7B * sum(mm.N * mm.K for mm in mats)
                                                       + LM_HEAD_7B.N * LM_HEAD_7B.K),
                            calls=(N_LAYERS_7B * {"separate": 6, "fused": 3, "grouped": 2}[mode] + 1))
            stream[str(M)] = rec
            yhead = q4.linear(xs[LM_HEAD_7B.K][:M], head)
            idx = records.add("qwen2.5-7b_decode_weight_stream", "lm_head", M, "auto",
                              best_per_call(lambda M=M, yh=yh: [q4.linear(xs[LM_HEAD_7B.K][:M], head, out=yh)], 1),
                              synth.algorithmic_bytes(M, LM_HEAD_7B.N, LM_HEAD_7B.K), 2 * M * LM_HEAD_7B.N * LM_HEAD_7B.K)
            records.sample(idx, yhead, xh[LM_HEAD_7B.K], True, hq, hs, LM_HEAD_7B.N, LM_HEAD_7B.K, rng)
            log("decode stream M=%d: %s" % (M, rec))
        del layers, head
        torch.cuda.empty_cache()

    # ---- the small workloads: the single 896 x 896 matvec at M = 1 and the
    # Qwen2.5-0.5B-shaped layer set at M = 1, 2, 4 (fp16 activations), and
    # the GPT-2-small-shaped projections (768 x 768, bf16) at M = 1..16.  Each
    # call on its own weight copy; these are latency-bound (well under a
    # microsecond of weight traffic at 8 TB/s): report us per call.
    small = {}
    wls = ([] if args.no_small else [1, 2]) + ([] if args.no_gpt2 else [6])
    # grouped form of the sets (q4_linear_grouped): the 0.5B layer's q, k, v,
    # gate and up in one launch (sharing x, as the 7B grouped step) and down
    # alone; GPT-2's q, k and v in one launch and o alone
    groups = {2: ([0, 1, 2, 3, 4], [5]), 6: ([0, 1, 2], [3])}
    for wl in wls:
        spec = synth.WORKLOADS[wl]
        smats = spec["matrices"]
        bf16 = spec["x"] == "bf16"
        gsel = groups.get(wl)
        sbytes = sum(sum(q4.packed_sizes(m.N, m.K)) for m in smats)
        SP = int(min(2048, max(2, np.ceil(args.pool_gib * (1 << 30) / 2 / sbytes))))
        sbase, shost = [], []
        for mi, m in enumerate(smats):
            wq_t, sc_t = synth.packed_weight(m.N, m.K, wl, mi)
            shost.append((wq_t, sc_t))
            sbase.append(q4.Q4Weight(torch.from_numpy(wq_t).to(dev),
                                     torch.from_numpy(sc_t.view(np.int16)).to(dev).view(torch.float16), m.N, m.K))
        spool = [[q4.Q4Weight(w.codes.clone(), w.scales.clone(), w.N, w.K) for w in sbase] for _ in range(SP)]
        Mx = max(spec["Ms"])
        sxh, sx = {}, {}
        for K in sorted({m.K for m in smats}):
            sxh[K] = synth.activations(Mx, K, spec["x"], wl, 100 + K)
            sx[K] = torch.from_numpy(sxh[K].view(np.int16)).to(dev).view(torch.bfloat16 if bf16 else torch.float16)
        rec = {}
        for M in spec["Ms"]:
            ysm = [torch.empty((M, m.N), dtype=torch.float32, device=dev) for m in smats]
            us = best_per_call(lambda M=M, ysm=ysm: [q4.linear(sx[m.K][:M], spool[p][mi], out=ysm[mi])
                                                    for p in range(SP) for mi, m in enumerate(smats)], SP)
            nb = sum(synth.algorithmic_bytes(M, m.N, m.K) for m in smats)
            rec[str(M)] = {"us_per_set": round(us, 2), "us_per_call": round(us / len(smats), 2),
                           "gbs": round(nb / (us * 1e-6) / 1e9, 1), "rows_per_s": round(M / (us * 1e-6), 1)}
            idx = records.add(spec["name"], "set of %d" % len(smats), M, "auto", us, nb,
                              sum(2 * M * m.N * m.K for m in smats), x=spec["x"], calls=len(smats))
            for mi, m in enumerate(smats):
                records.sample(idx, q4.linear(sx[m.K][:M], sbase[mi]), sxh[m.K], bf16, shost[mi][0], shost[mi][1],
                               m.N, m.K, rng, n=64)
            if gsel is not None:
                gi, rest = gsel
                Kg = smats[gi[0]].K

                def call_set_grouped(p, M=M, ysm=ysm):
                    q4.linear_grouped(sx[Kg][:M], [spool[p][i] for i in gi], outs=[ysm[i] for i in gi],
                                      workspace=False)
                    for r in rest:
                        q4.linear(sx[smats[r].K][:M], spool[p][r], out=ysm[r])

                gus = best_per_call(lambda: [call_set_grouped(p) for p in range(SP)], SP)
                ybase = [q4.linear(sx[m.K][:M], sbase[mi]).cpu().numpy().view(np.uint32) for mi, m in enumerate(smats)]
                yg = q4.linear_grouped(sx[Kg][:M], [sbase[i] for i in gi], workspace=False)
                same = all(np.array_equal(yg[j].cpu().numpy().view(np.uint32), ybase[i]) for j, i in enumerate(gi))
                gnb = nb - (len(gi) - 1) * 2 * M * Kg  # x read once for the group
                rec[str(M)].update({"grouped_us_per_set": round(gus, 2), "grouped_calls": 1 + len(rest),
                                    "grouped_gbs": round(gnb / (gus * 1e-6) / 1e9, 1),
                                    "grouped_bits_identical": same})
                records.add(spec["name"] + "_grouped", "%s in one launch + %d" % (
                    "|".join(smats[i].name for i in gi), len(rest)), M, "auto", gus, gnb,
                    sum(2 * M * m.N * m.K for m in smats), x=spec["x"], calls=1 + len(rest), bits_invariant=same)
        small[spec["name"]] = {"matrices": ["%s %dx%d" % (m.name, m.N, m.K) for m in smats],
                               "x": spec["x"], "weight_copies": SP, "per_M": rec,
                               "grouped": None if gsel is None else {
                                   "group": [smats[i].name for i in gsel[0]],
                                   "separate": [smats[i].name for i in gsel[1]]}}
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

    # ---- the CPU leg: the fp64 oracle (a) timed on the host's cores on a
    # bounded sample of the headline step (the baseline), plus short legs of
    # the other workloads and single-thread legs, and (b) checking every
    # sampled GPU output above against its fp64 value (max |y - y_ref| / A)
    cpu = parity = None
    if not args.no_cpu:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        os.environ.setdefault("OMP_NUM_THREADS", str(threads))
        oracle.load_library()
        gomp = ctypes.CDLL(ctypes.util.find_library("gomp") or "libgomp.so.1")

        def set_threads(n):
            gomp.omp_set_num_threads(int(n))

        set_threads(threads)
        x_host = {K: xh[K][:8] for K in xh}

        def timed(fn):
            t0 = time.perf_counter()
            fn()
            return time.perf_counter() - t0

        # (a) the baseline: whole steps (the 48 calls in order) until the
        # time budget is used; a step cut short still counts its calls
        done_bytes, done_rows, t_cpu, calls, passes_cpu = 0, 0, 0.0, 0, 0
        while t_cpu < args.cpu_seconds:
            for M in Ms:
                for mi, m in enumerate(mats):
                    if t_cpu >= args.cpu_seconds and calls % len(mats) == 0:
                        break
                    t_cpu += timed(lambda: oracle.linear_tiled(x_host[m.K][:M], True, base_host[mi][0],
                                                              base_host[mi][1], m.N, m.K))
                    done_bytes += synth.algorithmic_bytes(M, m.N, m.K)
                    done_rows += M
                    calls += 1
            passes_cpu += 1
        cpu = {"value": round(done_bytes / t_cpu / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": "%d calls of the step (%d pass(es) over its 48 calls, M = 1..8 x 6 matrices), %.1f s"
                         % (calls, passes_cpu, t_cpu),
               "rows_per_s": round(done_rows / t_cpu, 2)}
        log("cpu oracle %.3f GB/s on %d threads" % (cpu["value"], threads))

        # other workloads, all threads and one thread (bounded samples)
        legs = {}

        def leg(name, fn, nbytes, rows, one_thread):
            """fn repeated until 0.25 s have passed; time per call."""
            res = {}
            for n in ([threads, 1] if one_thread else [threads]):
                set_threads(n)
                fn()  # warm: thread pool, pages
                reps, t = 0, 0.0
                while t < 0.25:
                    t += timed(fn)
                    reps += 1
                t /= reps
                res["threads_%d" % n] = {"s_per_call": round(t, 5), "reps": reps, "gbs": round(nbytes / t / 1e9, 4),
                                         "rows_per_s": round(rows / t, 2)}
            set_threads(threads)
            legs[name] = res

        s1 = synth.WORKLOADS[1]["matrices"][0]
        w1 = synth.packed_weight(s1.N, s1.K, 1, 0)
        x1 = synth.activations(1, s1.K, "f16", 1, 100 + s1.K)
        leg("q4_matvec_896 M=1", lambda: oracle.linear_tiled(x1, False, w1[0], w1[1], s1.N, s1.K),
            synth.algorithmic_bytes(1, s1.N, s1.K), 1, True)
        s2 = synth.WORKLOADS[2]["matrices"]
        w2 = [synth.packed_weight(m.N, m.K, 2, mi) for mi, m in enumerate(s2)]
        x2 = {K: synth.activations(4, K, "f16", 2, 100 + K) for K in {m.K for m in s2}}
        for M in (1, 2, 4):
            leg("qwen2.5-0.5b_layer_set M=%d" % M,
                lambda M=M: [oracle.linear_tiled(x2[m.K][:M], False, w2[mi][0], w2[mi][1], m.N, m.K)
                             for mi, m in enumerate(s2)],
                sum(synth.algorithmic_bytes(M, m.N, m.K) for m in s2), M, True)
        for M in (1, 8):
            leg("qwen2.5-7b_layer_set M=%d" % M,
                lambda M=M: [oracle.linear_tiled(x_host[m.K][:M], True, base_host[mi][0], base_host[mi][1], m.N, m.K)
                             for mi, m in enumerate(mats)],
                step_bytes([M]), M, M == 1)
        # 124 rows: k_proj and v_proj (a bounded sample of the set)
        leg("qwen2.5-7b_mixed_124 k_proj+v_proj",
            lambda: [oracle.linear_tiled(xh[3584][:124], True, base_host[mi][0], base_host[mi][1],
                                         mats[mi].N, mats[mi].K) for mi in (1, 2)],
            sum(synth.algorithmic_bytes(124, mats[mi].N, mats[mi].K) for mi in (1, 2)), 124, False)
        # decode weight stream at one row: one layer set and the LM head,
        # scaled to the whole step (28 layer sets + the head)
        from synth import LM_HEAD_7B, N_LAYERS_7B
        hq5, hs5 = synth.packed_weight(LM_HEAD_7B.N, LM_HEAD_7B.K, 5, 6)
        t_head = timed(lambda: oracle.linear_tiled(x_host[3584][:1], True, hq5, hs5, LM_HEAD_7B.N, LM_HEAD_7B.K))
        t_set = legs["qwen2.5-7b_layer_set M=1"]["threads_%d" % threads]["s_per_call"]
        t5 = N_LAYERS_7B * t_set + t_head
        b5 = N_LAYERS_7B * step_bytes([1]) + synth.algorithmic_bytes(1, LM_HEAD_7B.N, LM_HEAD_7B.K)
        legs["qwen2.5-7b_decode_weight_stream M=1 (28 x layer set + lm_head, scaled)"] = {
            "threads_%d" % threads: {"s": round(t5, 3), "gbs": round(b5 / t5 / 1e9, 4), "rows_per_s": round(1 / t5, 3),
                                     "lm_head_s": round(t_head, 3)}}
        cpu["other_workloads"] = legs

        # (b) the sampled GPU outputs against the oracle
        worst = 0.0
        for smp in records.samples:
            y_ref, a_ref = oracle.linear_sampled(smp["x"], smp["bf16"], smp["wq"], smp["sc"], smp["ms"], smp["ns"],
                                                 tiled_nk=(smp["N"], smp["K"]))
            err = oracle.max_normalised_error(smp["vals"], y_ref, a_ref)
            worst = max(worst, err)
            for ri in smp["records"]:
                prev = records.rows[ri]["max_norm_err"]
                records.rows[ri]["max_norm_err"] = float("%.3g" % max(err, prev or 0.0))
        parity = {"max_norm_err": float("%.3g" % worst), "tolerance": 2e-3, "sampled_calls": len(records.samples),
                  "outputs_checked": int(sum(len(s["ms"]) for s in records.samples)), "pass": worst <= 2e-3}
        log("sampled outputs against the oracle: max normalised error %.3g over %d calls"
            % (worst, len(records.samples)))

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
                   "pct_of_calibration": round(100 * value / calib["gbs"], 1) if calib else None,
                   "rows_per_s": round(rows_per_s, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "q4_gemv (split and segment forms), bf16", "launches_per_step": n_launch,
                     "avg_bytes_per_launch": int(bytes_step / n_launch),
                     "avg_launch_us": round(disp_us, 3), "avg_launch_us_source": disp_src,
                     "timed_region_us_per_launch": round(ms_step * 1e3 / n_launch, 3)},
        "cpu_baseline": cpu,
        "detail": {"calibration_read": calib, "parity": parity,
                   "per_m_gbs": per_m, "per_matrix_gbs_m8": per_matrix_m8, "per_launch_us": per_launch_us,
                   "grouped_step": grouped_step, "fused_step": fused_step, "mixed_124": mixed, "issue_overlap": issue, "launch_floor": launch_floor,
                   "read_structure": read_structure,
                   "decode_stream_7b": stream, "small_workloads": small or None, "switching_schemes": schemes,
                   "crossover": crossover, "records": records.rows},
    }
    line = json.dumps(out)
    if args.detail_json:
        with open(args.detail_json, "w") as f:
            f.write(json.dumps(out, indent=1) + "\n")
    if args.records_csv and records.rows:
        with open(args.records_csv, "w", newline="") as f:
            wr = csv.DictWriter(f, fieldnames=list(records.rows[0].keys()))
            wr.writeheader()
            wr.writerows(records.rows)
    print(line)
    sys.stdout.flush()
    return 0


if __name__ == "__main__":
    sys.exit(main())
