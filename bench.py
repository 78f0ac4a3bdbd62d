#!/usr/bin/env python3
"""Benchmark of the SS2D hot path on one MI355X.

One step = one fused SS2D forward (cross-scan addressing -> four selective scans ->
cross-merge + skip + gate) over one batch of the stage-1 VMamba workload (batch 128,
56x56 map, D = 192 channels, N = 16 states, bf16 I/O, fp32 state, z gate).  Inputs are
seeded synthetic tensors already resident in HBM when the timed region starts.

Prints one JSON line: elements/s (B*K*D*L per second) as the value, per-step median /
min / max, the whole-step algorithmic HBM rate against the 8 TB/s peak and against a
device copy timed in the same run, the roofline of the dominant kernel (the route-scan
kernel, timed live with HIP events on the stream it is launched on; for state sizes 1, 2
and 4 the whole forward is one HBM-bound kernel per plane, and that one) and the fp64 CPU
oracle timed on this host on a bounded sample of the same workload.  `--workload`
selects one of the other shapes (0-4 SS2D, 5 the Vision Mamba bidirectional scan at
Vim-Tiny size); `--bwd` adds the fused backward to each step; `--front K` puts the
input front (depthwise K x K convolution + SiLU) ahead of the SS2D routes; `--ln` adds the
back half (LayerNorm over the channels of the merged map before the gate); `--proj R` makes
Δ, B and C come from the per-route projections of the scanned sequence (dt_rank R, on the
matrix cores) instead of being inputs.

When one input/output set is smaller than the 256 MB last-level cache (MALL) several
times over, the steps rotate over independent copies so that no step re-reads what the
previous one left in that cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SS2D scan elements/s (B·K·D·L) + achieved HBM GB/s vs peak, 56×56 stage"
HBM_PEAK_GBPS = 8000.0
CLOCK_HZ = 2.4e9
SIMDS = 256 * 4  # 256 CUs x 4 SIMDs, 16 fp32 lanes each
# The published fp32 vector peak of the MI355X: the roofline's peak.  It counts packed-FP32
# instructions (two lanes' FMAs in one), which this library does not issue (packed fp32 is
# disabled in its build), so the scan kernels cannot reach more than half of it.
PUBLISHED_FP32_VECTOR_TFLOPS = 157.3
# fp32 vector peak without packed math: 1024 SIMDs x 16 lanes x 2 flops (FMA) x 2.4 GHz (extra)
VALU_PEAK_TFLOPS = SIMDS * 16 * 2 * CLOCK_HZ / 1e12
# Per (element, state) the forward scan issues 4 full-rate VALU ops (Lam*A, (Lam*u)*B, the FMA into
# h, the FMA into y: 7 flops counting the exp as one) and one v_exp_f32.  A wave64 VALU op
# occupies a 16-lane SIMD for 4 cycles and a v_exp_f32 8 (`bench.py --valu-probe`, summarised in
# profiles/valu_issue_rates_probe.txt: the mix itself runs at ~24 cycles per 64 units), so 64
# units cost 4*4 + 8 = 24 SIMD cycles: the issue-limited peak of this instruction mix (extra).
FLOPS_PER_STATE_STEP = 7
MIX_PEAK_TFLOPS = SIMDS * CLOCK_HZ * 64 / 24 * FLOPS_PER_STATE_STEP / 1e12
# The backward scan per (element, state), from the gradient formulas: the forward recompute
# (mul, exp, mul, fma: 5 flops), the adjoint (mul + exp for the decay, fma into lambda, two
# muls for lambda a h, fmas into dA, ddelta and <lambda, B>, the decayed adjoint: 13 flops),
# the dB and dC terms (2 muls) and their sums over the channels (2 adds): 22 flops.
BWD_FLOPS_PER_STATE_STEP = 22
FP32_MFMA_PEAK_TFLOPS = 157.3  # dense fp32 matrix-core peak of the MI355X
MALL_BYTES = 256 << 20
COPY_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=1,
                    help="workload: 0 tiny, 1 SS2D stage-1 (default), 2 stage-3, 3 low-state, 4 high-res, 5 Vim-Tiny")
    ap.add_argument("--bwd", action="store_true", help="time forward + backward per step")
    ap.add_argument("--front", type=int, default=0,
                    help="SS2D only: K > 0 adds the input front (depthwise K x K convolution + SiLU)")
    ap.add_argument("--ln", action="store_true",
                    help="SS2D only: LayerNorm over the channels of the merged map before the gate")
    ap.add_argument("--proj", type=int, default=0,
                    help="SS2D only: R > 0 produces delta/B/C from per-route x_proj/dt_proj (dt_rank R)")
    ap.add_argument("--valu-probe", action="store_true",
                    help="instead of the benchmark: measure the SIMD cycles of a wave64 FMA, a v_exp_f32 and the "
                         "scan's per-(element, state) instruction mix (libss2d_probe.so) and print them as JSON")
    ap.add_argument("--summarize", metavar="DIR",
                    help="instead of the benchmark: render the rocprofv3 CSV output under DIR (kernel stats and/or "
                         "counter collection) as the text summaries kept in profiles/")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=30.0,
                    help="oracle wall-time budget: the whole batch when its estimate fits, else the first images")
    ap.add_argument("--no-train-step", action="store_true",
                    help="SS2D forward workloads: skip the training-step record (forward with states + backward)")
    return ap.parse_args()


def front_bytes(cfg, bwd=False):
    """The input front's own minimum: the forward reads x and writes the fp32 front output in
    grid and column-major order; the backward reads x and the fp32 gradient of the front output
    and writes dx (the filter partial sums are 200 bytes per plane)."""
    e = 2 if cfg.dtype == "bf16" else 4
    grid = cfg.batch * cfg.dim * cfg.seqlen
    return (e + 8) * grid + ((2 * e + 4) * grid if bwd else 0)


def proj_flops(cfg, R):
    """Multiply-adds x 2 of the Δ/B/C producer's matrix-core products per forward: x_proj (R + 2N
    rows) per route and pixel, and dt_proj when its rank exceeds 16 (up to 16 the route scans form
    the raw delta themselves, on the vector units)."""
    tokens = 4 * cfg.batch * cfg.seqlen
    return 2 * tokens * ((R + 2 * cfg.dstate) * cfg.dim + (cfg.dim * R if R > 16 else 0))


def algorithmic_bytes(cfg, bwd=False, proj=False):
    """Each tensor read once and each output written once (the fused minimum).  With the Δ/B/C
    producer, delta, B and C are not inputs (nor their gradients outputs)."""
    e = 2 if cfg.dtype == "bf16" else 4
    if proj and getattr(cfg, "kind", "ss2d") != "vim":
        grid = cfg.batch * cfg.dim * cfg.seqlen
        z = grid if cfg.has_z else 0
        fwd = e * (grid + z + grid)
        return fwd + (e * (grid + grid + z + grid + z) if bwd else 0)
    if getattr(cfg, "kind", "ss2d") == "vim":
        seq = cfg.batch * cfg.dim * cfg.seqlen  # one direction, or the gate / output sequence
        bc = 2 * cfg.batch * 2 * cfg.dstate * cfg.seqlen
        fwd = e * (2 * seq + 2 * seq + bc + (seq if cfg.has_z else 0) + seq)  # u, delta, B/C, z in; out
        if not bwd:
            return fwd
        # backward: reads u, delta, B, C, z, dout; writes du, ddelta, dB, dC, dz
        return fwd + e * (seq + 2 * seq + 2 * seq + bc + (seq if cfg.has_z else 0))
    grid = cfg.batch * cfg.dim * cfg.seqlen
    seq = cfg.batch * 4 * cfg.dim * cfg.seqlen
    bc = 2 * cfg.batch * 4 * cfg.dstate * cfg.seqlen
    fwd = e * (grid + seq + bc + (grid if cfg.has_z else 0) + grid)
    if not bwd:
        return fwd
    # backward: reads x, delta, B, C, z, dout; writes dx, ddelta, dB, dC, dz
    return fwd + e * (grid + grid + seq + bc + (grid if cfg.has_z else 0))


def scan_kernel_source_hash():
    h = hashlib.sha256()
    for name in ("scan_fwd_kernel.h", "scan_common.h", "device_common.h", "internal.h"):
        with open(os.path.join(ROOT, "selective_scan_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def plane_kernel_source_hash():
    h = hashlib.sha256()
    for name in ("plane_fwd.hip", "plane_fwd.h", "device_common.h"):
        with open(os.path.join(ROOT, "selective_scan_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(key, sha):
    """HBM traffic of the dominant kernel from the committed rocprofv3 counter summary, or None
    when that summary was taken on a different version of the kernel source."""
    path = os.path.join(ROOT, "profiles", "scan_fwd_traffic.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    entry = rec.get(key)
    if not entry or entry.get("kernel_source_sha") != sha:
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, target_s, bwd=False, front=None, ln=None, proj=None):
    """The fp64 oracle (as it stands) on the first images of the same batch (forward, or
    forward + backward when the GPU step includes the backward)."""
    import oracle
    from selective_scan_amd import synth

    vim = getattr(cfg, "kind", "ss2d") == "vim"

    def run_vim(nb):
        sl = lambda a: None if a is None else synth.storage_to_f64(a[:nb], cfg.dtype)
        args = (sl(inp["u"]), sl(inp["delta"]), inp["A"].astype(np.float64), sl(inp["B"]), sl(inp["C"]),
                inp["D"].astype(np.float64), inp["delta_bias"].astype(np.float64), sl(inp["z"]))
        t0 = time.perf_counter()
        oracle.vim_bidir_fwd(*args)
        if bwd:
            oracle.vim_bidir_bwd(*args, dout=sl(inp["dout"]))
        return time.perf_counter() - t0

    def run(nb):
        if vim:
            return run_vim(nb)
        sl = lambda a: None if a is None else synth.storage_to_f64(a[:nb], cfg.dtype)
        args = (sl(inp["x"]), sl(inp["delta"]), inp["A"].astype(np.float64), sl(inp["B"]), sl(inp["C"]),
                inp["D"].astype(np.float64), inp["delta_bias"].astype(np.float64), sl(inp["z"]))
        t0 = time.perf_counter()
        if proj is not None:
            kw = dict(x_proj_w=proj["x_proj_w"].astype(np.float64), dt_proj_w=proj["dt_proj_w"].astype(np.float64),
                      A=args[2], D=args[5], delta_bias=args[6], z=args[7])
            if front is not None:
                kw.update(conv_w=front["conv_w"].astype(np.float64), conv_b=front["conv_b"].astype(np.float64))
            if ln is not None:
                kw.update(layer_norm=True, ln_w=ln["ln_w"].astype(np.float64), ln_b=ln["ln_b"].astype(np.float64))
            oracle.ss2d_proj_fwd(args[0], **kw)
            if bwd:
                oracle.ss2d_proj_bwd(args[0], **kw, dout=sl(inp["dout"]))
        elif ln is not None:
            kw = dict(ln_w=ln["ln_w"].astype(np.float64), ln_b=ln["ln_b"].astype(np.float64))
            if front is not None:
                kw.update(conv_w=front["conv_w"].astype(np.float64), conv_b=front["conv_b"].astype(np.float64))
            oracle.ss2d_ln_fwd(*args, **kw)
            if bwd:
                oracle.ss2d_ln_bwd(*args, **kw, dout=sl(inp["dout"]))
        elif front is not None:
            fa = (args[0], front["conv_w"].astype(np.float64), front["conv_b"].astype(np.float64)) + args[1:]
            oracle.ss2d_front_fwd(*fa)
            if bwd:
                oracle.ss2d_front_bwd(*fa, dout=sl(inp["dout"]))
        else:
            oracle.ss2d_fwd(*args)
            if bwd:
                oracle.ss2d_bwd(*args, dout=sl(inp["dout"]))
        return time.perf_counter() - t0

    t1 = run(1)
    # the whole batch when it fits the time target (the default covers every workload's forward)
    nb = int(max(1, min(cfg.batch, math.floor(target_s / max(t1, 1e-3)))))
    t = run(nb) if nb > 1 else t1
    routes = 2 if vim else 4
    elems = nb * routes * cfg.dim * cfg.seqlen
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    single = single_thread_runs() if proj is None and front is None and ln is None and not bwd else None
    return {"value": elems / t, "unit": "elements/s", "cores": threads, "kind": "oracle", "single_thread": single,
            "sample": f"first {nb} of {cfg.batch} {'sequences' if vim else 'images'} (all {cfg.dim} channels, "
                      f"{routes} {'directions' if vim else 'routes'}, L={cfg.seqlen}, N={cfg.dstate}), fp64 C "
                      f"oracle with OpenMP over rows{', with the input front' if front is not None else ''}"
                      f"{', with the LayerNorm' if ln is not None else ''}"
                      f"{', with the delta/B/C producer' if proj is not None else ''}, "
                      f"{'forward + backward' if bwd else 'forward'}, {t:.2f} s wall",
            "cpu_model": cpu_model()}


def single_thread_runs():
    """The oracle's SS2D forward on one core: the tiny workload whole, and the first image of the
    stage-3 workload (the first image of each seeded tensor is the start of its stream, so a
    one-image draw is that image)."""
    import oracle
    from selective_scan_amd import synth

    out = []
    prev = oracle.set_num_threads(1)
    try:
        for cfg in (synth.TINY, synth.STAGE3):
            inp = synth.make_ss2d_inputs(1, cfg.height, cfg.width, cfg.dim, cfg.dstate, cfg.dtype, cfg.has_z,
                                         cfg.index, params="s4d")
            f = lambda a: None if a is None else synth.storage_to_f64(a, cfg.dtype)
            args = (f(inp["x"]), f(inp["delta"]), inp["A"].astype(np.float64), f(inp["B"]), f(inp["C"]),
                    inp["D"].astype(np.float64), inp["delta_bias"].astype(np.float64), f(inp["z"]))
            t0 = time.perf_counter()
            oracle.ss2d_fwd(*args)
            ts = time.perf_counter() - t0
            out.append({"workload": cfg.name, "value": 4 * cfg.dim * cfg.seqlen / ts, "unit": "elements/s",
                        "cores": 1, "sample": f"{'the whole batch' if cfg.batch == 1 else 'first image'}, forward, "
                                              f"{ts * 1e3:.2f} ms wall"})
    finally:
        oracle.set_num_threads(prev)
    return out


def train_step_record(cfg, ss, synth, d0, stream, steps, warmup):
    """One training step of the SS2D op: ss2d_fwd keeping its checkpoint states, then ss2d_bwd on
    them (seeded dout ~ N(0, 1)); HIP events on the launch stream around each half.  The backward's
    arithmetic roofline counts BWD_FLOPS_PER_STATE_STEP per (element, state) over the whole
    ss2d_bwd call (its scan kernel and the small gate, reduce and merge kernels around it)."""
    import torch

    rng = np.random.Generator(np.random.PCG64(1000 * cfg.index + synth.T_DOUT))
    g = rng.standard_normal(size=(cfg.batch, cfg.dim, cfg.height, cfg.width), dtype=np.float32)
    if cfg.dtype == "bf16":
        dout = torch.from_numpy(synth.f32_to_bf16_bits(g).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        dout = torch.from_numpy(g).cuda()
    del g
    plan = ss.SS2DForwardPlan(**d0, keep_states=True)

    def one(ev=None):
        if ev is not None:
            ev[0].record(stream)
        for stage in (0, 1, 2):
            plan.run_stage(stage)
        if ev is not None:
            ev[1].record(stream)
        ss.ss2d_bwd(**d0, dout=dout, workspace=plan.workspace, workspace_has_states=True)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        one(evs[i])
    torch.cuda.synchronize()
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    del plan, dout
    torch.cuda.empty_cache()
    bflops = cfg.elements * cfg.dstate * BWD_FLOPS_PER_STATE_STEP
    b_ms = float(np.median(bwd_ms))
    return {"what": "ss2d_fwd with keep_states + ss2d_bwd on its states, same inputs, dout ~ N(0,1)",
            "ms": stats(step_ms), "elements_per_s": cfg.elements / (float(np.median(step_ms)) * 1e-3),
            "fwd_keep_states_ms": stats(fwd_ms), "bwd_ms": stats(bwd_ms),
            "bwd_roofline": {"kernel": "ss2d_bwd (scan_bwd_kernel with its gate, reduce and merge kernels)",
                             "bound": "alu", "achieved": bflops / (b_ms * 1e-3) / 1e12,
                             "peak": PUBLISHED_FP32_VECTOR_TFLOPS, "unit": "TFLOP/s",
                             "frac": bflops / (b_ms * 1e-3) / 1e12 / PUBLISHED_FP32_VECTOR_TFLOPS,
                             "flops_per_unit": BWD_FLOPS_PER_STATE_STEP, "units": cfg.elements * cfg.dstate}}


def config_record(cfg, vim, bwd, n_sets, front_k=0, ln=False, proj_r=0):
    if vim:
        return {"workload": ("vim_bidir_fwd+bwd " if bwd else "vim_bidir_fwd ") + cfg.name, "batch": cfg.batch,
                "seqlen": cfg.seqlen, "directions": 2, "dim": cfg.dim, "dstate": cfg.dstate, "gate_z": cfg.has_z,
                "io_sets_rotated": n_sets}
    rec = {"workload": ("ss2d_fwd+bwd " if bwd else "ss2d_fwd ") + cfg.name, "batch": cfg.batch,
           "height": cfg.height, "width": cfg.width, "routes": 4, "dim": cfg.dim, "dstate": cfg.dstate,
           "gate_z": cfg.has_z, "io_sets_rotated": n_sets}
    if front_k:
        rec["workload"] = rec["workload"].replace("ss2d_fwd", f"ss2d_fwd(front dwconv{front_k}x{front_k}+silu)", 1)
        rec["front_conv_k"] = front_k
    if ln:
        rec["workload"] = rec["workload"].replace(" " + cfg.name, "(+layernorm) " + cfg.name, 1)
        rec["layer_norm"] = True
    if proj_r:
        rec["workload"] = rec["workload"].replace(" " + cfg.name, f"(+x_proj/dt_proj R={proj_r}) " + cfg.name, 1)
        rec["dt_rank"] = proj_r
    return rec


def stats(ms):
    return {"median": float(np.median(ms)), "min": float(np.min(ms)), "max": float(np.max(ms)),
            "mean": float(np.mean(ms))}


SES = 32  # shader engines (8 XCDs x 4); SQ_BUSY_CYCLES sums one count per engine
CALIB_COPY_BYTES = 1 << 30  # the device copy bench.py runs after its timed steps


def summarize(dirname):
    """Text summary of rocprofv3 CSV output (the rule profiles/ is rendered by).

    *_kernel_stats.csv (--kernel-trace --stats): calls and average / min / max duration per kernel.
    *_counter_collection.csv (--pmc): per kernel, the mean over its dispatches of each counter (the
    CSV holds one row per dispatch and counter; values summed over the device).  Derived, when the
    counters are present:
      * kernel cycles = SQ_BUSY_CYCLES / 32 (one count per shader engine while the kernel runs);
      * VALU busy per SIMD = 4 SQ_ACTIVE_INST_VALU / (1024 x kernel cycles): SQ_ACTIVE_INST_VALU
        counts quad-cycles of VALU issue (one per wave64 instruction, two per transcendental:
        SQ_INSTS_VALU + SQ_INSTS_VALU_TRANS_F32 equals it), summed over all wavefronts;
      * VALU instructions per wavefront = SQ_INSTS_VALU / SQ_WAVES;
      * LDS bank conflicts per LDS instruction = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS (both in
        cycles of the LDS pipe);
      * HBM bytes = FETCH_SIZE and WRITE_SIZE (KiB per dispatch) times the factors that make the
        1 GiB device copy of the same run (the copy kernel's largest dispatch) read and write 1 GiB."""
    import csv
    import glob as _glob

    out = []
    for path in sorted(_glob.glob(os.path.join(dirname, "**", "*kernel_stats.csv"), recursive=True)):
        out.append(f"# kernel stats: {os.path.relpath(path, dirname)}")
        out.append(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}  kernel")
        with open(path) as f:
            rows = list(csv.DictReader(f))
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
            out.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} {float(r['MinNs']) / 1e3:10.1f} "
                       f"{float(r['MaxNs']) / 1e3:10.1f}  {r['Name'][:160]}")
    for path in sorted(_glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True)):
        out.append(f"# counters: {os.path.relpath(path, dirname)}")
        per = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                k = (r["Kernel_Name"], r["Counter_Name"])
                per.setdefault(k, {}).setdefault(r["Dispatch_Id"], 0.0)
                per[k][r["Dispatch_Id"]] += float(r["Counter_Value"])
        kernels = {}
        for (kn, cn), d in per.items():
            kernels.setdefault(kn, {})[cn] = sum(d.values()) / len(d)
        copy_name = next((k for k in kernels if "copy" in k.lower()), None)
        fr = wr = None
        if copy_name:
            # the 1 GiB copies are the copy kernel's largest dispatches (the program makes small
            # device copies too)
            big = lambda cn: max(per[(copy_name, cn)].values()) if (copy_name, cn) in per else 0.0
            if big("FETCH_SIZE"):
                fr = CALIB_COPY_BYTES / (big("FETCH_SIZE") * 1024)
            if big("WRITE_SIZE"):
                wr = CALIB_COPY_BYTES / (big("WRITE_SIZE") * 1024)
            out.append(f"calibration ({copy_name[:60]}): FETCH_SIZE x {fr if fr else float('nan'):.3f}, "
                       f"WRITE_SIZE x {wr if wr else float('nan'):.3f}")
        for kn, c in sorted(kernels.items()):
            out.append(kn[:200])
            for cn in sorted(c):
                out.append(f"  {cn:30s} {c[cn]:12.4g}")
            if "SQ_BUSY_CYCLES" in c:
                cyc = c["SQ_BUSY_CYCLES"] / SES
                out.append(f"  {'kernel cycles (derived)':30s} {cyc:12.4g}")
                if "SQ_ACTIVE_INST_VALU" in c:
                    out.append(f"  {'VALU busy per SIMD (derived)':30s} {4 * c['SQ_ACTIVE_INST_VALU'] / (SIMDS * cyc):12.3f}")
            if "SQ_INSTS_VALU" in c and c.get("SQ_WAVES"):
                out.append(f"  {'VALU instr per wave (derived)':30s} {c['SQ_INSTS_VALU'] / c['SQ_WAVES']:12.4g}")
            if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_ACTIVE_INST_LDS"):
                out.append(f"  {'bank conflict / LDS (derived)':30s} {c['SQ_LDS_BANK_CONFLICT'] / c['SQ_ACTIVE_INST_LDS']:12.3f}")
            if fr and "FETCH_SIZE" in c:
                out.append(f"  {'HBM read bytes (derived)':30s} {c['FETCH_SIZE'] * 1024 * fr:12.4g}")
            if wr and "WRITE_SIZE" in c:
                out.append(f"  {'HBM write bytes (derived)':30s} {c['WRITE_SIZE'] * 1024 * wr:12.4g}")
    print("\n".join(out))


def valu_probe():
    """Issue rates of the vector unit, from the probe kernels' own clock stamps: per wavefront the
    shader-clock and 100 MHz real-time counters around a loop of independent chains; with k
    wavefronts per SIMD, cycles per instruction (one SIMD) = wavefront cycles / (k x instructions of
    the wavefront).  Kinds: 0 FMA, 1 v_exp_f32, 2 the scan's mix per (element, state)."""
    import ctypes

    import torch

    path = os.path.join(ROOT, "selective_scan_amd", "libss2d_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    lib.valu_probe_run.restype = ctypes.c_int
    lib.valu_probe_run.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.valu_probe_insts_per_iter.restype = ctypes.c_int
    lib.valu_probe_insts_per_iter.argtypes = [ctypes.c_int]
    stream = torch.cuda.current_stream()
    res = {"what": "SIMD cycles per wave64 instruction (FMA, v_exp_f32) and per 64 (element, state) units of "
                   "the scan's mix (v_mul, v_exp_f32, v_mul, v_fma, v_fma per unit, plus one v_fma per 8 units), "
                   "median over wavefronts, k wavefronts per SIMD", "runs": []}
    names = {0: "fma", 1: "exp", 2: "scan_mix"}
    for kind in (0, 1, 2):
        ipi = lib.valu_probe_insts_per_iter(kind)
        for k in (1, 2, 3):
            waves = SIMDS * k
            iters = 20000 if kind != 1 else 10000
            stamps = torch.zeros(4 * waves, dtype=torch.int64, device="cuda")
            sink = torch.empty(64 * waves, dtype=torch.float32, device="cuda")
            for _ in range(2):  # the first launch warms the clocks up
                st = lib.valu_probe_run(kind, waves, iters, ctypes.c_void_p(stamps.data_ptr()),
                                        ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
                if st != 0:
                    raise RuntimeError(f"valu_probe_run status {st}")
                torch.cuda.synchronize()
            t = stamps.view(-1, 4).cpu().numpy().astype(np.float64)
            cyc = t[:, 1] - t[:, 0]
            sec = (t[:, 3] - t[:, 2]) / 100e6
            clock = float(np.median(cyc / sec))
            # the whole launch, first wavefront start to last wavefront end (real-time counter),
            # in cycles of the median clock: SIMD cycles for k * iters * ipi instructions per SIMD
            span = (t[:, 3].max() - t[:, 2].min()) / 100e6 * clock
            rec = {"kind": names[kind], "waves_per_simd": k, "clock_GHz": clock / 1e9,
                   "launch_us": float((t[:, 3].max() - t[:, 2].min()) / 100.0),
                   "cycles_per_instruction": float(span / (k * iters * ipi)),
                   "wave_cycles_per_instruction": float(np.median(cyc) / (iters * ipi))}
            if kind == 2:
                units = iters * 64  # (element, state) units per lane and wavefront
                rec["cycles_per_64_units"] = float(span / (k * units))
            res["runs"].append(rec)
    print(json.dumps(res))


def main():
    args = parse()
    if args.valu_probe:
        valu_probe()
        return
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); every box here has a single "
              f"MI355X and no multi-GPU path is part of this library.", file=sys.stderr)
        sys.exit(2)
    import torch

    import selective_scan_amd as ss
    from selective_scan_amd import synth

    workloads = list(synth.WORKLOADS) + list(synth.VIM_WORKLOADS)
    cfg = workloads[args.workload]
    vim = getattr(cfg, "kind", "ss2d") == "vim"
    if (args.front or args.ln or args.proj) and vim:
        print("--front, --ln and --proj apply to the SS2D workloads only", file=sys.stderr)
        sys.exit(2)
    inp = (synth.make_vim_config_inputs if vim else synth.make_config_inputs)(cfg, with_dout=args.bwd)
    front = synth.make_front_params(cfg.dim, args.front, seed_base=cfg.index) if args.front else None
    ln = synth.make_ln_params(cfg.dim, seed_base=cfg.index) if args.ln else None
    proj = synth.make_proj_params(cfg.dim, cfg.dstate, args.proj, seed_base=cfg.index) if args.proj else None

    def dev(a, dtype):
        if a is None:
            return None
        if dtype == "bf16" and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    first = "u" if vim else "x"
    d0 = {first: dev(inp[first], cfg.dtype), "delta": dev(inp["delta"], cfg.dtype), "A": dev(inp["A"], "f32"),
          "B": dev(inp["B"], cfg.dtype), "C": dev(inp["C"], cfg.dtype), "D": dev(inp["D"], "f32"),
          "delta_bias": dev(inp["delta_bias"], "f32"), "z": dev(inp["z"], cfg.dtype) if cfg.has_z else None}
    if front is not None:
        d0.update(conv_w=dev(front["conv_w"], "f32"), conv_b=dev(front["conv_b"], "f32"))
    if ln is not None:
        d0.update(ln_w=dev(ln["ln_w"], "f32"), ln_b=dev(ln["ln_b"], "f32"))
    if proj is not None:
        d0.update(delta=None, B=None, C=None, x_proj_w=dev(proj["x_proj_w"], "f32"),
                  dt_proj_w=dev(proj["dt_proj_w"], "f32"))
    dout0 = dev(inp["dout"], cfg.dtype) if args.bwd else None
    # with --bwd a step is a training step: the forward keeps its checkpoint states and the
    # backward runs on them
    if vim:
        Plan = (lambda **kw: ss.VimForwardPlan(**kw, keep_states=True)) if args.bwd else ss.VimForwardPlan
        backward = (lambda **kw: ss.vim_bidir_bwd(**kw, workspace_has_states=True))
    else:
        Plan = (lambda **kw: ss.SS2DForwardPlan(**kw, keep_states=True)) if args.bwd else ss.SS2DForwardPlan
        backward = (lambda **kw: ss.ss2d_bwd(**kw, workspace_has_states=True))
    plan0 = Plan(**d0)
    single = (not vim) and plan0.single_kernel  # the forward runs as one kernel per plane (small state sizes)
    # bytes one step touches in HBM (inputs, output, workspace): rotate independent copies
    # until one cycle over them exceeds three times the MALL
    footprint = sum(t.numel() * t.element_size() for t in d0.values() if t is not None)
    footprint += plan0.out.numel() * plan0.out.element_size() + plan0.workspace.numel()
    n_sets = max(1, math.ceil(3 * MALL_BYTES / footprint))
    sets = [(d0, dout0, plan0)]
    for _ in range(n_sets - 1):
        dk = {k: (None if v is None else v.clone()) for k, v in d0.items()}
        sets.append((dk, None if dout0 is None else dout0.clone(), Plan(**dk)))
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        d, dout, plan = sets[i % n_sets]
        if single:
            if ev is not None:
                ev[0].record(stream)
                ev[1].record(stream)
            plan.run()
            if ev is not None:
                ev[2].record(stream)
                ev[3].record(stream)
            return
        if ev is not None:
            ev[0].record(stream)
        plan.run_stage(0)
        if ev is not None:
            ev[1].record(stream)
        plan.run_stage(1)
        if ev is not None:
            ev[2].record(stream)
        plan.run_stage(2)
        if args.bwd:
            backward(**d, dout=dout, workspace=plan.workspace)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(i, evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps
    step_ms = [e[0].elapsed_time(e[3]) for e in evs]
    scan_ms = [e[1].elapsed_time(e[2]) for e in evs]
    stage0_ms = [e[0].elapsed_time(e[1]) for e in evs]

    # the training step on the same inputs (forward keeping its states, then the backward on them)
    train = None
    if not vim and not args.bwd and not args.no_train_step and proj is None and front is None and ln is None:
        train = train_step_record(cfg, ss, synth, d0, stream, max(3, args.steps // 2), 2)
    # a plain device copy of known size in the same run: the practical HBM ceiling (its three
    # dispatches also calibrate the byte counters of a profiler run of this program)
    del sets, d0, plan0, dout0
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    copy_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(3)]
    for a, b in copy_ev:
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * COPY_BYTES / (np.median([a.elapsed_time(b) for a, b in copy_ev]) * 1e-3) / 1e9

    elements = cfg.elements
    step_bytes = algorithmic_bytes(cfg, args.bwd, proj is not None) + (front_bytes(cfg, args.bwd) if front is not None else 0)
    flops = elements * cfg.dstate * FLOPS_PER_STATE_STEP
    scan_mean = float(np.mean(scan_ms))
    achieved_tflops = flops / (scan_mean * 1e-3) / 1e12
    traffic = load_traffic(cfg.name, scan_kernel_source_hash())
    hbm_gbps = step_bytes / (ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": elements / (ms * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) inputs, S4D-real A, inverse-softplus dt bias)",
        "config": config_record(cfg, vim, args.bwd, n_sets, args.front, args.ln, args.proj),
        "step_ms": stats(step_ms),
        "hbm": {"algorithmic_bytes_per_step": step_bytes,
                "achieved_GBps": hbm_gbps,
                "peak_GBps": HBM_PEAK_GBPS,
                "frac": hbm_gbps / HBM_PEAK_GBPS,
                "copy_ceiling_GBps": copy_gbps,
                "frac_of_copy": hbm_gbps / copy_gbps},
        "roofline": {"kernel": ("direction" if vim else "route") + " scan (scan_fwd_kernel)", "bound": "alu",
                     "achieved": achieved_tflops, "peak": PUBLISHED_FP32_VECTOR_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved_tflops / PUBLISHED_FP32_VECTOR_TFLOPS, "traffic": traffic,
                     "flops_per_unit": FLOPS_PER_STATE_STEP, "units_per_launch": elements * cfg.dstate,
                     "unpacked_fp32_peak": VALU_PEAK_TFLOPS, "frac_of_unpacked_peak": achieved_tflops / VALU_PEAK_TFLOPS,
                     "mix_peak": MIX_PEAK_TFLOPS, "frac_of_mix_peak": achieved_tflops / MIX_PEAK_TFLOPS,
                     "ms_per_launch": scan_mean, "launch_ms": stats(scan_ms), "flops_per_launch": flops},
    }
    if single:
        # one kernel moves exactly the fused minimum: x, delta, B, C (and z) in, out written
        gbps = step_bytes / (scan_mean * 1e-3) / 1e9
        res["roofline"] = {"kernel": "plane_fwd_kernel (cross-scan, the four route scans and the cross-merge; "
                                     "one workgroup per plane)", "bound": "hbm",
                           "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                           "traffic": load_traffic(cfg.name + ":plane", plane_kernel_source_hash()),
                           "frac_of_copy": gbps / copy_gbps, "ms_per_launch": scan_mean,
                           "launch_ms": stats(scan_ms), "bytes_per_launch": step_bytes,
                           # what the counters show limiting it (profiles/sq_counters_ss2d_fwd_lowstate_56x56_b128_d96_n1_bf16_noz.txt):
                           # VALU issue (softplus, decay and the two scan passes, ~27 instructions per
                           # route step), not HBM
                           "limiter": "valu"}
    if front is not None:
        fb = front_bytes(cfg, False)
        f_ms = float(np.mean(stage0_ms))
        res["front"] = {"kernel": "front_fwd_kernel (stage 0)", "bound": "hbm", "ms_per_launch": f_ms,
                        "launch_ms": stats(stage0_ms), "algorithmic_bytes": fb,
                        "achieved_GBps": fb / (f_ms * 1e-3) / 1e9, "peak_GBps": HBM_PEAK_GBPS,
                        "frac": fb / (f_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    if proj is not None:
        pf = proj_flops(cfg, args.proj)
        s_ms = float(np.mean(stage0_ms))
        res["producer"] = {"kernel": "proj_kernel (v_mfma_f32_32x32x2f32, routes k and k+2 per tile); "
                                     "stage 0 also writes the fp32 copies of the map",
                           "bound": "mfma", "flops_per_step": pf, "stage0_ms": s_ms, "launch_ms": stats(stage0_ms),
                           "achieved_TFLOPs": pf / (s_ms * 1e-3) / 1e12, "peak_TFLOPs": FP32_MFMA_PEAK_TFLOPS,
                           "frac": pf / (s_ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS}
    if train is not None:
        res["train_step"] = train
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds, args.bwd, front, ln, proj)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
