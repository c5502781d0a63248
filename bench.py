"""Benchmark of the selective scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one full pass of the hot path over one batch: one selective-scan call
over the whole [batch, D, L] workload (softplus, discretisation, scan, readout,
skip, gate, final state), or for the decode workload one state-update call.
Inputs are synthetic and seeded (synth/), resident in HBM before timing.  Each
step reads a different copy of the inputs (enough copies to exceed the 256 MB
Infinity Cache), so every step streams its inputs from HBM.  The K steps are
captured in one HIP graph.  Before timing, the graph is replayed until at least
W steps and at least 100 ms of sustained load have run (over the first ~10 ms of
load the scan runs ~15 % slower while the clock ramps); the JSON reports the
warm-up steps actually run.  The timed region is one replay of the K steps
between two synchronisations; then 50 more replays, each bracketed by HIP events,
give the median, p10 and p90 per step.

The default workload is the largest of the five named configurations (the
131072-token scan, 2.69 GB per call); the other four are timed the same way and
reported under "workloads".  The JSON line carries:
  * value: elements/s (B*L*D*N per second) of the timed region;
  * roofline: algorithmic HBM bytes / average call time against 8 TB/s, with the
    VALU-slot figure (4 fp32 ops + one exp2 at half rate per element against the
    single-issue fp32 peak) under "alu";
  * calibration: a plain streaming copy's bandwidth and the measured FMA and exp2
    issue rates (include/ssm_calib.h);
  * cpu_baseline: the float64 CPU oracle timed on this host's cores on a bounded
    sample of the same workload, with the core count and CPU model.
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

import synth  # noqa: E402

PEAK_HBM_GBS = 8000.0
PEAK_VALU_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12    # 39.32 T single-issue fp32 lane slots/s
ALU_SLOTS_PER_ELEMENT = 6                           # 4 fp32 ops + one exp2 at half rate
# Backward, per element (b, t, d, n): the forward recomputation (exp2 at half rate = 2,
# Delta*u*B, the state FMA, the readout FMA for the pre-gate output: 5 slots) and the
# adjoint (lam = g*C + abar*lam': 2; sum_n lam*B: 1; dB term lam*Delta*u and its sum
# over d: 2; dC term g*h and its sum: 2; abar*lam*h_{t-1}: 2, times A into dDelta: 1,
# times Delta into dA: 1; 11 slots).
BWD_ALU_SLOTS_PER_ELEMENT = 16
# Full zero-order hold: the input term (e^{Delta A} - 1)/A * B * u costs u/A*B (2 ops)
# and one FMA against the one multiply of Delta*u*B.
ZOH_ALU_SLOTS_PER_ELEMENT = 8
MALL_BYTES = 256 << 20
CALIB_BYTES = 1 << 30
DEFAULT_WORKLOAD = "long131k_bf16"
GRADED = ("tiny_f32", "mamba130m_f32", "mamba1p4b_bf16", "long131k_bf16", "decode_bf16")
# bfloat16 workloads whose A rows (-(n+1)) let the library's arithmetic-progression
# decay path run; bench.py times them both ways and reports that path separately
AP_WORKLOADS = ("mamba1p4b_bf16", "long131k_bf16")
MIN_WARM_S = 0.1
STAT_REPS = 50
_CSRC = "selective_state_space_68_amd/csrc/"
KERNEL_SRC = {"scan_chunked_kernel": _CSRC + "scan_chunked.hip", "scan_tokseq_kernel": _CSRC + "scan_tokseq.hip",
              "scan_sequential_kernel": _CSRC + "scan_sequential.hip",
              "state_update_vec_kernel": _CSRC + "state_update.hip", "ssd_scan_kernel": _CSRC + "ssd.hip"}
KERNEL_NAME = {"decode": "state_update_vec_kernel",
               "bwd": "scan backward call (bwd_summary, bwd_combine, bwd_main, bwd_param_sums, bwd_bc_out kernels)",
               "bwd_saved": "scan backward call with saved chunk states (bwd_main chunk walk, bwd_param_sums, "
                            "bwd_bc_out kernels)",
               "train": "training pair: the forward scan saving chunk states, then the backward from them",
               "ssd": "ssd_scan_kernel"}
KERNEL_SRC[KERNEL_NAME["bwd"]] = _CSRC + "scan_bwd.hip"
KERNEL_SRC[KERNEL_NAME["bwd_saved"]] = _CSRC + "scan_bwd.hip"
KERNEL_SRC[KERNEL_NAME["train"]] = _CSRC + "scan_bwd.hip"
PEAK_MFMA_BF16_TFLOPS = 2500.0


def kernel_of(cfg, kind, variant=0, tokens_per_lane=0):
    """The kernel (or, for the backward, the call) a workload's timed region runs.
    The forward scan asks the library which kernel it picks for the shape."""
    if kind == "bwd" and cfg.saved:
        return KERNEL_NAME["train" if cfg.train else "bwd_saved"]
    if kind != "scan":
        return KERNEL_NAME[kind]
    import torch
    from selective_state_space_68_amd import selective_scan_fwd_kernel
    dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    return selective_scan_fwd_kernel(cfg.batch, cfg.L, cfg.D, cfg.N, dtype, cfg.gate, cfg.discretization,
                                     cfg.conv_k, variant, tokens_per_lane)


def src_hash(kernel):
    h = hashlib.sha256()
    for p in (KERNEL_SRC[kernel], "selective_state_space_68_amd/csrc/device_common.hpp"):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summaries
    (profile_summary.py writes them), or None when the kernel source changed since
    the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("source_hash") != src_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(a.astype(np.float32, copy=False)).to("cuda")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


# ---------------------------------------------------------------------------- CPU oracle

def _oracle_shard(args):
    """Worker: the oracle (forward, or backward when an output gradient is given) on one
    (batch row, channel block, token prefix) shard; returns seconds."""
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    import oracle
    (u, delta, A, B, C, Dk, z, bias, sp, dy, disc) = args
    t0 = time.perf_counter()
    if dy is None:
        oracle.selective_scan(u, delta, A, B, C, Dk, z, bias, sp, discretization=disc)
    else:
        oracle.selective_scan_bwd(u, delta, A, B, C, dy, Dk, z, bias, sp)
    return time.perf_counter() - t0


def _oracle_warm(_):
    import oracle  # noqa: F401
    return 0


def cpu_baseline_scan(cfg, inp, budget_s=20.0, workers=0, dy=None):
    """The float64 oracle, as it is, timed on this host's cores on a bounded sample: the
    first L_s tokens (a prefix of every sequence is itself a scan) of as many whole
    batch rows as fit in about budget_s of CPU time, split into (batch row, channel
    block) shards run by a pool of worker processes, repeated for a stable time when
    one pass is short.  With `dy` the oracle's backward pass is timed."""
    import concurrent.futures as cf
    import multiprocessing as mp
    ncpu = len(os.sched_getaffinity(0))
    workers = workers or max(1, min(16, ncpu))
    sl = lambda x, b0, b1, d0, d1, t1: None if x is None else x[b0:b1, d0:d1, :t1]
    vec = lambda x, d0, d1: None if x is None else x[d0:d1]
    # probe: one worker's share of one batch row over a short prefix, in this process
    dblk = max(1, -(-cfg.D // workers))
    t_probe = min(cfg.L, 512)
    t0 = time.perf_counter()
    _oracle_shard((inp.u[:1, :dblk, :t_probe], inp.delta[:1, :dblk, :t_probe], inp.A[:dblk], inp.B[:1, :t_probe],
                   inp.C[:1, :t_probe], vec(inp.Dskip, 0, dblk), sl(inp.z, 0, 1, 0, dblk, t_probe),
                   vec(inp.delta_bias, 0, dblk), inp.delta_softplus, sl(dy, 0, 1, 0, dblk, t_probe),
                   cfg.discretization))
    per_tok_row_cpu = (time.perf_counter() - t0) / t_probe * -(-cfg.D // dblk)   # CPU s per token of one row
    row_cpu = per_tok_row_cpu * cfg.L
    if row_cpu <= budget_s:
        L_s = cfg.L
        b_take = max(1, min(cfg.batch, int(budget_s / max(row_cpu, 1e-6))))
    else:
        b_take = 1
        L_s = max(min(cfg.L, 512), min(cfg.L, int(budget_s / per_tok_row_cpu) // 512 * 512))
    shards = []
    for b in range(b_take):
        for d0 in range(0, cfg.D, dblk):
            d1 = min(cfg.D, d0 + dblk)
            shards.append((sl(inp.u, b, b + 1, d0, d1, L_s), sl(inp.delta, b, b + 1, d0, d1, L_s), inp.A[d0:d1],
                           inp.B[b:b + 1, :L_s], inp.C[b:b + 1, :L_s], vec(inp.Dskip, d0, d1),
                           sl(inp.z, b, b + 1, d0, d1, L_s), vec(inp.delta_bias, d0, d1), inp.delta_softplus,
                           sl(dy, b, b + 1, d0, d1, L_s), cfg.discretization))
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        list(ex.map(_oracle_warm, range(workers)))   # start the workers and import the oracle
        t0 = time.perf_counter()
        one = sum(ex.map(_oracle_shard, shards))       # one pass: sizes the repetition count
        reps = max(1, min(50, int(budget_s / max(one, 1e-3))))
        t0 = time.perf_counter()
        secs = list(ex.map(_oracle_shard, shards * reps))
        wall = time.perf_counter() - t0
    elems = b_take * L_s * cfg.D * cfg.N
    return {"value": reps * elems / wall, "unit": "elements/s", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{'backward, ' if dy is not None else ''}{cfg.discretization} discretization, "
                      f"{b_take} of {cfg.batch} batch rows x all {cfg.D} channels x the first {L_s} of L={cfg.L} "
                      f"tokens, N={cfg.N} ({elems:.3e} elements), {reps}x, in {len(shards)} shards per pass "
                      f"over {workers} worker processes (float64 numpy, 1 thread each; {wall:.1f} s wall, "
                      f"{sum(secs):.1f} s CPU); host has {ncpu} usable cores"}


def cpu_baseline_ssd(cfg, inp, budget_s=20.0):
    """The float64 SSD oracle, as it is, on one process: whole heads of one batch row,
    as many as fit in about budget_s."""
    import oracle
    t0 = time.perf_counter()
    oracle.ssd_scan(inp.x[:1, :, :1], inp.dt[:1, :, :1], inp.A[:1], inp.B[:1], inp.C[:1], inp.D[:1],
                    inp.dt_bias[:1])
    per_head = time.perf_counter() - t0
    heads = max(1, min(cfg.H, int(budget_s / max(per_head, 1e-3))))
    t0 = time.perf_counter()
    oracle.ssd_scan(inp.x[:1, :, :heads], inp.dt[:1, :, :heads], inp.A[:heads], inp.B[:1], inp.C[:1],
                    inp.D[:heads], inp.dt_bias[:heads])
    wall = time.perf_counter() - t0
    elems = cfg.L * heads * cfg.P * cfg.N
    return {"value": elems / wall, "unit": "elements/s", "cores": 1, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"SSD, 1 of {cfg.batch} batch rows x {heads} of {cfg.H} heads x full L={cfg.L}, "
                      f"P={cfg.P}, N={cfg.N} ({elems:.3e} elements), float64 numpy, one process, "
                      f"{wall:.1f} s"}


# ---------------------------------------------------------------------------- workloads

def kind_of(name):
    cfg = synth.CONFIGS[name]
    if isinstance(cfg, synth.SSDConfig):
        return "ssd"
    if isinstance(cfg, synth.DecodeConfig):
        return "decode"
    return "bwd" if cfg.backward else "scan"


def prepare(name, args, torch, lib_ops):
    """Inputs in HBM for workload `name`; returns (cfg, inp, kind, nbytes, elements, sets, step, bufs)."""
    kind = kind_of(name)
    cfg = synth.CONFIGS[name]
    if kind == "decode":
        S, D, N = cfg.batch, cfg.D, cfg.N
        A, Dk, bias = (dev(torch, x) for x in synth.make_decode_params(S, D, N, seed=cfg.seed))
        nbytes = cfg.algorithmic_bytes_per_step()
        sets = args.sets or max(2, int(np.ceil(600e6 / nbytes)))
        st0 = synth.make_decode_state(S, D, N, seed=cfg.seed)
        bufs = []
        for i in range(sets):
            x = synth.make_decode_step(S, D, N, i, cfg.dtype, cfg.gate, seed=cfg.seed)
            t = {k: dev(torch, x.dev[k]) for k in ("u", "delta", "B", "C", "z")}
            t["state"] = dev(torch, st0)
            t["y"] = torch.empty((S, D), dtype=t["u"].dtype, device="cuda")
            bufs.append(t)

        def step(i):
            t = bufs[i % sets]
            lib_ops.state_update(t["state"], t["u"], t["delta"], A, t["B"], t["C"], Dk, t["z"], bias, True,
                                 y=t["y"])
        return cfg, None, kind, nbytes, cfg.elements_per_step, sets, step, bufs

    if kind == "ssd":
        inp = synth.make_ssd_inputs(cfg.batch, cfg.L, cfg.H, cfg.P, cfg.N, cfg.dtype, seed=cfg.seed)
        nbytes = cfg.algorithmic_bytes()
        sets = args.sets or max(2, int(np.ceil(600e6 / nbytes)))
        A, Dk, bias = dev(torch, inp.A), dev(torch, inp.D), dev(torch, inp.dt_bias)
        bufs = []
        for _ in range(sets):
            t = {k: dev(torch, inp.dev[k]) for k in ("x", "dt", "B", "C")}
            t["y"] = torch.empty_like(t["x"])
            t["fs"] = torch.empty((cfg.batch, cfg.H, cfg.P, cfg.N), dtype=torch.float32, device="cuda")
            bufs.append(t)

        def step(i):
            t = bufs[i % sets]
            lib_ops.ssd_scan_fwd(t["x"], t["dt"], A, t["B"], t["C"], Dk, bias, True, y=t["y"], final_state=t["fs"])
        return cfg, inp, kind, nbytes, cfg.elements, sets, step, bufs

    inp = synth.make_config_inputs(cfg)
    nbytes = cfg.algorithmic_bytes()
    sets = args.sets or max(2, int(np.ceil(600e6 / nbytes)))
    A, Dk, bias = dev(torch, inp.A), dev(torch, inp.Dskip), dev(torch, inp.delta_bias)
    bufs = []
    for _ in range(sets):
        t = {k: dev(torch, inp.upload_array(k)) if inp.upload_array(k) is not None else None
             for k in ("u", "delta", "B", "C", "z")}
        t["y"] = torch.empty_like(t["u"])
        t["fs"] = torch.empty((cfg.batch, cfg.D, cfg.N), dtype=torch.float32, device="cuda")
        bufs.append(t)

    if kind == "bwd":
        # gradients of the scan for an output gradient dy; outputs and workspace are
        # allocated once, outside the timed graph
        dyv, dyup, _ = synth.make_scan_cotangents(cfg.batch, cfg.L, cfg.D, cfg.N, cfg.dtype, seed=cfg.seed)
        inp.dy = dyv
        act = bufs[0]["u"].dtype
        ws = torch.empty((lib_ops.selective_scan_bwd_workspace_size(cfg.batch, cfg.L, cfg.D, cfg.N, act,
                                                                    saved=cfg.saved),),
                         dtype=torch.uint8, device="cuda")
        grads = None
        for t in bufs:
            t["dy"] = dev(torch, dyup)
            t["cs"] = None
            if cfg.saved:   # the forward pass that saves the chunk states (in the step too, when training)
                _, _, t["cs"] = lib_ops.selective_scan_fwd_save(t["u"], t["delta"], A, t["B"], t["C"], Dk, t["z"],
                                                                bias, True, y=t["y"], final_state=t["fs"])
            if not cfg.train:
                del t["y"], t["fs"]
        torch.cuda.synchronize()

        def step(i):
            nonlocal grads
            t = bufs[i % sets]
            if cfg.train:
                lib_ops.selective_scan_fwd_save(t["u"], t["delta"], A, t["B"], t["C"], Dk, t["z"], bias, True,
                                                y=t["y"], final_state=t["fs"], chunk_states=t["cs"])
            grads = lib_ops.selective_scan_bwd(t["u"], t["delta"], A, t["B"], t["C"], t["dy"], Dk, t["z"], bias,
                                               True, workspace=ws, out=grads, chunk_states=t["cs"])
            t["g"] = grads
        return cfg, inp, kind, nbytes, cfg.elements, sets, step, bufs

    if cfg.conv_k:
        cw, cb = (dev(torch, x) for x in synth.make_conv_params(cfg.D, cfg.conv_k, seed=cfg.seed))

        def step(i):              # u = SiLU(conv1d(x)) fused into the scan; t["u"] holds x
            t = bufs[i % sets]
            lib_ops.selective_scan_fwd_conv(t["u"], cw, cb, t["delta"], A, t["B"], t["C"], Dk, t["z"], bias, True,
                                            y=t["y"], final_state=t["fs"], tokens_per_lane=args.kpl)
        return cfg, inp, kind, nbytes, cfg.elements, sets, step, bufs

    def step(i):
        t = bufs[i % sets]
        lib_ops.selective_scan_fwd(t["u"], t["delta"], A, t["B"], t["C"], Dk, t["z"], bias, True,
                                   y=t["y"], final_state=t["fs"], variant=args.variant,
                                   tokens_per_lane=args.kpl, discretization=cfg.discretization)
    return cfg, inp, kind, nbytes, cfg.elements, sets, step, bufs


def measure(torch, step, K, warm_steps, use_graph, check=None, reps=STAT_REPS):
    """Capture K steps in a graph; warm up by replaying until at least `warm_steps`
    steps and MIN_WARM_S of load have run; time one replay (the timed region) with
    wall clock and HIP events; then `reps` replays each bracketed by events for the
    per-step distribution.  Returns a dict of times."""
    stream = torch.cuda.current_stream()
    step(0)                       # first call: loads the code objects
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(K):
                step(i)

    def run():
        if graph is not None:
            graph.replay()
        else:
            for i in range(K):
                step(i)

    warm, t0 = 0, time.perf_counter()
    while warm < warm_steps or time.perf_counter() - t0 < MIN_WARM_S:
        run()
        warm += K
        torch.cuda.synchronize()
    warm_s = time.perf_counter() - t0
    if check is not None and graph is not None:
        check(K)                  # replayed outputs equal an eager call's, bit for bit
        run()
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = ev0.elapsed_time(ev1)
    per = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run()
        b.record(stream)
        b.synchronize()
        per.append(a.elapsed_time(b) * 1e3 / K)
    per = np.array(per)
    return {"wall_s": wall, "launch_us": gpu_ms * 1e3 / K, "warm_steps": warm, "warm_s": warm_s,
            "us_median": float(np.median(per)), "us_p10": float(np.percentile(per, 10)),
            "us_p90": float(np.percentile(per, 90)), "iterations": reps, "steps_per_iteration": K,
            "graph": graph is not None}


def steps_for(nbytes):
    """Steps per graph for a workload not given on the command line: at least about
    2 ms of work per replay, so launch gaps stay small against the kernel time."""
    est_us = nbytes / (2.5e12) * 1e6 + 3.0
    return int(max(20, min(2000, np.ceil(2000.0 / est_us))))


def alu_roofline(kind, cfg, elements, launch_s):
    spe = (BWD_ALU_SLOTS_PER_ELEMENT + (ALU_SLOTS_PER_ELEMENT if getattr(cfg, "train", False) else 0)
           if kind == "bwd" else
           ZOH_ALU_SLOTS_PER_ELEMENT if cfg.discretization == "zoh" else ALU_SLOTS_PER_ELEMENT)
    slots = spe * elements
    alu = slots / launch_s / 1e12
    return {"achieved": alu, "peak": PEAK_VALU_TSLOTS, "unit": "T VALU slots/s", "frac": alu / PEAK_VALU_TSLOTS,
            "algorithmic_slots_per_launch": slots, "slots_per_element": spe}


def calibrate(torch, lib):
    """Streaming-copy bandwidth over 1 GiB, and the FMA / exp2 issue rates."""
    import ctypes
    stream = torch.cuda.current_stream()
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    sp = stream.cuda_stream

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / 1e3 / reps

    t_copy = timed(lambda: lib.ssm_calib_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                              CALIB_BYTES, ctypes.c_void_p(sp)), 20)
    assert torch.equal(src[-1024:], dst[-1024:])
    blocks, iters = 256 * 4 * 8, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    ops = lib.ssm_calib_alu_ops(blocks, iters)
    t_fma = timed(lambda: lib.ssm_calib_alu(0, ctypes.c_void_p(out.data_ptr()), blocks, iters, ctypes.c_void_p(sp)), 5)
    t_exp = timed(lambda: lib.ssm_calib_alu(1, ctypes.c_void_p(out.data_ptr()), blocks, iters, ctypes.c_void_p(sp)), 5)
    fma = ops / t_fma / 1e12
    pair = ops / t_exp / 1e12                       # one multiply + one exp2 per chain step
    exp2 = 1.0 / max(1.0 / pair - 1.0 / fma, 1e-9)
    del src, dst, out
    return {"copy_gbs": 2 * CALIB_BYTES / t_copy / 1e9, "copy_bytes": 2 * CALIB_BYTES,
            "fma_t_per_s": fma, "exp2_t_per_s": exp2,
            "note": "lane operations per second; a streaming 16-byte-vector copy of 1 GiB (read + write)"}


def run_workload(name, args, torch, lib_ops, K=None, warm=None, check=False):
    cfg, inp, kind, nbytes, elements, sets, step, bufs = prepare(name, args, torch, lib_ops)
    print(f"# workload {name}: {elements:.3e} elements/step, {nbytes / 1e6:.2f} MB/step algorithmic, "
          f"{sets} input copies", file=sys.stderr, flush=True)
    K = K or steps_for(nbytes)
    chk = None
    if check and kind in ("scan", "bwd", "ssd"):
        def chk(K):
            if kind in ("scan", "ssd"):
                get = lambda: {k: bufs[(K - 1) % sets][k] for k in ("y", "fs")}
            else:
                get = lambda: {k: bufs[(K - 1) % sets]["g"][k] for k in ("du", "ddelta", "dz", "dA", "dB", "dC")}
            ref = {k: v.clone() for k, v in get().items() if v is not None}
            step(K - 1)
            torch.cuda.synchronize()
            assert all(torch.equal(ref[k], v) for k, v in get().items() if v is not None), \
                "graph replay differs from eager"
    m = measure(torch, step, K, warm if warm is not None else K, not args.no_graph, chk)
    m.update(cfg=cfg, inp=inp, kind=kind, nbytes=nbytes, elements=elements, sets=sets,
             kernel=kernel_of(cfg, kind, args.variant, args.kpl))
    del bufs
    return m


def summary(name, m):
    launch_s = m["launch_us"] / 1e6
    out = {"kernel": m["kernel"], "us_per_call": m["launch_us"], "us_median": m["us_median"], "us_p10": m["us_p10"],
           "us_p90": m["us_p90"], "elements_per_s": m["elements"] / launch_s,
           "hbm_gbs": m["nbytes"] / launch_s / 1e9, "hbm_frac": m["nbytes"] / launch_s / 1e9 / PEAK_HBM_GBS,
           "algorithmic_bytes": m["nbytes"], "steps_per_iteration": m["steps_per_iteration"],
           "iterations": m["iterations"], "input_copies": m["sets"]}
    if m["kind"] in ("scan", "bwd"):
        out["alu_frac"] = alu_roofline(m["kind"], m["cfg"], m["elements"], launch_s)["frac"]
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(synth.CONFIGS))
    ap.add_argument("--variant", type=int, default=0, help="ssm_scan_variant (--ap adds SSM_SCAN_AP)")
    ap.add_argument("--ap", action="store_true",
                    help="let the scan take its arithmetic-progression decay path where A allows it "
                         "(default: the general path, one exp per element)")
    ap.add_argument("--kpl", type=int, default=0)
    ap.add_argument("--sets", type=int, default=0, help="input copies to rotate (0 = enough to exceed 600 MB)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="skip timing the other named workloads")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the selective scan shards by independent (batch, channel) "
              "pairs with no communication, and multi-GPU runs are not part of this build; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_68_amd as lib_ops
    lib = lib_ops.load_library()
    if args.ap:
        args.variant |= lib_ops.SSM_SCAN_AP
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)

    calib = calibrate(torch, lib)
    print(f"# calibration: copy {calib['copy_gbs']:.0f} GB/s, fma {calib['fma_t_per_s']:.1f} T/s, "
          f"exp2 {calib['exp2_t_per_s']:.1f} T/s", file=sys.stderr, flush=True)

    m = run_workload(args.workload, args, torch, lib_ops, K=args.steps, warm=args.warmup, check=True)
    cfg, kind, nbytes, elements = m["cfg"], m["kind"], m["nbytes"], m["elements"]
    K = m["steps_per_iteration"]
    ms_per_step = m["wall_s"] * 1e3 / K
    value = elements / (ms_per_step / 1e3)
    launch_s = m["launch_us"] / 1e6
    hbm_gbs = nbytes / launch_s / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        if kind == "ssd":
            cpu = cpu_baseline_ssd(cfg, m["inp"], args.cpu_budget)
        elif kind in ("scan", "bwd") and not cfg.conv_k:
            cpu = cpu_baseline_scan(cfg, m["inp"], args.cpu_budget, dy=getattr(m["inp"], "dy", None))
    m["inp"] = None

    others = {}
    if not args.no_others and args.workload in GRADED:
        oargs = argparse.Namespace(**vars(args))
        oargs.variant, oargs.kpl, oargs.sets = 0, 0, 0
        for name in GRADED:
            if name == args.workload:
                continue
            mo = run_workload(name, oargs, torch, lib_ops, warm=0)
            mo["inp"] = None
            others[name] = summary(name, mo)
            torch.cuda.empty_cache()

    # The arithmetic-progression decay path: the same calls with SSM_SCAN_AP
    ap_path = {}
    if not args.no_others and not args.ap and args.workload in GRADED:
        general = dict(others, **{args.workload: summary(args.workload, m)})
        oargs = argparse.Namespace(**vars(args))
        oargs.variant, oargs.kpl, oargs.sets = lib_ops.SSM_SCAN_AP, 0, 0
        for name in AP_WORKLOADS:
            mo = run_workload(name, oargs, torch, lib_ops, warm=0)
            mo["inp"] = None
            s = summary(name, mo)
            s["speedup_vs_general"] = general[name]["us_per_call"] / s["us_per_call"]
            ap_path[name] = s
            torch.cuda.empty_cache()

    kernel = m["kernel"]
    traffic = traffic_from_profiles(args.workload, kernel)
    hbm = {"achieved": hbm_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": hbm_gbs / PEAK_HBM_GBS,
           "algorithmic_bytes_per_launch": nbytes}
    roofline = dict(hbm, bound="hbm", kernel=kernel, traffic=traffic, avg_launch_us=m["launch_us"])
    if kind in ("scan", "bwd"):
        alu = alu_roofline(kind, cfg, elements, launch_s)
        # the HBM fraction the call would reach with the VALU at its peak: at N = 16
        # the bfloat16 scans (0.5 B per element) cannot pass ~0.41 of 8 TB/s
        alu["hbm_frac_at_alu_peak"] = (nbytes / (alu["algorithmic_slots_per_launch"] / (PEAK_VALU_TSLOTS * 1e12))
                                       / 1e9 / PEAK_HBM_GBS)
        roofline["alu"] = alu
    if kind == "ssd":
        fl = cfg.flops()
        roofline["mfma"] = {"achieved": fl / launch_s / 1e12, "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                            "frac": fl / launch_s / 1e12 / PEAK_MFMA_BF16_TFLOPS, "flops_per_launch": fl}
    metric = {"scan": "selective-scan elements/s (B*L*D*N) + achieved HBM GB/s vs peak, 1 GPU",
              "ssd": "SSD-scan elements/s (B*L*H*P*N) + achieved HBM GB/s vs peak, 1 GPU",
              "bwd": "selective-scan backward elements/s (B*L*D*N) + achieved HBM GB/s vs peak, 1 GPU",
              "decode": "decode-step elements/s (S*D*N per step) + achieved HBM GB/s vs peak, 1 GPU"}[kind]
    if kind in ("scan", "bwd"):
        config = {"workload": args.workload, "batch": cfg.batch, "L": cfg.L, "D": cfg.D, "N": cfg.N,
                  "act_dtype": cfg.dtype, "gate": cfg.gate, "conv_width": cfg.conv_k,
                  "discretization": cfg.discretization, "variant": args.variant,
                  "decay_path": "arithmetic progression (SSM_SCAN_AP)" if args.ap else
                  "general (one exp per element)",
                  "tokens_per_lane": args.kpl or "auto"}
    elif kind == "ssd":
        config = {"workload": args.workload, "batch": cfg.batch, "L": cfg.L, "H": cfg.H, "P": cfg.P, "N": cfg.N,
                  "act_dtype": cfg.dtype, "chunk": 64}
    else:
        config = {"workload": args.workload, "sequences": cfg.batch, "D": cfg.D, "N": cfg.N,
                  "act_dtype": cfg.dtype}
    config.update(graph=m["graph"], input_copies=m["sets"])
    out = {
        "metric": metric,
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": m["warm_steps"],
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if kind == "ssd" else "f32",
        "data": "synthetic (seeded; shapes and distributions of the named workload)",
        "config": config,
        "roofline": roofline,
        "hbm": hbm,
        "timing": {"us_median": m["us_median"], "us_p10": m["us_p10"], "us_p90": m["us_p90"],
                   "iterations": m["iterations"], "steps_per_iteration": K, "warmup_steps": m["warm_steps"],
                   "warmup_s": m["warm_s"], "min_warmup_s": MIN_WARM_S},
        "workloads": others,
        "ap_path": ap_path,
        "calibration": calib,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "hbm_gib": props.total_memory / 2 ** 30},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
