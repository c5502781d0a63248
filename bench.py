"""Benchmark of the selective scan (and the decode step) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one full pass of the hot path over one batch: one selective-scan call
over the whole [batch, D, L] workload (softplus, discretisation, scan, readout,
skip, gate, final state), or for the decode workload one state-update call.
Inputs are synthetic and seeded (synth/), resident in HBM before timing.  Each
step reads a different copy of the inputs (enough copies to exceed the 256 MB
Infinity Cache), so every step streams its inputs from HBM.  The K steps are
captured in one HIP graph and replayed between two synchronisations, after W
warm-up steps (whole replays of the same graph) have brought the GPU to its
sustained clock: over the first ~10 ms of load the scan runs ~15 % slower.

Prints one JSON line: elements/s (B*L*D*N per second); the roofline of the
call (the scan is bound by the vector ALUs: algorithmic VALU slots / average call
time against the single-issue fp32 peak; the decode step by HBM bandwidth); the
achieved HBM GB/s against 8 TB/s; and the float64 CPU oracle timed on this
host's cores on a bounded sample.
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
CALIB_BYTES = 256 << 20
DEFAULT_WORKLOAD = "mamba130m_f32"
_CSRC = "selective_state_space_68_amd/csrc/"
KERNEL_SRC = {"scan_chunked_kernel": _CSRC + "scan_chunked.hip", "scan_tokseq_kernel": _CSRC + "scan_tokseq.hip",
              "scan_sequential_kernel": _CSRC + "scan_sequential.hip",
              "state_update_vec_kernel": _CSRC + "state_update.hip", "ssd_scan_kernel": _CSRC + "ssd.hip"}
KERNEL_NAME = {"decode": "state_update_vec_kernel",
               "bwd": "scan backward call (bwd_summary, bwd_combine, bwd_main, bwd_param_sums, bwd_bc_out kernels)",
               "ssd": "ssd_scan_kernel"}
KERNEL_SRC[KERNEL_NAME["bwd"]] = _CSRC + "scan_bwd.hip"
PEAK_MFMA_BF16_TFLOPS = 2500.0


def kernel_of(cfg, kind, variant=0, tokens_per_lane=0):
    """The kernel (or, for the backward, the call) a workload's timed region runs.
    The forward scan asks the library which kernel it picks for the shape."""
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
    """HBM bytes per launch from committed rocprofv3 PMC summaries, or None when the
    kernel source changed since the counters were taken."""
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


def _oracle_shard(args):
    """Worker: the oracle (forward, or backward when an output gradient is given) on one
    (batch row, channel block) shard; returns seconds."""
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
    """The float64 oracle, as it is, timed on this host's cores: the workload is split
    into (batch row, channel block) shards run by a pool of worker processes, on as
    many whole batch rows as fit in about budget_s of CPU time.  With `dy` the oracle's
    backward pass is timed (each shard's dB and dC are its channels' partial sums;
    adding the partials is not timed)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    ncpu = len(os.sched_getaffinity(0))
    workers = workers or max(1, min(16, ncpu))
    # size the sample from a single-process probe on one channel block
    d_probe = min(cfg.D, 64)
    sl = lambda x, b0, b1, d0, d1: None if x is None else x[b0:b1, d0:d1]
    vec = lambda x, d0, d1: None if x is None else x[d0:d1]
    t0 = time.perf_counter()
    _oracle_shard((inp.u[:1, :d_probe], inp.delta[:1, :d_probe], inp.A[:d_probe], inp.B[:1], inp.C[:1],
                   vec(inp.Dskip, 0, d_probe), sl(inp.z, 0, 1, 0, d_probe),
                   vec(inp.delta_bias, 0, d_probe), inp.delta_softplus, sl(dy, 0, 1, 0, d_probe),
                   cfg.discretization))
    per_row_cpu = (time.perf_counter() - t0) * cfg.D / d_probe
    b_take = max(1, min(cfg.batch, int(budget_s / max(per_row_cpu, 1e-3))))
    dblk = max(1, -(-cfg.D // max(1, (workers + b_take - 1) // b_take)))
    shards = []
    for b in range(b_take):
        for d0 in range(0, cfg.D, dblk):
            d1 = min(cfg.D, d0 + dblk)
            shards.append((sl(inp.u, b, b + 1, d0, d1), sl(inp.delta, b, b + 1, d0, d1), inp.A[d0:d1],
                           inp.B[b:b + 1], inp.C[b:b + 1], vec(inp.Dskip, d0, d1), sl(inp.z, b, b + 1, d0, d1),
                           vec(inp.delta_bias, d0, d1), inp.delta_softplus, sl(dy, b, b + 1, d0, d1),
                           cfg.discretization))
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        list(ex.map(_oracle_warm, range(workers)))   # start the workers and import the oracle
        t0 = time.perf_counter()
        one = sum(ex.map(_oracle_shard, shards))       # one pass: sizes the repetition count
        # a pass far below the CPU budget (the whole workload) is repeated, for a stable time
        reps = max(1, min(50, int(budget_s / max(one, 1e-3))))
        t0 = time.perf_counter()
        secs = list(ex.map(_oracle_shard, shards * reps))
        wall = time.perf_counter() - t0
    elems = b_take * cfg.L * cfg.D * cfg.N
    return {"value": reps * elems / wall, "unit": "elements/s", "cores": workers, "kind": "oracle",
            "sample": f"{'backward, ' if dy is not None else ''}{cfg.discretization} discretization, {b_take} of {cfg.batch} batch rows x all {cfg.D} channels x full L={cfg.L}, N={cfg.N} "
                      f"({elems:.3e} elements), {reps}x, in {len(shards)} shards per pass over {workers} "
                      f"worker processes "
                      f"(float64 numpy, 1 thread each; {wall:.1f} s wall, {sum(secs):.1f} s CPU); "
                      f"host has {ncpu} usable cores"}


def bench_scan(args, torch, lib_ops):
    cfg = synth.CONFIGS[args.workload]
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

    if cfg.backward:
        # gradients of the scan for an output gradient dy; outputs and workspace are
        # allocated once, outside the timed graph
        dyv, dyup, _ = synth.make_scan_cotangents(cfg.batch, cfg.L, cfg.D, cfg.N, cfg.dtype, seed=cfg.seed)
        inp.dy = dyv
        act = bufs[0]["u"].dtype
        ws = torch.empty((lib_ops.selective_scan_bwd_workspace_size(cfg.batch, cfg.L, cfg.D, cfg.N, act),),
                         dtype=torch.uint8, device="cuda")
        grads = None
        for t in bufs:
            t["dy"] = dev(torch, dyup)
            del t["y"], t["fs"]
        dyv = dyup = None

        def step(i):
            nonlocal grads
            t = bufs[i % sets]
            grads = lib_ops.selective_scan_bwd(t["u"], t["delta"], A, t["B"], t["C"], t["dy"], Dk, t["z"], bias,
                                               True, workspace=ws, out=grads)
            t["g"] = grads
        return cfg, inp, nbytes, cfg.elements, sets, step, bufs

    if cfg.conv_k:
        cw, cb = (dev(torch, x) for x in synth.make_conv_params(cfg.D, cfg.conv_k, seed=cfg.seed))

        def step(i):              # u = SiLU(conv1d(x)) fused into the scan; t["u"] holds x
            t = bufs[i % sets]
            lib_ops.selective_scan_fwd_conv(t["u"], cw, cb, t["delta"], A, t["B"], t["C"], Dk, t["z"], bias, True,
                                            y=t["y"], final_state=t["fs"], tokens_per_lane=args.kpl)
        return cfg, inp, nbytes, cfg.elements, sets, step, bufs

    def step(i):
        t = bufs[i % sets]
        lib_ops.selective_scan_fwd(t["u"], t["delta"], A, t["B"], t["C"], Dk, t["z"], bias, True,
                                   y=t["y"], final_state=t["fs"], variant=args.variant,
                                   tokens_per_lane=args.kpl, discretization=cfg.discretization)

    return cfg, inp, nbytes, cfg.elements, sets, step, bufs


def bench_decode(args, torch, lib_ops):
    cfg = synth.CONFIGS[args.workload]
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

    return cfg, None, nbytes, cfg.elements_per_step, sets, step, bufs


def bench_ssd(args, torch, lib_ops):
    cfg = synth.CONFIGS[args.workload]
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

    return cfg, inp, nbytes, cfg.elements, sets, step, bufs


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
    return {"value": elems / wall, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"SSD, 1 of {cfg.batch} batch rows x {heads} of {cfg.H} heads x full L={cfg.L}, "
                      f"P={cfg.P}, N={cfg.N} ({elems:.3e} elements), float64 numpy, one process, "
                      f"{wall:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(synth.CONFIGS))
    ap.add_argument("--variant", type=int, default=0)
    ap.add_argument("--kpl", type=int, default=0)
    ap.add_argument("--sets", type=int, default=0, help="input copies to rotate (0 = enough to exceed 600 MB)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the selective scan shards by independent (batch, channel) "
              "pairs with no communication, and multi-GPU runs are not part of this build; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_68_amd as lib_ops
    lib_ops.load_library()
    torch.cuda.set_device(0)
    kind = "decode" if args.workload.startswith("decode") else "scan"
    maker = bench_decode if kind == "decode" else bench_scan
    if isinstance(synth.CONFIGS[args.workload], synth.SSDConfig):
        kind, maker = "ssd", bench_ssd
    elif kind == "scan" and synth.CONFIGS[args.workload].backward:
        kind = "bwd"
    cfg, inp, nbytes, elements, sets, step, bufs = maker(args, torch, lib_ops)
    print(f"# workload {args.workload}: {elements:.3e} elements/step, {nbytes / 1e6:.2f} MB/step "
          f"algorithmic, {sets} input copies", file=sys.stderr, flush=True)

    # A plain device-to-device copy of known size (256 MiB read + 256 MiB written):
    # the calibration that HBM-byte counters (FETCH_SIZE / WRITE_SIZE) are scaled by.
    calib_src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    stream = torch.cuda.current_stream()
    step(0)                       # first call: loads the code objects
    torch.cuda.synchronize()

    K = args.steps
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(K):
                step(i)
    # W untimed warm-up steps, run the way the timed steps run (whole replays of the
    # K-step graph, so W is rounded up to a multiple of K).  The GPU needs tens of
    # milliseconds of sustained load to reach its steady clock; the timed region
    # measures that sustained rate.
    warm = 0
    while warm < args.warmup:
        if graph is not None:
            graph.replay()
            warm += K
        else:
            step(warm)
            warm += 1
    torch.cuda.synchronize()
    if graph is not None and kind in ("scan", "bwd", "ssd"):
        # the replayed outputs must equal an eager call's, bit for bit
        if warm == 0:
            graph.replay()
            torch.cuda.synchronize()
        if kind in ("scan", "ssd"):
            get = lambda: {k: bufs[(K - 1) % sets][k] for k in ("y", "fs")}
        else:
            get = lambda: {k: bufs[(K - 1) % sets]["g"][k] for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD")}
        ref = {k: v.clone() for k, v in get().items()}
        step(K - 1)
        torch.cuda.synchronize()
        assert all(torch.equal(ref[k], v) for k, v in get().items()), "graph replay differs from eager"
        if warm:                  # back to the sustained state before timing
            graph.replay()
            torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(K):
            step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall * 1e3 / K
    launch_s = gpu_ms / K / 1e3       # events bracket the K calls; a call is one kernel launch
    value = elements / (ms_per_step / 1e3)
    hbm_gbs = nbytes / launch_s / 1e9

    cpu = None
    if kind == "ssd" and not args.no_cpu_baseline:
        cpu = cpu_baseline_ssd(cfg, inp, args.cpu_budget)
    elif kind in ("scan", "bwd") and not args.no_cpu_baseline and not cfg.conv_k:
        cpu = cpu_baseline_scan(cfg, inp, args.cpu_budget, dy=getattr(inp, "dy", None))

    kernel = kernel_of(cfg, kind, args.variant, args.kpl)
    traffic = traffic_from_profiles(args.workload, kernel)
    hbm = {"achieved": hbm_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": hbm_gbs / PEAK_HBM_GBS,
           "algorithmic_bytes_per_launch": nbytes}
    if kind in ("scan", "bwd"):
        # Bound by the vector ALUs: per element 4 fp32 VALU ops plus one exp2, which
        # issues at half the VALU rate (2 slots), against 256 CUs x 4 SIMDs x 16 lanes
        # x 2.4 GHz single-issue fp32 slots (the backward: BWD_ALU_SLOTS_PER_ELEMENT,
        # over the whole call of its five kernels).
        spe = (BWD_ALU_SLOTS_PER_ELEMENT if kind == "bwd" else
               ZOH_ALU_SLOTS_PER_ELEMENT if cfg.discretization == "zoh" else ALU_SLOTS_PER_ELEMENT)
        slots = spe * elements
        alu = slots / launch_s / 1e12
        roofline = {"bound": "alu", "kernel": kernel,
                    "achieved": alu, "peak": PEAK_VALU_TSLOTS, "unit": "T VALU slots/s",
                    "frac": alu / PEAK_VALU_TSLOTS, "traffic": traffic,
                    "algorithmic_slots_per_launch": slots, "slots_per_element": spe,
                    "avg_launch_us": launch_s * 1e6}
    else:
        roofline = dict(hbm, bound="hbm", kernel=kernel, traffic=traffic,
                        avg_launch_us=launch_s * 1e6)
        if kind == "ssd":
            # the matrix-core side, for reference: the chunked form's products
            fl = cfg.flops()
            roofline["mfma"] = {"achieved": fl / launch_s / 1e12, "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                                "frac": fl / launch_s / 1e12 / PEAK_MFMA_BF16_TFLOPS, "flops_per_launch": fl}
    out = {
        "metric": {"scan": "selective-scan elements/s (B*L*D*N) + achieved HBM GB/s vs peak, 1 GPU",
                   "ssd": "SSD-scan elements/s (B*L*H*P*N) + achieved HBM GB/s vs peak, 1 GPU",
                   "bwd": "selective-scan backward elements/s (B*L*D*N) + achieved HBM GB/s vs peak, 1 GPU",
                   "decode": "decode-step elements/s (S*D*N per step) + achieved HBM GB/s vs peak, 1 GPU"}[kind],
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warm,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if kind == "ssd" else "f32",
        "data": "synthetic (seeded; shapes and distributions of the named workload)",
        "config": ({"workload": args.workload, "batch": cfg.batch, "L": cfg.L, "D": cfg.D, "N": cfg.N,
                    "act_dtype": cfg.dtype, "gate": cfg.gate, "conv_width": cfg.conv_k,
                    "discretization": cfg.discretization, "variant": args.variant,
                    "tokens_per_lane": args.kpl or "auto", "graph": graph is not None, "input_copies": sets}
                   if kind in ("scan", "bwd") else
                   {"workload": args.workload, "batch": cfg.batch, "L": cfg.L, "H": cfg.H, "P": cfg.P, "N": cfg.N,
                    "act_dtype": cfg.dtype, "chunk": 64, "graph": graph is not None, "input_copies": sets}
                   if kind == "ssd" else
                   {"workload": args.workload, "sequences": cfg.batch, "D": cfg.D, "N": cfg.N,
                    "act_dtype": cfg.dtype, "graph": graph is not None, "input_copies": sets}),
        "roofline": roofline,
        "hbm": hbm,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
