"""Full-size parity against the float64 oracle, sharded over host cores.

The oracle is a plain loop over time vectorised over (batch, channel, state), so a
workload splits into independent (batch row, channel block) shards (B and C are
shared by the channels of a row, so a shard takes its row's B and C whole).  A pool
of worker processes (spawned, one numpy thread each, at most 16: the GPU machine's host
share) runs the oracle on each shard and compares it with the GPU's output for that
shard, in the metric of ssm_metrics; only the per-shard errors come back, so no
float64 copy of a whole workload's outputs is ever held.

Every output element is compared: nothing is sampled.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import time

import numpy as np


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _pool(n):
    return cf.ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"))


def _row_stats(x, ref, axis=-1):
    """Per-row max |x - ref| and max |ref| (the pieces of ssm_metrics.row_rel_err)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    num = np.max(np.abs(x - ref), axis=axis)
    den = np.max(np.abs(ref), axis=axis)
    if not np.all(np.isfinite(x)):
        num = np.full_like(num, np.inf)
    return num, den


def _err(num, den):
    err = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return float(np.max(err)) if err.size else 0.0


def _scan_shard(args):
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    import oracle
    (u, delta, A, B, C, Dk, z, bias, sp, h0, disc, conv, y_gpu, f_gpu, u_gpu, tail) = args
    eu = 0.0
    if conv is not None:                      # u holds the conv input x; the scan input is SiLU(conv(x))
        u = oracle.causal_conv1d(u, conv[0], conv[1], apply_silu=True)
        if u_gpu is not None:
            eu = _err(*_row_stats(u_gpu, u))
    ry, rf = oracle.selective_scan(u, delta, A, B, C, Dk, z, bias, sp, h0=h0, discretization=disc)
    ey = _err(*_row_stats(y_gpu, ry))
    ef = _err(*_row_stats(f_gpu, rf))
    et = _err(*_row_stats(y_gpu[..., -tail:], ry[..., -tail:]))
    return ey, ef, et, eu


def scan_errors(inp, y_gpu, f_gpu, h0=None, discretization="simplified", conv=None, u_gpu=None, tail_frac=64,
                nworkers=0, label=""):
    """Max row errors (y, final state, the last L/tail_frac tokens of y) of the GPU's
    scan outputs y_gpu [batch, D, L] and f_gpu [batch, D, N] (numpy, any float dtype)
    against the oracle, over every channel.  With conv = (w [D, K], bias [D] or
    None), inp.u is the input of the fused causal conv1d + SiLU, and u_gpu (if given)
    the GPU's conv output, whose error is returned fourth."""
    nw = nworkers or workers()
    batch, D, L = inp.u.shape
    tail = max(1, L // tail_frac)
    # about two shards per worker, whole batch rows where there are enough of them
    per_row = max(1, -(-2 * nw // batch))
    dblk = max(1, -(-D // per_row))
    sl = lambda x, b, d0, d1: None if x is None else x[b:b + 1, d0:d1]
    vec = lambda x, d0, d1: None if x is None else x[d0:d1]
    shards = []
    for b in range(batch):
        for d0 in range(0, D, dblk):
            d1 = min(D, d0 + dblk)
            shards.append((sl(inp.u, b, d0, d1), sl(inp.delta, b, d0, d1), inp.A[d0:d1], inp.B[b:b + 1],
                           inp.C[b:b + 1], vec(inp.Dskip, d0, d1), sl(inp.z, b, d0, d1),
                           vec(inp.delta_bias, d0, d1), inp.delta_softplus, sl(h0, b, d0, d1), discretization,
                           None if conv is None else (conv[0][d0:d1], vec(conv[1], d0, d1)),
                           np.asarray(y_gpu[b:b + 1, d0:d1], dtype=np.float32),
                           np.asarray(f_gpu[b:b + 1, d0:d1], dtype=np.float32),
                           None if u_gpu is None else np.asarray(u_gpu[b:b + 1, d0:d1], dtype=np.float32), tail))
    t0 = time.perf_counter()
    with _pool(nw) as ex:
        res = list(ex.map(_scan_shard, shards))
    ey = max(r[0] for r in res)
    ef = max(r[1] for r in res)
    et = max(r[2] for r in res)
    eu = max(r[3] for r in res)
    print(f"{label} oracle over {batch * D} channels in {len(shards)} shards on {nw} workers: "
          f"{time.perf_counter() - t0:.1f} s; y_err={ey:.3e} state_err={ef:.3e} tail_err={et:.3e}"
          + (f" u_err={eu:.3e}" if u_gpu is not None else ""), flush=True)
    return (ey, ef, et, eu) if conv is not None else (ey, ef, et)


def _decode_shard(args):
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    import oracle
    import synth
    (S, D, N, steps, dtype, gate, seed, s0, s1, y_gpu, f_gpu) = args
    A, Dsk, bias = synth.make_decode_params(S, D, N, seed=seed)
    h = synth.make_decode_state(S, D, N, seed=seed)[s0:s1].astype(np.float64)
    num = np.zeros((s1 - s0, D))
    den = np.zeros((s1 - s0, D))
    for step in range(steps):
        x = synth.make_decode_step(S, D, N, step, dtype, gate, seed=seed)
        y, h = oracle.state_update(h, x.u[s0:s1], x.delta[s0:s1], A, x.B[s0:s1], x.C[s0:s1], Dsk,
                                   None if x.z is None else x.z[s0:s1], bias, True)
        yg = np.asarray(y_gpu[step], dtype=np.float64)
        d = np.abs(yg - y)
        if not np.all(np.isfinite(yg)):
            d = np.full_like(d, np.inf)
        num = np.maximum(num, d)
        den = np.maximum(den, np.abs(y))
    ey = _err(num, den)                       # a row: one (sequence, channel)'s outputs over the steps
    ef = _err(*_row_stats(f_gpu, h))          # a row: one (sequence, channel)'s state vector
    return ey, ef


def decode_errors(cfg, y_gpu, f_gpu, nworkers=0, label=""):
    """Max row errors of `cfg.steps` decode steps: y_gpu [steps, S, D] and the final
    state f_gpu [S, D, N] against the oracle's steps from the same initial state, the
    sequences split over the workers (each regenerates the seeded per-step inputs)."""
    nw = nworkers or workers()
    S, D, N = cfg.batch, cfg.D, cfg.N
    blk = max(1, -(-S // nw))
    shards = [(S, D, N, cfg.steps, cfg.dtype, cfg.gate, cfg.seed, s0, min(S, s0 + blk),
               np.asarray(y_gpu[:, s0:min(S, s0 + blk)], dtype=np.float32),
               np.asarray(f_gpu[s0:min(S, s0 + blk)], dtype=np.float32)) for s0 in range(0, S, blk)]
    t0 = time.perf_counter()
    with _pool(nw) as ex:
        res = list(ex.map(_decode_shard, shards))
    ey = max(r[0] for r in res)
    ef = max(r[1] for r in res)
    print(f"{label} decode oracle over {S * D} channels x {cfg.steps} steps in {len(shards)} shards on {nw} "
          f"workers: {time.perf_counter() - t0:.1f} s; y_err={ey:.3e} state_err={ef:.3e}", flush=True)
    return ey, ef
