"""The sharded oracle comparison that the full-size GPU parity tests use, checked on
the CPU: sharding over worker processes gives the errors of one whole-workload oracle
call, and a single wrong output element anywhere (planted here in a copy of the
oracle's own result, standing in for a GPU output) is found."""
import numpy as np

import oracle
import oracle_pool
import synth
from ssm_metrics import row_rel_err


def test_scan_errors_match_one_oracle_call_and_catch_a_planted_error():
    inp = synth.make_scan_inputs(3, 200, 37, 16, "bf16", seed=5, a_kind="lognormal", d_skip="normal")
    h0 = synth.make_scan_initial_state(3, 37, 16, seed=2)
    ry, rf = oracle.selective_scan(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, inp.delta_bias,
                                   True, h0=h0)
    # a "GPU" output: the oracle's rounded to float32 (as the shards receive it)
    y32, f32 = ry.astype(np.float32), rf.astype(np.float32)
    ey, ef, et = oracle_pool.scan_errors(inp, y32, f32, h0=h0, nworkers=3)
    assert np.isclose(ey, row_rel_err(y32, ry), rtol=1e-12, atol=0)
    assert np.isclose(ef, row_rel_err(f32, rf), rtol=1e-12, atol=0)
    assert ey < 1e-6 and ef < 1e-6 and et < 1e-6
    bad = y32.copy()
    bad[2, 36, 150] += np.float32(0.05 * np.abs(ry[2, 36]).max())     # the last channel of the last row
    ey2, _, et2 = oracle_pool.scan_errors(inp, bad, f32, h0=h0, nworkers=3)
    assert 0.04 < ey2 < 0.06 and et2 < 1e-6                           # token 150 is before the tail
    badf = f32.copy()
    badf[0, 0, 0] = np.nan
    assert oracle_pool.scan_errors(inp, y32, badf, h0=h0, nworkers=2)[1] == np.inf


def test_scan_errors_with_the_fused_conv_and_the_full_hold():
    inp = synth.make_scan_inputs(1, 130, 9, 8, "f32", seed=6, a_kind="lognormal")
    w, cb = synth.make_conv_params(9, 4, seed=1)
    u = oracle.causal_conv1d(inp.u, w, cb, apply_silu=True)
    ry, rf = oracle.selective_scan(u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, inp.delta_bias,
                                   discretization="zoh")
    ey, ef, _, eu = oracle_pool.scan_errors(inp, ry, rf, discretization="zoh", conv=(w, cb), u_gpu=u,
                                            nworkers=2)
    assert ey < 1e-6 and ef < 1e-6 and eu < 1e-6
    ey2 = oracle_pool.scan_errors(inp, ry, rf, discretization="simplified", conv=(w, cb), nworkers=2)[0]
    assert ey2 > 1e-4                                                  # the other discretization differs


def test_decode_errors_match_stepping_the_oracle():
    cfg = synth.DecodeConfig("small_decode", 6, 40, 16, 5, "bf16", True, 3)
    A, Dsk, bias = synth.make_decode_params(cfg.batch, cfg.D, cfg.N, seed=cfg.seed)
    h = synth.make_decode_state(cfg.batch, cfg.D, cfg.N, seed=cfg.seed).astype(np.float64)
    ys = []
    for step in range(cfg.steps):
        x = synth.make_decode_step(cfg.batch, cfg.D, cfg.N, step, cfg.dtype, cfg.gate, seed=cfg.seed)
        y, h = oracle.state_update(h, x.u, x.delta, A, x.B, x.C, Dsk, x.z, bias, True)
        ys.append(y)
    ys = np.stack(ys).astype(np.float32)
    ey, ef = oracle_pool.decode_errors(cfg, ys, h.astype(np.float32), nworkers=4)
    assert ey < 1e-6 and ef < 1e-6
    bad = ys.copy()
    bad[4, 5, 39] *= np.float32(1.5)                                   # last step, last sequence and channel
    assert oracle_pool.decode_errors(cfg, bad, h.astype(np.float32), nworkers=4)[0] > 1e-3
