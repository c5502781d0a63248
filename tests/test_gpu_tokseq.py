"""GPU parity of the token-sequential scan kernel (SSM_SCAN_TOKSEQ) against the
float64 oracle, through the C ABI.

The kernel gives each lane 4 (or 2) states of a channel and walks the tokens in
order in blocks of 32 (or 64); these cases cover both lane layouts, both
activation types, with and without the gate and skip term, channel counts that
leave the last wave and the last lane group partly idle, sequence lengths that
end inside a block, a given initial state, every output of the full 1.4B-shaped
workload in the 2-states-per-lane build, determinism and the shapes the kernel
rejects.
"""
import numpy as np
import pytest

import oracle
import synth
import oracle_pool
from gpu_util import TOL, dev, host, oracle_scan, run_scan, upload_scan
from ssm_metrics import row_rel_err

pytestmark = pytest.mark.gpu

TOKSEQ = 3


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_state_space_68_amd import load_library
    load_library()


def _check(y, fs, ry, rf, dtype, what):
    ey, ef = row_rel_err(y, ry), row_rel_err(fs, rf)
    print(f"{what} y_err={ey:.3e} state_err={ef:.3e} tol={TOL[dtype]:.0e}", flush=True)
    assert ey <= TOL[dtype], (what, ey)
    assert ef <= TOL[dtype], (what, ef)


SHAPES = [
    # batch, L, D, dtype, gate, d_skip, bias
    (1, 8, 1, "f32", True, "normal", True),        # one token piece, one lane group in use
    (2, 40, 17, "bf16", True, "ones", True),       # L ends inside the first block; 17 channels
    (3, 72, 70, "f32", False, "normal", True),     # several waves, the last one partly idle
    (1, 1032, 33, "bf16", True, "normal", False),  # many blocks, ragged last block, no bias
    (2, 264, 64, "f32", True, "none", True),       # no skip term
]


@pytest.mark.parametrize("spl", [4, 2])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:3])) + f"-{s[3]}")
def test_tokseq_matches_oracle(shape, spl):
    batch, L, D, dtype, gate, dsk, bias = shape
    inp = synth.make_scan_inputs(batch, L, D, 16, dtype, gate=gate, d_skip=dsk, seed=L + D,
                                 a_kind="lognormal", with_bias=bias)
    ry, rf = oracle_scan(inp)
    y, fs = run_scan(inp, variant=TOKSEQ, tokens_per_lane=spl)
    _check(host(y), host(fs), ry, rf, dtype, f"tokseq spl={spl} {shape}")


@pytest.mark.parametrize("spl", [4, 2])
def test_tokseq_from_initial_state(spl):
    inp = synth.make_scan_inputs(2, 520, 21, 16, "bf16", gate=True, seed=5, a_kind="lognormal")
    h0 = np.random.default_rng(6).standard_normal((2, 21, 16)).astype(np.float32)
    ry, rf = oracle.selective_scan(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, inp.delta_bias,
                                   inp.delta_softplus, h0=h0)
    t = upload_scan(inp)
    y, fs = run_scan(inp, t, variant=TOKSEQ, tokens_per_lane=spl, initial_state=dev(h0))
    _check(host(y), host(fs), ry, rf, "bf16", f"tokseq from h0 spl={spl}")


def test_tokseq_full_1p4b_workload_two_states_per_lane():
    """The 1.4B-shaped workload (8 x 2048 x 4096, bfloat16) in the 2-states-per-lane
    build of the token-sequential kernel (the automatic choice, 4 per lane, is checked
    by test_gpu_parity), every output against the oracle."""
    cfg = synth.CONFIGS["mamba1p4b_bf16"]
    inp = synth.make_config_inputs(cfg)
    y, fs = run_scan(inp, variant=TOKSEQ, tokens_per_lane=2)
    yh, fh = host(y), host(fs)
    del y, fs
    ey, ef, _ = oracle_pool.scan_errors(inp, yh, fh, label="tokseq 2 states per lane, 1.4B")
    assert ey <= TOL[cfg.dtype] and ef <= TOL[cfg.dtype], (ey, ef)


def test_tokseq_deterministic():
    import torch
    inp = synth.make_scan_inputs(2, 1024, 300, 16, "bf16", gate=True, seed=9)
    t = upload_scan(inp)
    y1, f1 = run_scan(inp, t, variant=TOKSEQ)
    y2, f2 = run_scan(inp, t, variant=TOKSEQ)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


@pytest.mark.parametrize("shape", [(1, 64, 4, 8), (1, 100, 4, 16)], ids=["N8", "L100"])
def test_tokseq_rejects_unsupported_shapes(shape):
    from selective_state_space_68_amd import SsmError
    batch, L, D, N = shape
    inp = synth.make_scan_inputs(batch, L, D, N, "f32", seed=1)
    with pytest.raises(SsmError):
        run_scan(inp, variant=TOKSEQ)
