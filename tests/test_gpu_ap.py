"""The scan's arithmetic-progression decay path against the float64 oracle and
against the general path, through the C ABI.

For an A row with A[d, n] = A[d, 0] + n b, b <= 0 (S4D-real -(n+1), the
HiPPO-derived -(2n+1) of the interview-prep page's "Discretization and
initialization details"), exp(Delta A[d, n]) = exp(Delta A[d, n0]) exp(Delta b)^(n - n0),
and, asked to (SSM_SCAN_AP), the bfloat16 N = 16 kernels form most decays by
multiplying.  Checked here:
both paths within the bfloat16 bar of the oracle, in the chunked kernel (12-wave
vector-load build) and the token-sequential kernel (4 states per lane); the
detection (the path changes the final states of arithmetic rows, a lognormal row or
a row one ulp off takes the general path bit for bit, per channel in the chunked
kernel and per 16-channel wave in the token-sequential one); increasing rows
(b > 0) and the chunked kernel's scalar-load build stay on the general path;
float32 is unaffected.
"""
import numpy as np
import pytest

import synth
from gpu_util import TOL, host, oracle_scan, run_scan, upload_scan
from ssm_metrics import row_rel_err

pytestmark = pytest.mark.gpu

CHUNKED, TOKSEQ = 2, 3


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _ap_flag():
    from selective_state_space_68_amd import SSM_SCAN_AP
    return SSM_SCAN_AP


def _both(inp, variant, kpl):
    """(y, final) with SSM_SCAN_AP, then without it (the general path)."""
    t = upload_scan(inp)
    y_ap, f_ap = run_scan(inp, t, variant=variant | _ap_flag(), tokens_per_lane=kpl)
    y_g, f_g = run_scan(inp, t, variant=variant, tokens_per_lane=kpl)
    return y_ap, f_ap, y_g, f_g


def _check(y, fs, ry, rf, what):
    ey, ef = row_rel_err(host(y), ry), row_rel_err(host(fs), rf)
    print(f"{what}: y_err={ey:.3e} state_err={ef:.3e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (what, ey, ef)


# (batch, L, D, gate, variant, tokens_per_lane): the chunked kernel's 12-wave build
# runs up to 3072 channels, its vector-load build needs L % 8 == 0; several chunks
# of 512 tokens and a ragged tail; the token-sequential kernel with a partly idle
# last wave
CASES = [
    (2, 1096, 40, True, CHUNKED, 8),
    (1, 4096 + 40, 13, False, CHUNKED, 8),
    (2, 1032, 70, True, TOKSEQ, 4),
    (1, 296, 33, False, TOKSEQ, 4),
]


@pytest.mark.parametrize("a_kind", ["s4d", "hippo"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"-v{c[4]}")
def test_ap_path_matches_oracle_and_differs_from_general(case, a_kind):
    import torch
    batch, L, D, gate, variant, kpl = case
    inp = synth.make_scan_inputs(batch, L, D, 16, "bf16", gate=gate, d_skip="normal", seed=L + D, a_kind=a_kind)
    ry, rf = oracle_scan(inp)
    y_ap, f_ap, y_g, f_g = _both(inp, variant, kpl)
    _check(y_ap, f_ap, ry, rf, f"ap {a_kind} {case}")
    _check(y_g, f_g, ry, rf, f"general {a_kind} {case}")
    # the multiply chains round differently from direct exponentials: the float32
    # final states show that the arithmetic path ran
    assert not torch.equal(f_ap, f_g)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"-v{c[4]}")
def test_lognormal_rows_take_the_general_path(case):
    import torch
    batch, L, D, gate, variant, kpl = case
    inp = synth.make_scan_inputs(batch, L, D, 16, "bf16", gate=gate, seed=L + D + 1, a_kind="lognormal")
    y_ap, f_ap, y_g, f_g = _both(inp, variant, kpl)
    assert torch.equal(y_ap, y_g) and torch.equal(f_ap, f_g)


def test_increasing_rows_take_the_general_path():
    """b > 0 (A[d, n] = -16 + n): the ratio would exceed 1, so the chain is not used."""
    import torch
    for variant, kpl in ((CHUNKED, 8), (TOKSEQ, 4)):
        inp = synth.make_scan_inputs(1, 704, 20, 16, "bf16", seed=3)
        inp.A = np.broadcast_to(np.arange(16, dtype=np.float32) - 16.0, (20, 16)).copy()
        y_ap, f_ap, y_g, f_g = _both(inp, variant, kpl)
        assert torch.equal(y_ap, y_g) and torch.equal(f_ap, f_g), variant


@pytest.mark.parametrize("variant,kpl,group", [(CHUNKED, 8, 1), (TOKSEQ, 4, 16)])
def test_detection_granularity(variant, kpl, group):
    """One element of channel 5's A row moved by one ulp: that channel (chunked) or
    its 16-channel wave (token-sequential) runs the general path bit for bit, and the
    other channels still take the arithmetic path."""
    import torch
    D = 40
    inp = synth.make_scan_inputs(2, 904, D, 16, "bf16", seed=11)
    inp.A = inp.A.copy()
    inp.A[5, 9] = np.nextafter(inp.A[5, 9], np.float32(0.0))
    ry, rf = oracle_scan(inp)
    y_ap, f_ap, y_g, f_g = _both(inp, variant, kpl)
    _check(y_ap, f_ap, ry, rf, f"ap one-ulp row v{variant}")
    lo = (5 // group) * group
    hi = min(lo + group, D)
    assert torch.equal(f_ap[:, lo:hi], f_g[:, lo:hi]) and torch.equal(y_ap[:, lo:hi], y_g[:, lo:hi])
    rest = [d for d in range(D) if not lo <= d < hi]
    assert all(not torch.equal(f_ap[:, d], f_g[:, d]) for d in rest[:8])


def test_scalar_load_build_has_no_arithmetic_path():
    """L % 8 != 0: the chunked kernel's scalar-load build, general path only."""
    import torch
    inp = synth.make_scan_inputs(2, 1100, 30, 16, "bf16", seed=4)
    y_ap, f_ap, y_g, f_g = _both(inp, CHUNKED, 8)
    assert torch.equal(y_ap, y_g) and torch.equal(f_ap, f_g)


@pytest.mark.parametrize("variant,kpl", [(CHUNKED, 8), (TOKSEQ, 4), (0, 0)])
def test_float32_ignores_the_flag(variant, kpl):
    import torch
    inp = synth.make_scan_inputs(2, 600, 24, 16, "f32", seed=7)
    y_ap, f_ap, y_g, f_g = _both(inp, variant, kpl)
    assert torch.equal(y_ap, y_g) and torch.equal(f_ap, f_g)
