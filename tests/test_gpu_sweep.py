"""A seeded random sweep of small shapes through every forward kernel and option,
judged by an error bound that holds where outputs cancel.

Each case draws a shape (L from 1 token to about two 512-token chunks past a
boundary, 1 to 64 states, up to 24 channels), a dtype, the optional inputs and an
A kind, and runs the automatic choice, the sequential kernel, the chunked kernel
at 8, 12 and 16 tokens per lane, the token-sequential kernel at 4 and 2 states per
lane (where the shape fits it) and, in bfloat16, the arithmetic-progression flag.

Every output must satisfy |y - y_oracle| <= tol * m, with m the size of its
summands (oracle.selective_scan_magnitude: the readout and the state recurrence
on absolute values), and every final state likewise against the absolute-value
state.  A float32 evaluation is within a few ulps per step of every summand, so
tol = 16 (L + N) 2^-24 for float32; bfloat16 adds the output's rounding (2^-8)
and the bfloat16 build's softplus (up to 2e-3 of the smallest steps, where
log2(1 + 2^x) loses digits).  Unlike the row-relative metric this bounds single
elements, so it holds on any seed for L = 1 and N = 1 rows whose outputs cancel.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, host

pytestmark = pytest.mark.gpu

VARIANTS = [(0, 0), (1, 0), (2, 8), (2, 12), (2, 16), (3, 4), (3, 2)]
LENGTHS = [1, 2, 7, 8, 63, 64, 65, 255, 256, 511, 512, 513, 768, 769, 1024, 1104]
STATES = [1, 2, 3, 4, 5, 8, 15, 16, 16, 16, 17, 24, 32, 33, 64]


def _cases(n=96, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        L = int(rng.choice(LENGTHS)) if rng.random() < 0.7 else int(rng.integers(1, 1200))
        out.append(dict(batch=int(rng.integers(1, 4)), L=L, D=int(rng.integers(1, 25)), N=int(rng.choice(STATES)),
                        dtype=str(rng.choice(["f32", "bf16"])), gate=bool(rng.random() < 0.6),
                        d_skip=str(rng.choice(["none", "ones", "normal"])), bias=bool(rng.random() < 0.7),
                        softplus=bool(rng.random() < 0.85), h0=bool(rng.random() < 0.4),
                        a_kind=str(rng.choice(["s4d", "hippo", "lognormal"])), seed=1000 + i))
    return out


CASES = _cases()


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_state_space_68_amd import load_library
    load_library()


def _tol(c):
    t = 16.0 * (c["L"] + c["N"]) * 2.0 ** -24
    return t + (2.0 ** -8 + 2e-3 if c["dtype"] == "bf16" else 0.0), t + (2e-3 if c["dtype"] == "bf16" else 0.0)


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"{c['batch']}x{c['L']}x{c['D']}x{c['N']}-{c['dtype']}")
def test_random_shape_every_kernel_within_summand_bound(c):
    import torch
    from selective_state_space_68_amd import SSM_SCAN_AP, SsmError, selective_scan_fwd, _lib
    inp = synth.make_scan_inputs(c["batch"], c["L"], c["D"], c["N"], c["dtype"], gate=c["gate"], d_skip=c["d_skip"],
                                 seed=c["seed"], a_kind=c["a_kind"], with_bias=c["bias"],
                                 delta_softplus=c["softplus"])
    if not c["softplus"]:
        # a positive step without the softplus (else exp(Delta A) > 1 and the state diverges)
        inp.delta = np.abs(inp.delta)
        inp.delta_bias = None
        inp.refresh()
    h0 = synth.make_scan_initial_state(c["batch"], c["D"], c["N"], seed=c["seed"]) if c["h0"] else None
    args = (inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, inp.delta_bias, c["softplus"])
    ry, rf = oracle.selective_scan(*args, h0=h0)
    m, mf = oracle.selective_scan_magnitude(*args, h0=h0)
    tol_y, tol_f = _tol(c)
    t = {k: dev(inp.upload_array(k)) for k in ("u", "delta", "B", "C", "z")}
    variants = list(VARIANTS) + ([(SSM_SCAN_AP, 0)] if c["dtype"] == "bf16" else [])
    ran, worst = [], 0.0
    for variant, kpl in variants:
        try:
            y, fs = selective_scan_fwd(t["u"], t["delta"], dev(inp.A), t["B"], t["C"], dev(inp.Dskip), t["z"],
                                       dev(inp.delta_bias), c["softplus"], initial_state=dev(h0), variant=variant,
                                       tokens_per_lane=kpl)
        except SsmError as e:
            assert e.status == _lib.SSM_ERR_UNSUPPORTED, (variant, kpl, e)
            continue
        torch.cuda.synchronize()
        ey = float(np.max(np.abs(host(y) - ry) / (tol_y * m + 1e-30)))
        ef = float(np.max(np.abs(host(fs) - rf) / (tol_f * mf + 1e-30)))
        ran.append((variant, kpl))
        worst = max(worst, ey, ef)
        assert ey <= 1.0 and ef <= 1.0, (c, variant, kpl, ey, ef)
    # the automatic choice, the sequential kernel and at least one chunked build always run
    assert (0, 0) in ran and (1, 0) in ran and any(v == 2 for v, _ in ran), ran
    print(f"{c}: {len(ran)} kernel options, worst error {worst:.3f} of the bound", flush=True)
