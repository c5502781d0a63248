"""Pins of the float64 oracle against facts that do not come from the oracle itself.

Each test checks the oracle against something the pages or the mathematics fix:
a worked example printed on a page, an independently written closed form, the
convolution form of the time-invariant case, the masked quadratic (dual) form of
the scalar-decay case, limits with exact answers, and structural invariants.
Together they fail for a dropped term, a wrong sign, a shifted time index, a
swapped B/C, a bias applied after the softplus or a gate applied before the skip.
"""
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth
from ssm_metrics import row_rel_err

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _softplus_lib(x):
    # numpy's log(e^0 + e^x): a library routine, not the oracle's formula
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def _silu_lib(z):
    z = np.asarray(z, dtype=np.float64)
    return z * expit(z)


def brute_force(u, delta, A, B, C, Dskip=None, z=None, bias=None, softplus=True, h0=None):
    """Unrolled closed form with no recurrence.

    h[t,n] = exp(A_n S_t) h0_n + sum_{s<=t} exp(A_n (S_t - S_s)) Delta_s B[s,n] u_s,
    with S the running sum of Delta (S_t includes step t).
    """
    u = np.asarray(u, np.float64)
    Bt, Dc, L = u.shape
    N = A.shape[1]
    y = np.zeros((Bt, Dc, L))
    hf = np.zeros((Bt, Dc, N))
    for b in range(Bt):
        for d in range(Dc):
            raw = np.asarray(delta[b, d], np.float64) + (0.0 if bias is None else float(bias[d]))
            dl = _softplus_lib(raw) if softplus else raw
            S = np.cumsum(dl)
            for t in range(L):
                h = np.zeros(N)
                if h0 is not None:
                    h += np.exp(A[d].astype(np.float64) * S[t]) * h0[b, d]
                for s in range(t + 1):
                    h += np.exp(A[d].astype(np.float64) * (S[t] - S[s])) * dl[s] * B[b, s].astype(np.float64) * u[b, d, s]
                yt = float(np.dot(C[b, t].astype(np.float64), h))
                if Dskip is not None:
                    yt += float(Dskip[d]) * u[b, d, t]
                if z is not None:
                    yt *= float(_silu_lib(z[b, d, t]))
                y[b, d, t] = yt
                if t == L - 1:
                    hf[b, d] = h
    return y, hf


def _run_oracle(inp, **kw):
    return oracle.selective_scan(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z,
                                 inp.delta_bias, inp.delta_softplus, **kw)


# ---------------------------------------------------------------- worked example

def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "worked_example.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                tok, dl, ab = line.split()
                rows.append((int(tok), float(dl), float(ab)))
    return rows


def test_worked_example_decay_via_decode_step():
    """Abar = exp(Delta*A): a unit state with no input decays to the printed value."""
    for _, dl, printed in _golden_rows():
        y, h = oracle.state_update(np.ones((1, 1, 1)), np.zeros((1, 1)), np.array([[dl]]),
                                   np.array([[-1.0]]), np.zeros((1, 1)), np.ones((1, 1)),
                                   delta_softplus=False)
        assert abs(h[0, 0, 0] - printed) <= 5e-4, (dl, h[0, 0, 0], printed)
        assert abs(y[0, 0] - printed) <= 5e-4


def test_worked_example_decay_via_scan():
    """Write a unit state at token 1, then watch tokens 2 and 3 decay it."""
    rows = _golden_rows()
    dls = np.array([r[1] for r in rows])
    u = np.array([[[1.0, 0.0, 0.0]]])
    B = np.array([[[1.0 / dls[0]], [0.0], [0.0]]])      # Delta_1 * B_1 * u_1 = 1
    C = np.ones((1, 3, 1))
    y, hf = oracle.selective_scan(u, dls[None, None, :], np.array([[-1.0]]), B, C,
                                  delta_softplus=False)
    assert abs(y[0, 0, 0] - 1.0) < 1e-15
    assert abs(y[0, 0, 1] / y[0, 0, 0] - rows[1][2]) <= 5e-4
    assert abs(y[0, 0, 2] / y[0, 0, 1] - rows[2][2]) <= 5e-4
    assert hf[0, 0, 0] == y[0, 0, 2]


# ---------------------------------------------------------------- softplus / silu

def test_softplus_against_library_and_identity():
    x = np.concatenate([np.linspace(-40, 40, 2001), [-800.0, -1e-300, 0.0, 1e-300, 800.0, 1e-8, -1e-8]])
    sp = oracle.softplus(x)
    ref = _softplus_lib(x)
    assert np.all(np.abs(sp - ref) <= 2 * np.finfo(np.float64).eps * np.maximum(np.abs(ref), 1e-300))
    assert np.allclose(sp - oracle.softplus(-x), x, rtol=0, atol=1e-12 * (1 + np.abs(x)).max())
    assert np.all(sp > np.maximum(x, 0.0)) or np.all(sp >= np.maximum(x, 0.0))
    assert oracle.softplus(200.0) == 200.0


def test_silu_against_library():
    z = np.linspace(-60, 60, 1201)
    assert np.allclose(oracle.silu(z), _silu_lib(z), rtol=1e-14, atol=1e-300)
    assert oracle.silu(0.0) == 0.0


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed,shape,gate,dskip,softplus,bias", [
    (0, (1, 12, 3, 4), False, "normal", True, True),
    (1, (2, 17, 2, 3), True, "ones", True, True),
    (2, (1, 9, 3, 1), True, "normal", False, False),
    (3, (2, 20, 1, 5), False, "none", True, False),
])
def test_oracle_matches_unrolled_closed_form(seed, shape, gate, dskip, softplus, bias):
    Bt, L, Dc, N = shape
    inp = synth.make_scan_inputs(Bt, L, Dc, N, "f32", gate=gate, d_skip=dskip, seed=seed,
                                 a_kind="lognormal", with_bias=bias, delta_softplus=softplus)
    y, hf = _run_oracle(inp)
    yb, hb = brute_force(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z,
                         inp.delta_bias, softplus)
    assert row_rel_err(y, yb) < 1e-12
    assert row_rel_err(hf, hb) < 1e-12


def test_oracle_matches_closed_form_on_tiny_workload():
    cfg = synth.CONFIGS["tiny_f32"]
    inp = synth.make_config_inputs(cfg)
    sub = slice(0, 4)
    y, hf = oracle.selective_scan(inp.u[:, sub], inp.delta[:, sub], inp.A[sub], inp.B, inp.C,
                                  inp.Dskip[sub], None, inp.delta_bias[sub], True)
    yb, hb = brute_force(inp.u[:, sub], inp.delta[:, sub], inp.A[sub], inp.B, inp.C,
                         inp.Dskip[sub], None, inp.delta_bias[sub], True)
    assert row_rel_err(y, yb) < 1e-12
    assert row_rel_err(hf, hb) < 1e-12


def test_oracle_initial_state_matches_closed_form():
    inp = synth.make_scan_inputs(2, 11, 2, 3, "f32", gate=True, seed=7, a_kind="lognormal")
    h0 = np.random.default_rng(5).standard_normal((2, 2, 3))
    y, hf = _run_oracle(inp, h0=h0)
    yb, hb = brute_force(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z,
                         inp.delta_bias, True, h0=h0)
    assert row_rel_err(y, yb) < 1e-12 and row_rel_err(hf, hb) < 1e-12


# ---------------------------------------------------------------- LTI convolution

@pytest.mark.parametrize("seed", [0, 1])
def test_time_invariant_case_is_a_causal_convolution(seed):
    """Constant Delta, B, C: y = K * u + D u with K_k = sum_n C_n Delta B_n e^{k Delta A_n}."""
    rng = np.random.default_rng(seed)
    L, N = 96, 6
    dl = 0.05 + 0.1 * rng.random()
    A = -np.exp(rng.standard_normal((1, N)))
    Bv, Cv = rng.standard_normal(N), rng.standard_normal(N)
    u = rng.standard_normal((1, 1, L))
    Dv = np.array([0.7])
    y, _ = oracle.selective_scan(u, np.full((1, 1, L), dl), A, np.tile(Bv, (1, L, 1)),
                                 np.tile(Cv, (1, L, 1)), Dv, None, None, False)
    k = np.arange(L)
    K = (Cv * dl * Bv * np.exp(k[:, None] * dl * A[0][None, :])).sum(-1)
    ref_direct = np.convolve(u[0, 0], K)[:L] + Dv[0] * u[0, 0]
    nfft = 2 * L
    ref_fft = np.fft.irfft(np.fft.rfft(u[0, 0], nfft) * np.fft.rfft(K, nfft), nfft)[:L] + Dv[0] * u[0, 0]
    assert row_rel_err(y[0, 0], ref_direct) < 1e-12
    assert row_rel_err(y[0, 0], ref_fft) < 1e-11


# ---------------------------------------------------------------- SSD dual form

def test_scalar_decay_case_equals_masked_quadratic_form():
    """A[d, n] = a_d for all n: y = tril((C B^T) o M) (Delta o u) + D u, M_ts = exp(a_d (S_t - S_s))."""
    inp = synth.make_scan_inputs(2, 40, 3, 5, "f32", gate=False, d_skip="normal", seed=11)
    a = -np.exp(np.random.default_rng(3).standard_normal(3))
    inp.A = np.repeat(a[:, None], 5, axis=1).astype(np.float32)
    y, _ = _run_oracle(inp)
    for b in range(2):
        CB = inp.C[b].astype(np.float64) @ inp.B[b].astype(np.float64).T      # [t, s]
        for d in range(3):
            dl = _softplus_lib(inp.delta[b, d].astype(np.float64) + inp.delta_bias[d])
            S = np.cumsum(dl)
            M = np.exp(float(inp.A[d, 0]) * (S[:, None] - S[None, :]))
            Y = np.tril(CB * M) @ (dl * inp.u[b, d]) + float(inp.Dskip[d]) * inp.u[b, d].astype(np.float64)
            assert row_rel_err(y[b, d], Y) < 1e-12


# ---------------------------------------------------------------- limits

def test_hold_limit_zero_step_keeps_state():
    inp = synth.make_scan_inputs(2, 33, 4, 4, "f32", gate=True, d_skip="normal", seed=4,
                                 with_bias=False, delta_softplus=False)
    inp.delta = np.zeros_like(inp.delta)
    y, hf = _run_oracle(inp)
    assert np.all(hf == 0.0)
    ref = inp.Dskip[None, :, None].astype(np.float64) * inp.u * _silu_lib(inp.z)
    assert row_rel_err(y, ref) < 1e-15
    st = np.random.default_rng(0).standard_normal((3, 4, 4))
    _, h1 = oracle.state_update(st, np.ones((3, 4)), np.zeros((3, 4)), inp.A,
                                np.ones((3, 4)), np.ones((3, 4)), delta_softplus=False)
    assert np.array_equal(h1, st)


def test_forget_limit_large_step_overwrites_state():
    """Delta = softplus(200) = 200 with A <= -1: the old state is wiped each token."""
    inp = synth.make_scan_inputs(1, 25, 3, 4, "f32", gate=False, d_skip="normal", seed=9,
                                 with_bias=False)
    inp.delta = np.full_like(inp.delta, 200.0)
    y, hf = _run_oracle(inp)
    dl = 200.0
    ref = (dl * inp.u.astype(np.float64) * np.einsum("btn,btn->bt", inp.C.astype(np.float64),
                                                      inp.B.astype(np.float64))[:, None, :]
           + inp.Dskip[None, :, None].astype(np.float64) * inp.u)
    assert row_rel_err(y, ref) < 1e-12
    assert row_rel_err(hf, dl * inp.B[:, -1, None, :].astype(np.float64) * inp.u[:, :, -1, None]) < 1e-12


def test_gate_and_skip_special_cases():
    inp = synth.make_scan_inputs(1, 20, 3, 4, "f32", gate=True, d_skip="normal", seed=12)
    inp.z = np.zeros_like(inp.z)
    y, _ = _run_oracle(inp)
    assert np.all(y == 0.0)
    inp = synth.make_scan_inputs(1, 20, 3, 4, "f32", gate=True, d_skip="normal", seed=12)
    inp.B = np.zeros_like(inp.B)
    y, hf = _run_oracle(inp)
    assert np.all(hf == 0.0)
    assert row_rel_err(y, inp.Dskip[None, :, None].astype(np.float64) * inp.u * _silu_lib(inp.z)) < 1e-15


# ---------------------------------------------------------------- chunked composition

def _combine(first, second):
    """(a1, b1) then (a2, b2) -> (a2 a1, a2 b1 + b2): the scan's associative operator."""
    a1, b1 = first
    a2, b2 = second
    return a2 * a1, a2 * b1 + b2


@pytest.mark.parametrize("chunk", [1, 7, 64, 100])
def test_chunked_composition_equals_sequential(chunk):
    """Scan each chunk from zero, then fix it up with the carried state.

    Chunk aggregates (decay exp(A * sum Delta), end state from zero) are composed with
    the associative operator to give each chunk's incoming state; the fix-up adds
    C_t . (exp(A (S_t - S_start)) h_in).  Agreement with the plain sequential loop pins
    the operator algebra the GPU kernel is built on.
    """
    inp = synth.make_scan_inputs(2, 100, 3, 4, "f32", gate=True, seed=21, a_kind="lognormal")
    y_ref, h_ref = _run_oracle(inp)
    L = inp.L
    y = np.zeros_like(y_ref)
    carry = (np.ones((2, 3, 4)), np.zeros((2, 3, 4)))     # identity element
    for c0 in range(0, L, chunk):
        sl = slice(c0, min(L, c0 + chunk))
        yl, hl = oracle.selective_scan(inp.u[:, :, sl], inp.delta[:, :, sl], inp.A, inp.B[:, sl],
                                       inp.C[:, sl], inp.Dskip, None, inp.delta_bias, True)
        dl = _softplus_lib(inp.delta[:, :, sl].astype(np.float64) + inp.delta_bias[None, :, None])
        S = np.cumsum(dl, axis=-1)                                       # [b, d, t]
        h_in = carry[1]
        fix = np.exp(S[..., None] * inp.A[None, :, None, :]) * h_in[:, :, None, :]   # [b,d,t,n]
        y[:, :, sl] = (yl + np.einsum("bdtn,btn->bdt", fix, inp.C[:, sl].astype(np.float64))) \
            * _silu_lib(inp.z[:, :, sl])
        agg = (np.exp(S[..., -1, None] * inp.A[None]), hl)
        carry = _combine(carry, agg)
    assert row_rel_err(y, y_ref) < 1e-12
    assert row_rel_err(carry[1], h_ref) < 1e-12


def test_scan_then_decode_equals_longer_scan():
    inp = synth.make_scan_inputs(2, 30, 3, 4, "f32", gate=True, seed=31, a_kind="lognormal")
    y_ref, h_ref = _run_oracle(inp)
    k = 5
    y0, h = oracle.selective_scan(inp.u[:, :, :-k], inp.delta[:, :, :-k], inp.A, inp.B[:, :-k],
                                  inp.C[:, :-k], inp.Dskip, inp.z[:, :, :-k], inp.delta_bias, True)
    assert row_rel_err(y0, y_ref[:, :, :-k]) == 0.0
    for j in range(inp.L - k, inp.L):
        yt, h = oracle.state_update(h, inp.u[:, :, j], inp.delta[:, :, j], inp.A, inp.B[:, j],
                                    inp.C[:, j], inp.Dskip, inp.z[:, :, j], inp.delta_bias, True)
        assert np.allclose(yt, y_ref[:, :, j], rtol=1e-13, atol=1e-13 * np.abs(y_ref).max())
    assert row_rel_err(h, h_ref) < 1e-13


# ---------------------------------------------------------------- structure

def test_linear_in_u_without_gate():
    inp = synth.make_scan_inputs(1, 40, 3, 4, "f32", gate=False, d_skip="normal", seed=41)
    u2 = np.random.default_rng(1).standard_normal(inp.u.shape)
    y1, h1 = oracle.selective_scan(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, None, inp.delta_bias)
    y2, h2 = oracle.selective_scan(u2, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, None, inp.delta_bias)
    y3, h3 = oracle.selective_scan(2.0 * inp.u - 3.0 * u2, inp.delta, inp.A, inp.B, inp.C,
                                   inp.Dskip, None, inp.delta_bias)
    assert row_rel_err(y3, 2 * y1 - 3 * y2) < 1e-12
    assert row_rel_err(h3, 2 * h1 - 3 * h2) < 1e-12


def test_causal_batch_and_channel_independent():
    inp = synth.make_scan_inputs(2, 50, 4, 3, "f32", gate=True, d_skip="normal", seed=51)
    y, hf = _run_oracle(inp)
    u = inp.u.copy()
    u[:, :, 30] += 1.0
    y2, _ = oracle.selective_scan(u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, inp.delta_bias)
    assert np.array_equal(y2[:, :, :30], y[:, :, :30]) and not np.array_equal(y2[:, :, 30], y[:, :, 30])
    perm = np.array([2, 0, 3, 1])
    yp, hp = oracle.selective_scan(inp.u[:, perm], inp.delta[:, perm], inp.A[perm], inp.B, inp.C,
                                   inp.Dskip[perm], inp.z[:, perm], inp.delta_bias[perm])
    assert row_rel_err(yp, y[:, perm]) < 1e-15 and row_rel_err(hp, hf[:, perm]) < 1e-15
    y1, h1 = oracle.selective_scan(inp.u[1:], inp.delta[1:], inp.A, inp.B[1:], inp.C[1:],
                                   inp.Dskip, inp.z[1:], inp.delta_bias)
    assert row_rel_err(y1, y[1:]) < 1e-15 and row_rel_err(h1, hf[1:]) < 1e-15


# ---------------------------------------------------------------- generator

def test_generator_is_deterministic_and_bf16_exact():
    a = synth.make_scan_inputs(2, 64, 8, 4, "bf16", seed=3)
    b = synth.make_scan_inputs(2, 64, 8, 4, "bf16", seed=3)
    for name in ("u", "delta", "B", "C", "z"):
        assert np.array_equal(a.dev[name], b.dev[name])
        vals = synth.f32_from_bf16_bits(a.dev[name])
        assert np.array_equal(vals, getattr(a, name))
    c = synth.make_scan_inputs(2, 64, 8, 4, "bf16", seed=4)
    assert not np.array_equal(a.dev["u"], c.dev["u"])
    # stream independence: dropping the gate does not change the other tensors
    d = synth.make_scan_inputs(2, 64, 8, 4, "bf16", seed=3, gate=False)
    assert np.array_equal(a.dev["u"], d.dev["u"]) and np.array_equal(a.dev["C"], d.dev["C"])


def test_bf16_rounding_rule():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                     -(1.0 + 2 ** -8), 3.40282e38, np.inf, -np.inf, 0.0, -0.0, 3.3895314e38],
                    dtype=np.float32)
    bits = synth.bf16_bits_from_f32(vals)
    # ties go to even mantissa; just-above-tie rounds up; float32 max rounds to inf,
    # bfloat16's own max stays finite
    assert list(bits[:5]) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBF80]
    assert bits[5] == 0x7F80 and bits[6] == 0x7F80 and bits[7] == 0xFF80
    assert bits[8] == 0x0000 and bits[9] == 0x8000 and bits[10] == 0x7F7F
    nan = synth.bf16_bits_from_f32(np.array([np.nan], dtype=np.float32))
    assert np.isnan(synth.f32_from_bf16_bits(nan)[0])


def test_decode_steps_regenerate_independently():
    s1 = synth.make_decode_step(4, 8, 4, step=7)
    s2 = synth.make_decode_step(4, 8, 4, step=7)
    s3 = synth.make_decode_step(4, 8, 4, step=8)
    assert np.array_equal(s1.dev["u"], s2.dev["u"]) and not np.array_equal(s1.dev["u"], s3.dev["u"])


# ---------------------------------------------------------------- readout magnitude

def _brute_magnitude(u, delta, A, B, C, Dskip=None, z=None, bias=None, softplus=True, h0=None):
    """The unrolled closed form of brute_force with every summand in absolute value."""
    u = np.asarray(u, np.float64)
    Bt, Dc, L = u.shape
    N = A.shape[1]
    m = np.zeros((Bt, Dc, L))
    for b in range(Bt):
        for d in range(Dc):
            raw = np.asarray(delta[b, d], np.float64) + (0.0 if bias is None else float(bias[d]))
            dl = _softplus_lib(raw) if softplus else raw
            S = np.cumsum(dl)
            for t in range(L):
                H = np.zeros(N)
                if h0 is not None:
                    H += np.exp(A[d].astype(np.float64) * S[t]) * np.abs(h0[b, d])
                for s in range(t + 1):
                    H += np.exp(A[d].astype(np.float64) * (S[t] - S[s])) * np.abs(
                        dl[s] * B[b, s].astype(np.float64) * u[b, d, s])
                mt = float(np.dot(np.abs(C[b, t].astype(np.float64)), H))
                if Dskip is not None:
                    mt += abs(float(Dskip[d]) * u[b, d, t])
                if z is not None:
                    mt *= abs(float(_silu_lib(z[b, d, t])))
                m[b, d, t] = mt
    return m


@pytest.mark.parametrize("seed", [0, 1])
def test_magnitude_matches_unrolled_closed_form(seed):
    inp = synth.make_scan_inputs(2, 23, 3, 5, "f32", gate=True, d_skip="normal", seed=60 + seed,
                                 a_kind="lognormal")
    h0 = synth.make_scan_initial_state(2, 3, 5, seed=seed)
    m, _ = oracle.selective_scan_magnitude(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z,
                                           inp.delta_bias, True, h0=h0)
    ref = _brute_magnitude(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, inp.delta_bias, True, h0)
    assert np.max(np.abs(m - ref) / ref) < 1e-12


def test_magnitude_equals_output_for_nonnegative_inputs():
    # every summand nonnegative: the sizes add up to the output itself, bit for bit
    inp = synth.make_scan_inputs(2, 40, 4, 6, "f32", gate=True, d_skip="normal", seed=71)
    u, B, C = np.abs(inp.u), np.abs(inp.B), np.abs(inp.C)
    Dk, z = np.abs(inp.Dskip), np.abs(inp.z)
    h0 = np.abs(synth.make_scan_initial_state(2, 4, 6, seed=7))
    y, hf = oracle.selective_scan(u, inp.delta, inp.A, B, C, Dk, z, inp.delta_bias, True, h0=h0)
    m, mf = oracle.selective_scan_magnitude(u, inp.delta, inp.A, B, C, Dk, z, inp.delta_bias, True, h0=h0)
    assert np.array_equal(m, y) and np.array_equal(mf, hf)


def test_magnitude_bounds_output_and_ignores_signs():
    inp = synth.make_scan_inputs(2, 60, 5, 16, "f32", gate=True, d_skip="normal", seed=73, a_kind="lognormal")
    h0 = synth.make_scan_initial_state(2, 5, 16, seed=3)
    args = (inp.delta, inp.A)
    y, hf = oracle.selective_scan(inp.u, *args, inp.B, inp.C, inp.Dskip, inp.z, inp.delta_bias, True, h0=h0)
    m, mf = oracle.selective_scan_magnitude(inp.u, *args, inp.B, inp.C, inp.Dskip, inp.z, inp.delta_bias, True,
                                            h0=h0)
    assert np.all(m >= np.abs(y) * (1 - 1e-12)) and np.all(mf >= np.abs(hf) * (1 - 1e-12))
    assert np.mean(m > 2 * np.abs(y)) > 0.1            # cancellation: the size exceeds the value
    # flipping the signs of u, C, D and h0 changes y but not the sizes
    m2, mf2 = oracle.selective_scan_magnitude(-inp.u, *args, inp.B, -inp.C, -inp.Dskip, inp.z, inp.delta_bias,
                                              True, h0=-h0)
    assert np.allclose(m2, m, rtol=1e-13, atol=0) and np.allclose(mf2, mf, rtol=1e-13, atol=0)
