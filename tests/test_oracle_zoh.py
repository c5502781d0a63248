"""Pins of the oracle's full zero-order-hold discretization (input term
(exp(Delta A) - 1)/A * B * u) against sources independent of its code:

* scipy's zero-order-hold discretization of the continuous system (the matrix
  exponential of the augmented [[A, B], [0, 0]] matrix) and its discrete-time
  simulation, on a time-invariant case;
* a numerical ODE integration of h' = A h + B_t u_t over each step of length
  Delta_t with the input held, on a selective (time-varying) case;
* the limits: at A = 0 the input term is Delta*B*u, and as Delta -> 0 the full and
  simplified forms differ by O(Delta^2);
* the decode step equals one scan step.
"""
import numpy as np
import pytest
from scipy import integrate, signal

import oracle


def _lti_inputs(seed, Dc=2, N=3, L=40):
    r = np.random.default_rng(seed)
    return dict(
        u=r.standard_normal((1, Dc, L)),
        A=-np.exp(r.standard_normal((Dc, N))),
        Bv=r.standard_normal(N),
        Cv=r.standard_normal(N),
        dt=np.exp(r.uniform(np.log(0.01), np.log(0.8), size=Dc)),
    )


def test_zoh_matches_scipy_cont2discrete_lti():
    p = _lti_inputs(1)
    Dc, L = p["u"].shape[1:]
    N = p["A"].shape[1]
    # time-invariant: constant Delta per channel (softplus off, no bias), B and C constant
    delta = np.broadcast_to(p["dt"][None, :, None], (1, Dc, L)).copy()
    Bm = np.broadcast_to(p["Bv"], (1, L, N)).copy()
    Cm = np.broadcast_to(p["Cv"], (1, L, N)).copy()
    y, _ = oracle.selective_scan(p["u"], delta, p["A"], Bm, Cm, delta_softplus=False, discretization="zoh")
    for d in range(Dc):
        Ad, Bd, Cd, Dd, _ = signal.cont2discrete((np.diag(p["A"][d]), p["Bv"][:, None], p["Cv"][None, :],
                                                 np.zeros((1, 1))), p["dt"][d], method="zoh")
        # the scan reads y_t after the update at t: y_t = C (Ad h_{t-1} + Bd u_t) = C Ad h_{t-1} + C Bd u_t
        _, yd, _ = signal.dlsim((Ad, Bd, Cd @ Ad, Cd @ Bd, p["dt"][d]), p["u"][0, d])
        assert np.allclose(y[0, d], yd[:, 0], rtol=1e-11, atol=1e-12)


def test_zoh_is_the_exact_step_of_the_continuous_system():
    # selective: Delta_t, B_t and u_t change every step; over step t the input is held
    r = np.random.default_rng(3)
    N, L = 3, 6
    A = -np.exp(r.standard_normal((1, N)))
    u = r.standard_normal((1, 1, L))
    delta = np.exp(r.uniform(np.log(0.05), np.log(1.5), size=(1, 1, L)))
    Bm = r.standard_normal((1, L, N))
    Cm = r.standard_normal((1, L, N))
    h0 = r.standard_normal((1, 1, N))
    y, fin = oracle.selective_scan(u, delta, A, Bm, Cm, delta_softplus=False, h0=h0, discretization="zoh")
    h = h0[0, 0].copy()
    for t in range(L):
        sol = integrate.solve_ivp(lambda _, x: A[0] * x + Bm[0, t] * u[0, 0, t], (0.0, delta[0, 0, t]), h,
                                  rtol=1e-12, atol=1e-13, method="DOP853")
        h = sol.y[:, -1]
        assert np.isclose(y[0, 0, t], Cm[0, t] @ h, rtol=1e-9, atol=1e-10)
    assert np.allclose(fin[0, 0], h, rtol=1e-9, atol=1e-10)


def test_zoh_limits():
    r = np.random.default_rng(5)
    Bt, Dc, L, N = 1, 3, 20, 4
    u = r.standard_normal((Bt, Dc, L))
    Bm = r.standard_normal((Bt, L, N))
    Cm = r.standard_normal((Bt, L, N))
    # A = 0: the input term is Delta*B*u in both forms (and the state only accumulates)
    A0 = np.zeros((Dc, N))
    delta = np.exp(r.uniform(-3, 0, size=(Bt, Dc, L)))
    yz, hz = oracle.selective_scan(u, delta, A0, Bm, Cm, delta_softplus=False, discretization="zoh")
    ys, hs = oracle.selective_scan(u, delta, A0, Bm, Cm, delta_softplus=False)
    assert np.array_equal(yz, ys) and np.array_equal(hz, hs)
    assert np.allclose(hz, np.einsum("bdt,btn->bdn", delta * u, Bm), rtol=1e-12)
    # Delta -> 0: (e^{x}-1)/A = Delta (1 + x/2 + ...), so the forms differ by O(Delta^2)
    A = -np.exp(r.standard_normal((Dc, N)))
    diffs = []
    for s in (1e-2, 1e-3):
        dd = np.full((Bt, Dc, 1), s)
        _, a = oracle.selective_scan(u[:, :, :1], dd, A, Bm[:, :1], Cm[:, :1], delta_softplus=False,
                                     discretization="zoh")
        _, b = oracle.selective_scan(u[:, :, :1], dd, A, Bm[:, :1], Cm[:, :1], delta_softplus=False)
        diffs.append(np.max(np.abs(a - b)))
    assert 80 < diffs[0] / diffs[1] < 120          # a tenth of Delta, a hundredth of the difference


def test_zoh_decode_step_is_one_scan_step():
    r = np.random.default_rng(7)
    S, Dc, N = 2, 5, 4
    A = -np.exp(r.standard_normal((Dc, N)))
    st = r.standard_normal((S, Dc, N))
    u, dl, z = (r.standard_normal((S, Dc)) for _ in range(3))
    Bt, Ct = r.standard_normal((S, N)), r.standard_normal((S, N))
    Dk, bias = r.standard_normal(Dc), r.standard_normal(Dc) * 0.3
    y1, h1 = oracle.state_update(st, u, dl, A, Bt, Ct, Dk, z, bias, discretization="zoh")
    y2, h2 = oracle.selective_scan(u[:, :, None], dl[:, :, None], A, Bt[:, None], Ct[:, None], Dk, z[:, :, None],
                                   bias, h0=st, discretization="zoh")
    assert np.allclose(y1, y2[:, :, 0], rtol=1e-14) and np.allclose(h1, h2, rtol=1e-14)


def test_unknown_discretization_rejected():
    with pytest.raises(ValueError):
        oracle.selective_scan(np.zeros((1, 1, 2)), np.zeros((1, 1, 2)), -np.ones((1, 1)), np.zeros((1, 2, 1)),
                              np.zeros((1, 2, 1)), discretization="bilinear")
