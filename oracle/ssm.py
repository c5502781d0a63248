"""Plain, sequential float64 definition of the selective scan and its decode step.

TEST INFRASTRUCTURE ONLY (see the package docstring): the GPU library never
imports this module, and this module never imports the GPU library.

What is computed, for batch b, time t, channel d, state n (all in float64, on the
exact values the device receives):

  delta'[b,t,d] = delta_raw[b,t,d] + bias[d]                     (bias = 0 if absent)
  Delta[b,t,d]  = softplus(delta') if the flag is set, else delta'
  abar          = exp(Delta * A[d,n])                            zero-order-hold decay
  bbar*u        = Delta * B[b,t,n] * u[b,t,d]                    simplified input term
  h[b,t,d,n]    = abar * h[b,t-1,d,n] + Delta * B[b,t,n] * u[b,t,d],  h[b,-1] = h0 (0)
  y[b,t,d]      = sum_n C[b,t,n] * h[b,t,d,n] + Dskip[d] * u[b,t,d]
  y            <- y * silu(z[b,t,d])                              if z is given
  final[b,d,n]  = h[b,L-1,d,n]

Sources, by page and section:
  * the recurrence, the readout after the update and the zero initial state follow
    the interview-prep page's "Selective scan pseudo-code" and the slide deck's
    "Mamba selective" listing (decay exp(Delta*A), input term Delta*B);
  * Delta = softplus(W x + b) with the bias added before the softplus is the
    interview-prep page's "Discretization and initialization details";
  * the skip term D*u is the output equation y = Cx + Du of the slide deck's S4
    section; the SiLU(z) gate multiplies the SSM output (lecture notes §6 "The
    block"; interview-prep page "The Mamba Block").
  Readings taken where the pages are silent: the gate multiplies (C.h + D.u), the
  softplus has no threshold, SiLU(z) = z / (1 + exp(-z)).

Full zero-order hold (``discretization="zoh"``): the input term becomes
  bbar*u        = (exp(Delta*A) - 1) / A * B[b,t,n] * u[b,t,d]   (Delta*B*u where A = 0)
which is the exact solution over one step of h' = A h + B u with u, B held
constant, the (Delta A)^-1 (exp(Delta A) - I) Delta B of the slide deck's S4
section and the lecture notes' §3 "Discretisation" for a diagonal A.

Memory order: u, delta, z are [batch][D][L] (as in the library); B, C are
[batch][L][N] (the pages' order, as in the library); A is [D][N]; Dskip and bias
are [D].
"""
from __future__ import annotations

import numpy as np


def softplus(x):
    """log(1 + e^x) in float64, written in the overflow-free form max(x,0) + log1p(e^-|x|)."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z), float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def _input_scale(dt, A, discretization):
    """Factor multiplying B*u in the input term, [.., D, N] from Delta [.., D] and A [D, N].

    "simplified": Delta.  "zoh": expm1(Delta*A)/A, whose limit at A = 0 is Delta."""
    dA = dt[..., None] * A
    if discretization == "simplified":
        return np.broadcast_to(dt[..., None], dA.shape)
    if discretization == "zoh":
        safe = np.where(A == 0.0, 1.0, A)
        return np.where(A == 0.0, dt[..., None], np.expm1(dA) / safe)
    raise ValueError(f"unknown discretization {discretization!r}")


def _step_delta(delta_raw, bias, delta_softplus):
    d = np.asarray(delta_raw, dtype=np.float64)
    if bias is not None:
        d = d + bias
    return softplus(d) if delta_softplus else d


def selective_scan(u, delta, A, B, C, Dskip=None, z=None, delta_bias=None,
                   delta_softplus=True, h0=None, discretization="simplified"):
    """Return (y [batch][D][L], final_state [batch][D][N]) in float64.

    A plain loop over time, vectorised over (batch, channel, state).
    """
    u = np.asarray(u, dtype=np.float64)
    Bt, Dc, L = u.shape
    A = np.asarray(A, dtype=np.float64)
    N = A.shape[1]
    Bm = np.asarray(B, dtype=np.float64)
    Cm = np.asarray(C, dtype=np.float64)
    assert A.shape == (Dc, N) and Bm.shape == (Bt, L, N) and Cm.shape == (Bt, L, N)
    delta = np.asarray(delta, dtype=np.float64)
    bias = None if delta_bias is None else np.asarray(delta_bias, dtype=np.float64)[None, :]
    Dv = None if Dskip is None else np.asarray(Dskip, dtype=np.float64)[None, :]

    h = np.zeros((Bt, Dc, N)) if h0 is None else np.array(h0, dtype=np.float64)
    y = np.empty((Bt, Dc, L))
    for t in range(L):
        dt = _step_delta(delta[:, :, t], bias, delta_softplus)          # [Bt, Dc]
        abar = np.exp(dt[:, :, None] * A[None, :, :])                   # [Bt, Dc, N]
        scale = _input_scale(dt, A[None, :, :], discretization)          # Delta, or expm1(Delta A)/A
        inp = scale * u[:, :, t, None] * Bm[:, t, None, :]              # Bbar*u
        h = abar * h + inp
        yt = np.einsum("bdn,bn->bd", h, Cm[:, t, :])
        if Dv is not None:
            yt = yt + Dv * u[:, :, t]
        y[:, :, t] = yt
    if z is not None:
        y = y * silu(z)
    return y, h


def selective_scan_magnitude(u, delta, A, B, C, Dskip=None, z=None, delta_bias=None,
                             delta_softplus=True, h0=None, discretization="simplified"):
    """Return (m [batch][D][L], m_final [batch][D][N]): the size of the summands of each
    output of selective_scan, in float64.

    The state recurrence is run on absolute values, H_t = exp(Delta*A) H_{t-1} + |bbar*u|
    (the decay is positive), from H_{-1} = |h0|, and each output's readout is sized the same
    way: m = (sum_n |C| H + |D u|) |SiLU(z)|.  Every term a floating-point evaluation of y adds
    up is bounded by m, so an evaluation in precision eps is off by a small multiple of eps*m.
    This is the scale for comparing outputs that cancel to near zero, where a relative error
    is undefined; the pages fix no error metric, so the scale is a reading (the test's own).
    The operations follow selective_scan's step by step, so with nonnegative inputs
    m == y and m_final == final exactly.
    """
    u = np.asarray(u, dtype=np.float64)
    Bt, Dc, L = u.shape
    A = np.asarray(A, dtype=np.float64)
    N = A.shape[1]
    Bm = np.asarray(B, dtype=np.float64)
    Cm = np.abs(np.asarray(C, dtype=np.float64))
    delta = np.asarray(delta, dtype=np.float64)
    bias = None if delta_bias is None else np.asarray(delta_bias, dtype=np.float64)[None, :]
    Dv = None if Dskip is None else np.asarray(Dskip, dtype=np.float64)[None, :]

    H = np.zeros((Bt, Dc, N)) if h0 is None else np.abs(np.array(h0, dtype=np.float64))
    m = np.empty((Bt, Dc, L))
    for t in range(L):
        dt = _step_delta(delta[:, :, t], bias, delta_softplus)
        abar = np.exp(dt[:, :, None] * A[None, :, :])
        scale = _input_scale(dt, A[None, :, :], discretization)
        inp = np.abs(scale * u[:, :, t, None] * Bm[:, t, None, :])
        H = abar * H + inp
        mt = np.einsum("bdn,bn->bd", H, Cm[:, t, :])
        if Dv is not None:
            mt = mt + np.abs(Dv * u[:, :, t])
        m[:, :, t] = mt
    if z is not None:
        m = m * np.abs(silu(z))
    return m, H


def state_update(state, u_t, delta_t, A, B_t, C_t, Dskip=None, z_t=None,
                 delta_bias=None, delta_softplus=True, discretization="simplified"):
    """One recurrent decode step: returns (y_t [S][D], new_state [S][D][N]) in float64.

    The same step as one iteration of ``selective_scan`` started from ``state``.
    """
    h = np.asarray(state, dtype=np.float64)
    u_t = np.asarray(u_t, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    bias = None if delta_bias is None else np.asarray(delta_bias, dtype=np.float64)[None, :]
    dt = _step_delta(delta_t, bias, delta_softplus)                       # [S, D]
    abar = np.exp(dt[:, :, None] * A[None, :, :])
    scale = _input_scale(dt, A[None, :, :], discretization)
    inp = scale * u_t[:, :, None] * np.asarray(B_t, dtype=np.float64)[:, None, :]
    h = abar * h + inp
    y = np.einsum("sdn,sn->sd", h, np.asarray(C_t, dtype=np.float64))
    if Dskip is not None:
        y = y + np.asarray(Dskip, dtype=np.float64)[None, :] * u_t
    if z_t is not None:
        y = y * silu(z_t)
    return y, h


def causal_conv1d(x, w, b=None, apply_silu=True):
    """Depthwise causal convolution along L, then SiLU: returns [batch][D][L] float64.

    out[b,d,t] = sum_{k<K} w[d,k] * x[b,d,t-K+1+k] + b[d]   (x = 0 before t = 0)

    The branch of the Mamba block in front of the selective SSM: a depthwise
    (per-channel) 1-D convolution of width K (4 in the models) followed by SiLU
    (dileepadev "Mamba Architecture", SSM block internals; vanos001 "The Mamba
    Block" diagram and its model card's d_conv).  Causal: output t sees inputs up
    to t only, as the recurrence that consumes it does.  w[d, K-1] weighs the
    current token.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    Bt, Dc, L = x.shape
    K = w.shape[1]
    assert w.shape == (Dc, K)
    xp = np.concatenate([np.zeros((Bt, Dc, K - 1)), x], axis=2)     # left zero padding
    out = np.zeros((Bt, Dc, L))
    for k in range(K):
        out += w[None, :, k, None] * xp[:, :, k:k + L]
    if b is not None:
        out += np.asarray(b, dtype=np.float64)[None, :, None]
    return silu(out) if apply_silu else out



def selective_scan_bwd(u, delta, A, B, C, dy, Dskip=None, z=None, delta_bias=None,
                       delta_softplus=True, h0=None, dfinal=None):
    """Gradients of sum(dy * y) + sum(dfinal * final) for (y, final) =
    selective_scan(...), float64 (dfinal None: the final state is not used).

    Returns a dict with du, ddelta (w.r.t. the raw delta), dA, dB, dC, dD, dz,
    ddelta_bias and dh0, each shaped like its input (None where the input is None).

    The reverse-time (adjoint) recurrence of the same linear system: with
    g_t = dy_t * SiLU(z_t) the gradient of the pre-gate output,
    lam_t = g_t C_t + abar_{t+1} lam_{t+1} is the gradient of the state h_t, and
    every parameter's gradient is a sum over t of lam_t (or g_t) times the partial
    derivative of one step.  This is the backward pass that recomputes the states
    instead of storing them (slide deck "Mamba selective"; blog "Hardware-Aware
    Parallel Scan"), written plainly: the forward states are kept here.
    """
    u = np.asarray(u, dtype=np.float64)
    Bt, Dc, L = u.shape
    A = np.asarray(A, dtype=np.float64)
    N = A.shape[1]
    Bm = np.asarray(B, dtype=np.float64)
    Cm = np.asarray(C, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    raw = np.asarray(delta, dtype=np.float64)
    if delta_bias is not None:
        raw = raw + np.asarray(delta_bias, dtype=np.float64)[None, :, None]
    dlt = softplus(raw) if delta_softplus else raw                     # [Bt, Dc, L]
    Dv = np.zeros(Dc) if Dskip is None else np.asarray(Dskip, dtype=np.float64)

    # forward, keeping every state and the pre-gate output
    hs = np.empty((L + 1, Bt, Dc, N))
    hs[0] = 0.0 if h0 is None else np.asarray(h0, dtype=np.float64)
    abar = np.exp(dlt[..., None] * A[None, :, None, :])                # [Bt, Dc, L, N]
    for t in range(L):
        hs[t + 1] = abar[:, :, t] * hs[t] + (dlt[:, :, t] * u[:, :, t])[..., None] * Bm[:, t, None, :]
    ytil = np.einsum("tbdn,btn->bdt", hs[1:], Cm) + Dv[None, :, None] * u

    if z is not None:
        zz = np.asarray(z, dtype=np.float64)
        sig = 1.0 / (1.0 + np.exp(-zz))
        g = dy * zz * sig                                              # dy * SiLU(z)
        dz = dy * ytil * sig * (1.0 + zz * (1.0 - sig))                # dy * ytil * SiLU'(z)
    else:
        g = dy
        dz = None

    du = Dv[None, :, None] * g
    ddl = np.zeros((Bt, Dc, L))
    dA = np.zeros((Dc, N))
    dB = np.zeros((Bt, L, N))
    dC = np.zeros((Bt, L, N))
    # abar_{t+1} * lam_{t+1}; past the last token it is the final state's cotangent
    lam_next = np.zeros((Bt, Dc, N)) if dfinal is None else np.array(dfinal, dtype=np.float64)
    for t in range(L - 1, -1, -1):
        lam = g[:, :, t, None] * Cm[:, t, None, :] + lam_next          # dL/dh_t
        dC[:, t] = np.einsum("bd,bdn->bn", g[:, :, t], hs[t + 1])
        dB[:, t] = np.einsum("bdn,bd->bn", lam, dlt[:, :, t] * u[:, :, t])
        du[:, :, t] += dlt[:, :, t] * np.einsum("bdn,bn->bd", lam, Bm[:, t])
        da = lam * hs[t]                                               # dL/dabar_t
        ddl[:, :, t] = (np.einsum("bdn,bn->bd", lam, Bm[:, t]) * u[:, :, t]
                        + np.einsum("bdn,bdn->bd", da * abar[:, :, t], np.broadcast_to(A, da.shape)))
        dA += np.einsum("bdn,bd->dn", da * abar[:, :, t], dlt[:, :, t])
        lam_next = abar[:, :, t] * lam
    dh0 = lam_next if h0 is not None else None
    ddraw = ddl * (1.0 / (1.0 + np.exp(-raw))) if delta_softplus else ddl
    return {
        "du": du, "ddelta": ddraw, "dA": dA, "dB": dB, "dC": dC,
        "dD": None if Dskip is None else np.einsum("bdt,bdt->d", g, u),
        "dz": dz,
        "ddelta_bias": None if delta_bias is None else ddraw.sum(axis=(0, 2)),
        "dh0": dh0,
    }
