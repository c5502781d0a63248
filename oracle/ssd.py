"""Plain, sequential float64 definition of the Mamba-2 SSD scan (scalar decay per head).

TEST INFRASTRUCTURE ONLY (see the package docstring): the GPU library never
imports this module, and this module never imports the GPU library.

For batch b, time t, head h, head channel p (< P) and state n (< N):

  Delta[b,t,h] = softplus(dt[b,t,h] + dt_bias[h])        (without softplus if the flag is off)
  a[b,t,h]     = exp(Delta[b,t,h] * A[h])                 one scalar decay per head and token
  h[b,t,h,p,n] = a * h[b,t-1,h,p,n] + Delta[b,t,h] * x[b,t,h,p] * B[b,t,n]
  y[b,t,h,p]   = sum_n C[b,t,n] * h[b,t,h,p,n] + D[h] * x[b,t,h,p]
  final        = h[b,L-1]                                 h[b,-1] = h0 (0 if absent)

This is the recurrence of the slide deck's "Mamba-2" table (h_t = A_t h_{t-1} + B_t x_t
with A_t a scalar per head) and of the interview-prep page's "Mamba-2 and State Space
Duality" (A-bar_t = a_t I), with each head's state a P x N matrix (the prep page's
"per-head matrices" row) and Delta-scaled input and exp(Delta A) decay as in the
Mamba-1 scan.  B and C are shared by all heads of a batch row.

Memory order (the pages' (batch, L, ...) order): x, y [batch][L][H][P]; dt [batch][L][H];
B, C [batch][L][N]; A, D, dt_bias [H]; states [batch][H][P][N].
"""
from __future__ import annotations

import numpy as np

from .ssm import softplus


def ssd_scan(x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True, h0=None):
    """Return (y [batch][L][H][P], final_state [batch][H][P][N]) in float64.

    A plain loop over time, vectorised over (batch, head, channel, state)."""
    x = np.asarray(x, dtype=np.float64)
    Bt, L, H, P = x.shape
    Bm = np.asarray(B, dtype=np.float64)
    Cm = np.asarray(C, dtype=np.float64)
    N = Bm.shape[2]
    A = np.asarray(A, dtype=np.float64)
    assert Bm.shape == (Bt, L, N) and Cm.shape == (Bt, L, N) and A.shape == (H,)
    raw = np.asarray(dt, dtype=np.float64)
    if dt_bias is not None:
        raw = raw + np.asarray(dt_bias, dtype=np.float64)[None, None, :]
    delta = softplus(raw) if dt_softplus else raw                        # [Bt, L, H]
    h = np.zeros((Bt, H, P, N)) if h0 is None else np.array(h0, dtype=np.float64)
    y = np.empty((Bt, L, H, P))
    for t in range(L):
        a = np.exp(delta[:, t, :] * A[None, :])                          # [Bt, H]
        inp = (delta[:, t, :, None] * x[:, t])[..., None] * Bm[:, t, None, None, :]
        h = a[:, :, None, None] * h + inp
        y[:, t] = np.einsum("bhpn,bn->bhp", h, Cm[:, t])
    if D is not None:
        y = y + np.asarray(D, dtype=np.float64)[None, None, :, None] * x
    return y, h


def ssd_step(state, x_t, dt_t, A, B_t, C_t, D=None, dt_bias=None, dt_softplus=True):
    """One recurrent step of ``ssd_scan`` from ``state`` [S][H][P][N]: returns
    (y_t [S][H][P], new_state)."""
    y, h = ssd_scan(np.asarray(x_t)[:, None], np.asarray(dt_t)[:, None], A, np.asarray(B_t)[:, None],
                    np.asarray(C_t)[:, None], D, dt_bias, dt_softplus, h0=state)
    return y[:, 0], h
