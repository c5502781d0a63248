"""Pins of the SSD oracle (oracle.ssd_scan) against sources independent of its code:

* the selective-scan oracle (itself pinned in test_oracle.py): with the decay A
  constant over the states of a head and Delta shared by its P channels, the SSD is
  a selective scan over H*P channels with B and C shared;
* the quadratic (dual) form of the deck's "Mamba-2" table and the prep page's
  "Mamba-2 and State Space Duality": Y = tril(C B^T o M) (Delta x) + D x with the
  decay mask M[j, i] = prod_{k=i+1..j} a_k, by matrix products;
* a chunked evaluation (intra-chunk quadratic form, inter-chunk state passing),
  the prep page's chunk-parallel row, at chunk lengths 1, 3, 64 and L;
* the step form and state continuation.
"""
import numpy as np
import pytest

import oracle


def _inputs(seed, Bt=2, L=37, H=3, P=4, N=5, h0=False, bias=True):
    r = np.random.default_rng(seed)
    return dict(
        x=r.standard_normal((Bt, L, H, P)),
        dt=r.standard_normal((Bt, L, H)) * 0.5 - 1.0,
        A=-np.exp(r.standard_normal(H)),
        B=r.standard_normal((Bt, L, N)),
        C=r.standard_normal((Bt, L, N)),
        D=r.standard_normal(H),
        dt_bias=r.standard_normal(H) * 0.3 if bias else None,
        h0=r.standard_normal((Bt, H, P, N)) if h0 else None,
    )


@pytest.mark.parametrize("h0", [False, True])
def test_ssd_equals_selective_scan_with_per_head_scalar_decay(h0):
    p = _inputs(1, h0=h0)
    Bt, L, H, P = p["x"].shape
    N = p["B"].shape[2]
    y, fin = oracle.ssd_scan(**p)
    # channel (h, p) of the selective scan: u = x[..., h, p], raw delta = dt[..., h],
    # A[(h, p), n] = A[h], bias and skip per head
    u = p["x"].transpose(0, 2, 3, 1).reshape(Bt, H * P, L)
    dl = np.repeat(p["dt"].transpose(0, 2, 1), P, axis=1)
    A1 = np.repeat(np.repeat(p["A"][:, None], N, axis=1), P, axis=0)
    h01 = None if p["h0"] is None else p["h0"].reshape(Bt, H * P, N)
    y1, f1 = oracle.selective_scan(u, dl, A1, p["B"], p["C"], np.repeat(p["D"], P), None,
                                   np.repeat(p["dt_bias"], P), True, h0=h01)
    assert np.allclose(y, y1.reshape(Bt, H, P, L).transpose(0, 3, 1, 2), rtol=1e-12, atol=1e-12)
    assert np.allclose(fin, f1.reshape(Bt, H, P, N), rtol=1e-12, atol=1e-12)


def _delta(p):
    raw = p["dt"] + (0 if p["dt_bias"] is None else p["dt_bias"][None, None, :])
    return np.logaddexp(0.0, raw)


def test_ssd_quadratic_dual_form():
    p = _inputs(2, L=23)
    y, _ = oracle.ssd_scan(**p)
    dl = _delta(p)                                                   # [Bt, L, H]
    Bt, L, H, P = p["x"].shape
    for b in range(Bt):
        for h in range(H):
            cs = np.cumsum(dl[b, :, h] * p["A"][h])                 # log of the cumulative decay
            M = np.tril(np.exp(cs[:, None] - cs[None, :]))           # prod_{k=i+1..j} a_k for j >= i
            G = (p["C"][b] @ p["B"][b].T) * M                        # [L, L]
            ref = G @ (dl[b, :, h, None] * p["x"][b, :, h]) + p["D"][h] * p["x"][b, :, h]
            assert np.allclose(y[b, :, h], ref, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("Q", [1, 3, 64, 40])
def test_ssd_chunked_form(Q):
    p = _inputs(3, L=40, h0=True)
    y, fin = oracle.ssd_scan(**p)
    dl = _delta(p)
    Bt, L, H, P = p["x"].shape
    N = p["B"].shape[2]
    for b in range(Bt):
        for h in range(H):
            S = p["h0"][b, h].copy()                                  # [P, N]
            for c0 in range(0, L, Q):
                c1 = min(L, c0 + Q)
                d = dl[b, c0:c1, h]
                cs = np.cumsum(d * p["A"][h])                        # decay from the chunk start
                M = np.tril(np.exp(cs[:, None] - cs[None, :]))
                Cc, Bc, Xc = p["C"][b, c0:c1], p["B"][b, c0:c1], d[:, None] * p["x"][b, c0:c1, h]
                yc = ((Cc @ Bc.T) * M) @ Xc + np.exp(cs)[:, None] * (Cc @ S.T) + p["D"][h] * p["x"][b, c0:c1, h]
                assert np.allclose(y[b, c0:c1, h], yc, rtol=1e-10, atol=1e-10)
                S = np.exp(cs[-1]) * S + (Xc * np.exp(cs[-1] - cs)[:, None]).T @ Bc
            assert np.allclose(fin[b, h], S, rtol=1e-10, atol=1e-10)


def test_ssd_step_and_continuation():
    p = _inputs(4, L=12)
    y, fin = oracle.ssd_scan(**p)
    q = dict(p, x=p["x"][:, :7], dt=p["dt"][:, :7], B=p["B"][:, :7], C=p["C"][:, :7])
    ya, fa = oracle.ssd_scan(**q)
    st = fa
    for t in range(7, 12):
        yt, st = oracle.ssd_step(st, p["x"][:, t], p["dt"][:, t], p["A"], p["B"][:, t], p["C"][:, t], p["D"],
                                 p["dt_bias"])
        assert np.allclose(yt, y[:, t], rtol=1e-12)
    assert np.allclose(ya, y[:, :7], rtol=1e-12) and np.allclose(st, fin, rtol=1e-12)


def test_ssd_generator_is_seeded_and_in_dtype():
    import synth
    a = synth.make_ssd_inputs(1, 8, 2, 4, 3, "bf16", seed=3, with_h0=True)
    b = synth.make_ssd_inputs(1, 8, 2, 4, 3, "bf16", seed=3, with_h0=True)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.h0, b.h0) and np.array_equal(a.dev["B"], b.dev["B"])
    assert np.array_equal(synth.f32_from_bf16_bits(a.dev["x"]), a.x)
    assert np.all(a.A <= -1.0) and np.all(a.A >= -16.0)
