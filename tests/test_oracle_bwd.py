"""Pins of the oracle's backward pass against central finite differences of the
oracle's forward pass (float64), and against closed forms of the simplest terms.
Each gradient is checked entry by entry on tiny shapes; a dropped term, a wrong
sign, a time index off by one or a gate derivative applied at the wrong place
fails here."""
import numpy as np
import pytest

import oracle


def _inputs(seed, Bt=2, Dc=3, L=7, N=4, gate=True, bias=True, softplus=True, h0=True):
    r = np.random.default_rng(seed)
    return dict(
        u=r.standard_normal((Bt, Dc, L)),
        delta=r.standard_normal((Bt, Dc, L)) * 0.5 - (1.0 if softplus else -0.6),
        A=-np.exp(r.standard_normal((Dc, N))),
        B=r.standard_normal((Bt, L, N)),
        C=r.standard_normal((Bt, L, N)),
        Dskip=r.standard_normal(Dc),
        z=r.standard_normal((Bt, Dc, L)) if gate else None,
        delta_bias=r.standard_normal(Dc) * 0.3 if bias else None,
        delta_softplus=softplus,
        h0=r.standard_normal((Bt, Dc, N)) if h0 else None,
    )


NAMES = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "Dskip": "dD", "z": "dz",
         "delta_bias": "ddelta_bias", "h0": "dh0"}


def _loss(inp, dy, dfinal=None):
    y, fin = oracle.selective_scan(**inp)
    return float(np.sum(y * dy)) + (0.0 if dfinal is None else float(np.sum(fin * dfinal)))


@pytest.mark.parametrize("cfg", [
    dict(),
    dict(gate=False, bias=False, h0=False),
    dict(softplus=False),
    dict(L=1, N=1, Dc=1, Bt=1),
    dict(dfinal=True),
    dict(dfinal=True, h0=False, gate=False),
])
def test_gradients_match_finite_differences(cfg):
    cfg = dict(cfg)
    with_dfinal = cfg.pop("dfinal", False)
    inp = _inputs(3, **cfg)
    r = np.random.default_rng(11)
    y, fin = oracle.selective_scan(**inp)
    dy = r.standard_normal(y.shape)
    dfinal = r.standard_normal(fin.shape) if with_dfinal else None
    grads = oracle.selective_scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], dy,
                                      inp["Dskip"], inp["z"], inp["delta_bias"], inp["delta_softplus"], inp["h0"],
                                      dfinal)
    eps = 1e-6
    for name, gname in NAMES.items():
        if inp[name] is None:
            assert grads[gname] is None
            continue
        x = inp[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(inp, dy, dfinal)
            x[idx] = old - eps
            lm = _loss(inp, dy, dfinal)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - grads[gname])) / max(1.0, np.max(np.abs(fd)))
        assert err < 1e-6, (gname, err)


def test_skip_gradient_closed_form():
    # with B = 0 the state never moves: y = D u SiLU(z), so dD = sum dy u SiLU(z) and du = D dy SiLU(z)
    inp = _inputs(5)
    inp["B"] = np.zeros_like(inp["B"])
    inp["h0"] = None
    dy = np.random.default_rng(2).standard_normal(inp["u"].shape)
    g = oracle.selective_scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], dy, inp["Dskip"],
                                  inp["z"], inp["delta_bias"])
    s = inp["z"] / (1 + np.exp(-inp["z"]))
    assert np.allclose(g["dD"], np.sum(dy * inp["u"] * s, axis=(0, 2)), rtol=1e-13)
    assert np.allclose(g["du"], inp["Dskip"][None, :, None] * dy * s, rtol=1e-13)
    assert np.allclose(g["dC"], 0.0) and np.allclose(g["dA"], 0.0)
