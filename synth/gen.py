"""Seeded input generator (numpy PCG64, one SeedSequence child per tensor).

Layouts (row-major):
  u, delta (raw, before bias/softplus), z : [batch][D][L]
  B, C                                    : [batch][L][N] (the pages' order, which
                                            both the oracle and the library take)
  A                                       : [D][N]   (float32 always)
  Dskip, delta_bias                       : [D]      (float32 always)
Decode step tensors:
  state                                   : [S][D][N] float32
  u_t, delta_t, z_t                       : [S][D]
  B_t, C_t                                : [S][N]

Distributions (the workloads' recipe): u, B, C, z ~ N(0, 1); raw delta ~ N(0, 0.5^2)
(0.5 is read as the standard deviation); the delta bias per channel is the inverse
softplus, log(expm1(dt)), of dt drawn log-uniformly in [1e-3, 1e-1]; A[d, n] = -(n+1)
("S4D-real") unless ``a_kind="hippo"`` (A[d, n] = -(2n+1)) or ``a_kind="lognormal"``
(A = -exp(N(0,1)), an input that is not an arithmetic progression along n); the skip
vector is N(0,1) or all ones.

Activations are drawn in float32 and, for bf16 workloads, rounded to bfloat16 by
round-to-nearest-even on the bit pattern.  Every float array returned here holds
exactly the values the GPU receives, so a float64 reference can consume it as is.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Fixed order of SeedSequence children; adding a tensor at the end keeps old streams.
_SCAN_STREAMS = ("u", "delta", "dt", "B", "C", "Dskip", "z", "h0", "A", "conv", "dy", "dfinal")
_STEP_STREAMS = ("u", "delta", "B", "C", "z")
_DECODE_STEP_KEY = 4


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    NaNs stay NaN (quiet bit set); overflow past the largest bf16 gives +-inf.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    is_nan = (b & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    r = np.where(is_nan, (b >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _act(x32: np.ndarray, dtype: str):
    """Return (float32 values as the GPU sees them, array to upload)."""
    if dtype == "f32":
        x32 = np.ascontiguousarray(x32, dtype=np.float32)
        return x32, x32
    if dtype == "bf16":
        bits = bf16_bits_from_f32(x32)
        return f32_from_bf16_bits(bits), bits
    raise ValueError(f"unknown activation dtype {dtype!r}")


@dataclass
class ScanInputs:
    batch: int
    L: int
    D: int
    N: int
    dtype: str
    # float32 values exactly as the device receives them
    u: np.ndarray
    delta: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    Dskip: Optional[np.ndarray]
    z: Optional[np.ndarray]
    delta_bias: Optional[np.ndarray]
    delta_softplus: bool = True
    # upload arrays (float32 for f32, uint16 bit patterns for bf16)
    dev: dict = field(default_factory=dict)

    def upload_array(self, name: str) -> Optional[np.ndarray]:
        if name in self.dev:
            return self.dev[name]
        return getattr(self, name)

    def refresh(self) -> None:
        """Re-derive the upload arrays after a caller edited the float arrays.

        Edited values must already be representable in the activation dtype.
        """
        self.dev = {}
        for name in ("u", "delta", "B", "C", "z"):
            v = getattr(self, name)
            if v is None:
                continue
            vals, up = _act(v, self.dtype)
            if not np.array_equal(vals, v.astype(np.float32), equal_nan=True):
                raise ValueError(f"{name} holds values not representable in {self.dtype}")
            setattr(self, name, vals)
            self.dev[name] = up


def make_scan_inputs(batch: int, L: int, D: int, N: int, dtype: str = "f32",
                     gate: bool = True, d_skip: str = "ones", seed: int = 0,
                     a_kind: str = "s4d", with_bias: bool = True,
                     delta_softplus: bool = True) -> ScanInputs:
    ss = np.random.SeedSequence(seed)
    kids = dict(zip(_SCAN_STREAMS, ss.spawn(len(_SCAN_STREAMS))))
    rng = {k: np.random.Generator(np.random.PCG64(v)) for k, v in kids.items()}

    u32 = rng["u"].standard_normal((batch, D, L), dtype=np.float32)
    dl32 = rng["delta"].standard_normal((batch, D, L), dtype=np.float32)
    dl32 *= np.float32(0.5)
    B32 = rng["B"].standard_normal((batch, L, N), dtype=np.float32)
    C32 = rng["C"].standard_normal((batch, L, N), dtype=np.float32)

    lo, hi = np.log(1e-3), np.log(1e-1)
    dt = np.exp(rng["dt"].uniform(lo, hi, size=D))
    bias = np.log(np.expm1(dt)).astype(np.float32) if with_bias else None

    if a_kind == "s4d":
        A = np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (D, N)).copy()
    elif a_kind == "hippo":
        A = np.broadcast_to(-(2.0 * np.arange(N, dtype=np.float32) + 1.0), (D, N)).copy()
    elif a_kind == "lognormal":
        A = (-np.exp(rng["A"].standard_normal((D, N)))).astype(np.float32)
    else:
        raise ValueError(f"unknown a_kind {a_kind!r}")

    if d_skip == "ones":
        Dsk = np.ones(D, dtype=np.float32)
    elif d_skip == "normal":
        Dsk = rng["Dskip"].standard_normal(D, dtype=np.float32)
    elif d_skip == "none":
        Dsk = None
    else:
        raise ValueError(f"unknown d_skip {d_skip!r}")

    z32 = rng["z"].standard_normal((batch, D, L), dtype=np.float32) if gate else None

    inp = ScanInputs(batch, L, D, N, dtype, u=None, delta=None, A=A, B=None, C=None,
                     Dskip=Dsk, z=None, delta_bias=bias, delta_softplus=delta_softplus)
    for name, v in (("u", u32), ("delta", dl32), ("B", B32), ("C", C32), ("z", z32)):
        if v is None:
            continue
        vals, up = _act(v, dtype)
        setattr(inp, name, vals)
        inp.dev[name] = up
        del v
    return inp


def make_scan_initial_state(batch: int, D: int, N: int, seed: int = 0) -> np.ndarray:
    """Initial state [batch][D][N] ~ N(0, 1), float32, from the seed's "h0" stream."""
    ss = np.random.SeedSequence(seed)
    kid = ss.spawn(len(_SCAN_STREAMS))[_SCAN_STREAMS.index("h0")]
    return np.random.Generator(np.random.PCG64(kid)).standard_normal((batch, D, N), dtype=np.float32)


def make_conv_params(D: int, K: int, seed: int = 0):
    """Causal conv1d taps [D][K] ~ N(0, 1/K) and bias [D] ~ N(0, 0.1^2), float32,
    from the seed's "conv" stream (the scale keeps the conv output near unit variance)."""
    ss = np.random.SeedSequence(seed)
    kid = ss.spawn(len(_SCAN_STREAMS))[_SCAN_STREAMS.index("conv")]
    r = np.random.Generator(np.random.PCG64(kid))
    w = (r.standard_normal((D, K)) / np.sqrt(K)).astype(np.float32)
    b = (r.standard_normal(D) * 0.1).astype(np.float32)
    return w, b


def make_scan_cotangents(batch: int, L: int, D: int, N: int, dtype: str = "f32", seed: int = 0,
                         with_dfinal: bool = False):
    """Output cotangents for a backward pass: dy [batch][D][L] ~ N(0, 1) in the
    activation dtype (returned as (float32 values, upload array)) and, if asked,
    dfinal [batch][D][N] ~ N(0, 1) float32 for the final state; from the seed's
    "dy" and "dfinal" streams."""
    ss = np.random.SeedSequence(seed)
    kids = dict(zip(_SCAN_STREAMS, ss.spawn(len(_SCAN_STREAMS))))
    dy32 = np.random.Generator(np.random.PCG64(kids["dy"])).standard_normal((batch, D, L), dtype=np.float32)
    vals, up = _act(dy32, dtype)
    dfin = None
    if with_dfinal:
        dfin = np.random.Generator(np.random.PCG64(kids["dfinal"])).standard_normal((batch, D, N), dtype=np.float32)
    return vals, up, dfin


_SSD_STREAMS = ("x", "dt", "dt0", "A", "B", "C", "D", "h0")
_SSD_KEY = 7


@dataclass
class SSDInputs:
    """Inputs of the Mamba-2 SSD scan (float32 values as the device receives them, and
    upload arrays).  Layouts: x [batch][L][H][P]; dt [batch][L][H]; B, C [batch][L][N];
    A, D, dt_bias [H]; h0 [batch][H][P][N]."""
    batch: int
    L: int
    H: int
    P: int
    N: int
    dtype: str
    x: np.ndarray
    dt: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    D: Optional[np.ndarray]
    dt_bias: Optional[np.ndarray]
    h0: Optional[np.ndarray] = None
    dev: dict = field(default_factory=dict)


def make_ssd_inputs(batch: int, L: int, H: int, P: int, N: int, dtype: str = "bf16", seed: int = 0,
                    with_h0: bool = False, with_D: bool = True, with_bias: bool = True) -> SSDInputs:
    """Seeded SSD inputs: x, B, C ~ N(0, 1); raw dt ~ N(0, 0.5^2) plus the per-head bias
    log(expm1(dt0)) with dt0 log-uniform in [1e-3, 1e-1] (the Mamba-1 recipe); the
    per-head decay A = -U[1, 16]; D = 1; h0 ~ N(0, 1) when asked.  Child streams of
    SeedSequence([seed, 7]) in the order x, dt, dt0, A, B, C, D, h0."""
    ss = np.random.SeedSequence([seed, _SSD_KEY])
    kids = dict(zip(_SSD_STREAMS, ss.spawn(len(_SSD_STREAMS))))
    rng = {k: np.random.Generator(np.random.PCG64(v)) for k, v in kids.items()}
    x32 = rng["x"].standard_normal((batch, L, H, P), dtype=np.float32)
    dt32 = rng["dt"].standard_normal((batch, L, H), dtype=np.float32) * np.float32(0.5)
    dt0 = np.exp(rng["dt0"].uniform(np.log(1e-3), np.log(1e-1), size=H))
    bias = np.log(np.expm1(dt0)).astype(np.float32) if with_bias else None
    A = (-rng["A"].uniform(1.0, 16.0, size=H)).astype(np.float32)
    B32 = rng["B"].standard_normal((batch, L, N), dtype=np.float32)
    C32 = rng["C"].standard_normal((batch, L, N), dtype=np.float32)
    Dv = np.ones(H, dtype=np.float32) if with_D else None
    h0 = rng["h0"].standard_normal((batch, H, P, N), dtype=np.float32) if with_h0 else None
    out = SSDInputs(batch, L, H, P, N, dtype, None, None, A, None, None, Dv, bias, h0)
    for name, v in (("x", x32), ("dt", dt32), ("B", B32), ("C", C32)):
        vals, up = _act(v, dtype)
        setattr(out, name, vals)
        out.dev[name] = up
    return out


def make_config_inputs(cfg, seed: Optional[int] = None, **kw) -> ScanInputs:
    """Inputs of a named scan workload (see synth.configs)."""
    return make_scan_inputs(cfg.batch, cfg.L, cfg.D, cfg.N, cfg.dtype, gate=cfg.gate,
                            d_skip=cfg.d_skip, seed=cfg.seed if seed is None else seed, **kw)


@dataclass
class DecodeInputs:
    """One decode step's per-token tensors (float32 values + upload arrays)."""
    u: np.ndarray
    delta: np.ndarray
    B: np.ndarray
    C: np.ndarray
    z: Optional[np.ndarray]
    dev: dict = field(default_factory=dict)

    def upload_array(self, name: str):
        return self.dev.get(name, getattr(self, name))


def make_decode_params(S: int, D: int, N: int, seed: int = 0, d_skip: str = "ones",
                       a_kind: str = "s4d"):
    """(A [D][N], Dskip [D] or None, delta_bias [D]) for a decode workload."""
    p = make_scan_inputs(1, 1, D, N, "f32", gate=False, d_skip=d_skip, seed=seed,
                         a_kind=a_kind)
    return p.A, p.Dskip, p.delta_bias


def make_decode_state(S: int, D: int, N: int, seed: int = 0) -> np.ndarray:
    """Initial decode state [S][D][N] ~ N(0, 1), float32."""
    ss = np.random.SeedSequence(seed)
    kid = dict(zip(_SCAN_STREAMS, ss.spawn(len(_SCAN_STREAMS))))["h0"]
    rng = np.random.Generator(np.random.PCG64(kid))
    return rng.standard_normal((S, D, N), dtype=np.float32)


def make_decode_step(S: int, D: int, N: int, step: int, dtype: str = "bf16",
                     gate: bool = True, seed: int = 0) -> DecodeInputs:
    """Per-token tensors of decode step ``step``; any step can be regenerated alone."""
    ss = np.random.SeedSequence([seed, _DECODE_STEP_KEY, step])
    kids = dict(zip(_STEP_STREAMS, ss.spawn(len(_STEP_STREAMS))))
    rng = {k: np.random.Generator(np.random.PCG64(v)) for k, v in kids.items()}
    raw = {
        "u": rng["u"].standard_normal((S, D), dtype=np.float32),
        "delta": rng["delta"].standard_normal((S, D), dtype=np.float32) * np.float32(0.5),
        "B": rng["B"].standard_normal((S, N), dtype=np.float32),
        "C": rng["C"].standard_normal((S, N), dtype=np.float32),
        "z": rng["z"].standard_normal((S, D), dtype=np.float32) if gate else None,
    }
    out = DecodeInputs(None, None, None, None, None)
    for name, v in raw.items():
        if v is None:
            continue
        vals, up = _act(v, dtype)
        setattr(out, name, vals)
        out.dev[name] = up
    return out
