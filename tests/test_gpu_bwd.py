"""GPU parity of the backward pass (ssm_selective_scan_bwd) against the float64
oracle's adjoint recurrence (oracle.selective_scan_bwd, itself pinned to finite
differences of the forward pass).

Every gradient is compared with the row-wise metric of the forward tests: rows
are a channel's time series (du, ddelta, dz), a state's time series in one batch
row (dB, dC), a channel's N entries (dA, dinitial_state) and the whole vector
(dD, ddelta_bias).  Tolerances are the forward pass's: 1e-4 for float32
activations, 2e-2 for bfloat16 (whose outputs are rounded to bfloat16).  Shapes
cover several chunks with a ragged tail, the non-vector path, one token, every
state-count tier (N <= 16, N <= 32 and N <= 64 hold different kernels), missing
optional inputs, a given initial state and final-state gradient, and more
channels than one workgroup covers.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, dev, host
from ssm_metrics import row_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_state_space_68_amd import load_library
    load_library()


def _case(batch, L, D, N, dtype="f32", gate=True, d_skip="ones", bias=True, softplus=True, h0=False,
          dfinal=False, seed=0, a_kind="s4d"):
    inp = synth.make_scan_inputs(batch, L, D, N, dtype, gate=gate, d_skip=d_skip, seed=seed, a_kind=a_kind,
                                 with_bias=bias, delta_softplus=softplus)
    if not softplus:
        # without the softplus the step must still be positive, or exp(Delta*A) > 1 and
        # the state grows without bound in any precision
        inp.delta = np.abs(inp.delta)
        inp.delta_bias = None
        inp.refresh()
    dyv, dyup, dfin = synth.make_scan_cotangents(batch, L, D, N, dtype, seed=seed, with_dfinal=dfinal)
    hz = synth.make_scan_initial_state(batch, D, N, seed=seed) if h0 else None
    return inp, dyv, dyup, hz, dfin


def _run_gpu(inp, dyup, hz, dfin, want_dh0=None):
    import torch
    from selective_state_space_68_amd import selective_scan_bwd
    t = {k: dev(inp.upload_array(k)) for k in ("u", "delta", "B", "C", "z")}
    g = selective_scan_bwd(t["u"], t["delta"], dev(inp.A), t["B"], t["C"], dev(dyup), dev(inp.Dskip), t["z"],
                           dev(inp.delta_bias), inp.delta_softplus, initial_state=dev(hz),
                           dfinal_state=dev(dfin), want_dinitial_state=want_dh0)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in g.items()}


def _run_oracle(inp, dyv, hz, dfin):
    return oracle.selective_scan_bwd(inp.u, inp.delta, inp.A, inp.B, inp.C, dyv, inp.Dskip, inp.z,
                                     inp.delta_bias, inp.delta_softplus, hz, dfin)


def _compare(got, ref, dtype, what, dh0_ref=None):
    tol = TOL[dtype]
    errs = {
        "du": row_rel_err(got["du"], ref["du"]),
        "ddelta": row_rel_err(got["ddelta"], ref["ddelta"]),
        "dA": row_rel_err(got["dA"], ref["dA"]),
        # dB/dC are [batch][L][N] on both sides; a row is one state's time series
        "dB": row_rel_err(got["dB"], ref["dB"], axis=1),
        "dC": row_rel_err(got["dC"], ref["dC"], axis=1),
    }
    if ref["dz"] is not None:
        errs["dz"] = row_rel_err(got["dz"], ref["dz"])
    else:
        assert got["dz"] is None
    if ref["dD"] is not None:
        errs["dD"] = row_rel_err(got["dD"], ref["dD"])
    if ref["ddelta_bias"] is not None:
        errs["ddelta_bias"] = row_rel_err(got["ddelta_bias"], ref["ddelta_bias"])
    dh0 = ref["dh0"] if dh0_ref is None else dh0_ref
    if dh0 is not None:
        errs["dh0"] = row_rel_err(got["dinitial_state"], dh0)
    print(what, " ".join(f"{k}={v:.2e}" for k, v in errs.items()), f"tol={tol:.0e}", flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, (what, bad)


CASES = [
    # batch, L, D, N, kwargs
    (1, 64, 16, 4, dict()),
    (2, 1100, 13, 16, dict()),                                   # 3 chunks, ragged tail, vector path off (L % 8)
    (2, 1536, 24, 16, dict(h0=True, dfinal=True)),
    (1, 1, 3, 16, dict()),                                       # one token
    (1, 513, 9, 16, dict(gate=False, bias=False, d_skip="none")),
    (1, 700, 5, 16, dict(softplus=False, a_kind="lognormal")),
    (2, 600, 6, 5, dict(h0=True)),                               # N not a multiple of 4
    (1, 520, 7, 24, dict(dfinal=True)),                          # 17..32 states: 4 tokens per lane
    (1, 300, 4, 40, dict(h0=True)),                              # 33..64 states: global accumulation
    (1, 256, 3, 64, dict()),
    (2, 2048, 200, 16, dict()),                                  # several channel slices and rounds
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("batch,L,D,N,kw", CASES)
def test_bwd_matches_oracle(batch, L, D, N, kw, dtype):
    inp, dyv, dyup, hz, dfin = _case(batch, L, D, N, dtype, **kw)
    got = _run_gpu(inp, dyup, hz, dfin)
    ref = _run_oracle(inp, dyv, hz, dfin)
    _compare(got, ref, dtype, f"bwd {dtype} b={batch} L={L} D={D} N={N} {kw}")


def test_bwd_dinitial_state_without_initial_state():
    # the gradient at a zero initial state is the same adjoint; the oracle reports
    # it when given an explicit zero state
    inp, dyv, dyup, _, dfin = _case(1, 700, 6, 16, "f32", dfinal=True)
    got = _run_gpu(inp, dyup, None, dfin, want_dh0=True)
    ref = _run_oracle(inp, dyv, np.zeros((1, 6, 16)), dfin)
    _compare(got, ref, "f32", "bwd dh0 at zero state")


def test_bwd_zero_length():
    import torch
    from selective_state_space_68_amd import selective_scan_bwd
    inp, _, _, hz, dfin = _case(2, 8, 4, 16, "f32", h0=True, dfinal=True)
    e = torch.empty((2, 4, 0), device="cuda")
    B0 = torch.empty((2, 0, 16), device="cuda")              # [batch][L][N]
    g = selective_scan_bwd(e, e, dev(inp.A), B0, B0, e, dev(inp.Dskip), None, dev(inp.delta_bias), True,
                           initial_state=dev(hz), dfinal_state=dev(dfin))
    torch.cuda.synchronize()
    assert np.all(host(g["dA"]) == 0) and np.all(host(g["dD"]) == 0) and np.all(host(g["ddelta_bias"]) == 0)
    assert np.array_equal(host(g["dinitial_state"]), dfin.astype(np.float64))


def test_bwd_repeatable_and_workspace_reuse():
    # every output is bitwise reproducible; a dirty, reused workspace changes nothing
    import torch
    from selective_state_space_68_amd import selective_scan_bwd, selective_scan_bwd_workspace_size
    inp, dyv, dyup, hz, dfin = _case(2, 1024, 40, 16, "bf16", h0=True, dfinal=True)
    t = {k: dev(inp.upload_array(k)) for k in ("u", "delta", "B", "C", "z")}
    n = selective_scan_bwd_workspace_size(2, 1024, 40, 16, torch.bfloat16)
    ws = torch.full((n,), 0x7f, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        g = selective_scan_bwd(t["u"], t["delta"], dev(inp.A), t["B"], t["C"], dev(dyup), dev(inp.Dskip), t["z"],
                               dev(inp.delta_bias), True, initial_state=dev(hz), dfinal_state=dev(dfin),
                               workspace=ws)
        torch.cuda.synchronize()
        outs.append({k: host(v) for k, v in g.items()})
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dinitial_state"):
        assert np.array_equal(outs[0][k], outs[1][k]), k
    ref = _run_oracle(inp, dyv, hz, dfin)
    _compare(outs[1], ref, "bf16", "bwd reused workspace")


def _run_oracle_sliced(inp, dyv, hz, dfin, step=512):
    """The oracle's adjoint over slices of channels.  Every per-channel gradient
    depends only on its own channel; dB and dC are sums over channels, so the
    slices' partial sums add up to the whole.  Keeps the oracle's stored states
    to one slice at a time."""
    D = inp.u.shape[1]
    out = None
    for d0 in range(0, D, step):
        s = slice(d0, min(D, d0 + step))
        cut = lambda x: None if x is None else x[:, s]
        vec = lambda x: None if x is None else x[s]
        r = oracle.selective_scan_bwd(inp.u[:, s], inp.delta[:, s], inp.A[s], inp.B, inp.C, dyv[:, s],
                                      vec(inp.Dskip), cut(inp.z), vec(inp.delta_bias), inp.delta_softplus,
                                      cut(hz), cut(dfin))
        if out is None:
            out = {k: (None if v is None else [v]) for k, v in r.items()}
        else:
            for k, v in r.items():
                if v is not None:
                    out[k].append(v)
    cat_axis = {"du": 1, "ddelta": 1, "dz": 1, "dh0": 1, "dA": 0, "dD": 0, "ddelta_bias": 0}
    res = {}
    for k, v in out.items():
        if v is None:
            res[k] = None
        elif k in ("dB", "dC"):
            res[k] = np.sum(v, axis=0)
        else:
            res[k] = np.concatenate(v, axis=cat_axis[k])
    return res


@pytest.mark.parametrize("batch,L,D,dtype,kw", [
    (2, 4104, 3640, "f32", dict(h0=True, dfinal=True)),
    (8, 1032, 2728, "bf16", dict()),
    (2, 1032, 1000, "f32", dict(h0=True, dfinal=True)),
    (3, 1544, 700, "bf16", dict(gate=False)),
])
def test_bwd_many_channel_chunks(batch, L, D, dtype, kw):
    """Shapes where the chunk summaries come from the token-sequential summary
    kernel.  The first two have at least 4096 (chunk, 16-channel group) pairs (one
    wave each); the last two have from 256 to 4095, where four waves take the four
    128-token quarters of a chunk and are joined.  In all of them the last 512-token
    chunk holds 8 tokens (so three of its quarters are past the end), and the last
    16-channel group is partly idle; in the first two, so is the last workgroup's
    64 channels."""
    inp, dyv, dyup, hz, dfin = _case(batch, L, D, 16, dtype, seed=D, **kw)
    got = _run_gpu(inp, dyup, hz, dfin)
    ref = _run_oracle_sliced(inp, dyv, hz, dfin)
    _compare(got, ref, dtype, f"bwd many chunks {dtype} b={batch} L={L} D={D} {kw}")


# ---- the training pair with saved chunk states ---------------------------------------

SAVE = 512


def _oracle_chunk_states(inp, hz):
    """The state entering every 512-token chunk: the oracle's scan over each chunk,
    started from the state the previous chunk ended in (entry 0: the initial state)."""
    batch, D, L = inp.u.shape
    N = inp.A.shape[1]
    h = np.zeros((batch, D, N)) if hz is None else np.asarray(hz, np.float64)
    out = []
    for t0 in range(0, L, SAVE):
        out.append(h)
        s = slice(t0, min(L, t0 + SAVE))
        _, h = oracle.selective_scan(inp.u[:, :, s], inp.delta[:, :, s], inp.A, inp.B[:, s], inp.C[:, s],
                                     inp.Dskip, None if inp.z is None else inp.z[:, :, s], inp.delta_bias,
                                     inp.delta_softplus, h0=h)
    return np.stack(out, axis=2), h                          # [batch][D][chunks][N], final state


def _run_gpu_saved(inp, dyup, hz, dfin, want_dh0=None):
    import torch
    from selective_state_space_68_amd import selective_scan_bwd, selective_scan_fwd_save
    t = {k: dev(inp.upload_array(k)) for k in ("u", "delta", "B", "C", "z")}
    y, fs, cs = selective_scan_fwd_save(t["u"], t["delta"], dev(inp.A), t["B"], t["C"], dev(inp.Dskip), t["z"],
                                        dev(inp.delta_bias), inp.delta_softplus, initial_state=dev(hz))
    g = selective_scan_bwd(t["u"], t["delta"], dev(inp.A), t["B"], t["C"], dev(dyup), dev(inp.Dskip), t["z"],
                           dev(inp.delta_bias), inp.delta_softplus, initial_state=dev(hz),
                           dfinal_state=dev(dfin), chunk_states=cs, want_dinitial_state=want_dh0)
    torch.cuda.synchronize()
    return host(y), host(fs), host(cs), {k: host(v) for k, v in g.items()}


SAVE_FWD_CASES = [
    # batch, L, D, N, dtype, kwargs; the forward kernel that saves
    (2, 1536, 24, 16, "bf16", dict(h0=True)),                  # chunked, 3 whole chunks
    (1, 2056, 40, 16, "f32", dict()),                          # chunked; last chunk 8 tokens
    (2, 1100, 13, 16, "bf16", dict(h0=True)),                  # L % 8: the sequential kernel
    (1, 1300, 9, 5, "f32", dict(h0=True, gate=False)),         # N != 16: the sequential kernel
    (2, 1032, 16400, 16, "bf16", dict(h0=True)),               # 32800 channels: the token-sequential kernel
    (1, 512, 7, 16, "f32", dict()),                            # one whole chunk: entry 0 only
    (1, 40, 3, 16, "f32", dict(h0=True)),                      # shorter than a chunk
]


@pytest.mark.parametrize("batch,L,D,N,dtype,kw", SAVE_FWD_CASES)
def test_fwd_save_chunk_states_match_oracle(batch, L, D, N, dtype, kw):
    import torch
    from selective_state_space_68_amd import selective_scan_fwd_save, selective_scan_fwd_kernel
    inp = synth.make_scan_inputs(batch, L, D, N, dtype, gate=kw.get("gate", True), seed=L + D)
    hz = synth.make_scan_initial_state(batch, D, N, seed=L) if kw.get("h0") else None
    t = {k: dev(inp.upload_array(k)) for k in ("u", "delta", "B", "C", "z")}
    y, fs, cs = selective_scan_fwd_save(t["u"], t["delta"], dev(inp.A), t["B"], t["C"], dev(inp.Dskip), t["z"],
                                        dev(inp.delta_bias), True, initial_state=dev(hz))
    torch.cuda.synchronize()
    kern = selective_scan_fwd_kernel(batch, L, D, N, torch.bfloat16 if dtype == "bf16" else torch.float32,
                                     gate=inp.z is not None)
    ref_cs, ref_fs = _oracle_chunk_states(inp, hz)
    ry, _ = oracle.selective_scan(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, inp.delta_bias, True,
                                  h0=hz)
    assert cs.shape == (batch, D, -(-L // SAVE), N)
    e_cs = row_rel_err(host(cs), ref_cs)
    e_fs = row_rel_err(host(fs), ref_fs)
    e_y = row_rel_err(host(y), ry)
    print(f"fwd_save {kern} b={batch} L={L} D={D} N={N} {dtype}: cs {e_cs:.2e} fs {e_fs:.2e} y {e_y:.2e}",
          flush=True)
    tol = TOL[dtype]
    assert e_cs <= tol and e_fs <= tol and e_y <= tol
    # entry 0 is the initial state itself (zeros without one)
    want0 = np.zeros((batch, D, N)) if hz is None else np.asarray(hz, np.float64)
    assert np.array_equal(host(cs)[:, :, 0], want0)


SAVED_BWD_CASES = [
    # batch, L, D, dtype, kwargs (N = 16); batch * D >= 16384 walks the chunks
    (1, 1100, 16384, "bf16", dict(h0=True, dfinal=True)),     # non-vector path (L % 8), ragged last chunk
    (2, 1536, 8192, "f32", dict(gate=False)),                 # vector path, 3 whole chunks
    (4, 2056, 4100, "bf16", dict(dfinal=True)),               # last chunk 8 tokens; last slice partly idle
    (2, 1032, 16400, "bf16", dict(h0=True)),                  # forward states from the token-sequential kernel
    (2, 1100, 13, "f32", dict(h0=True, dfinal=True)),         # few channels: the chunk-parallel decomposition
]


@pytest.mark.parametrize("batch,L,D,dtype,kw", SAVED_BWD_CASES)
def test_bwd_saved_matches_oracle(batch, L, D, dtype, kw):
    inp, dyv, dyup, hz, dfin = _case(batch, L, D, 16, dtype, seed=D + 1, **kw)
    _, _, _, got = _run_gpu_saved(inp, dyup, hz, dfin)
    ref = _run_oracle_sliced(inp, dyv, hz, dfin)
    _compare(got, ref, dtype, f"bwd saved {dtype} b={batch} L={L} D={D} {kw}")


def test_bwd_saved_fewer_states():
    # N = 5 (an odd count: a zero padding state) on the chunk walk, from the
    # sequential kernel's saved states
    inp, dyv, dyup, hz, dfin = _case(1, 1000, 16400, 5, "f32", seed=5, h0=True, dfinal=True)
    _, _, _, got = _run_gpu_saved(inp, dyup, hz, dfin)
    ref = _run_oracle_sliced(inp, dyv, hz, dfin)
    _compare(got, ref, "f32", "bwd saved N=5")


def test_bwd_saved_dinitial_state_without_initial_state():
    inp, dyv, dyup, _, dfin = _case(1, 1024, 16384, 16, "bf16", seed=3, dfinal=True)
    _, _, _, got = _run_gpu_saved(inp, dyup, None, dfin, want_dh0=True)
    ref = _run_oracle_sliced(inp, dyv, np.zeros((1, 16384, 16)), dfin)
    _compare(got, ref, "bf16", "bwd saved dh0 at zero state")


def test_bwd_saved_repeatable_and_workspace_reuse():
    # bitwise reproducible on the chunk walk too; a dirty, reused workspace changes nothing
    import torch
    from selective_state_space_68_amd import (selective_scan_bwd, selective_scan_bwd_workspace_size,
                                              selective_scan_fwd_save)
    batch, L, D = 2, 1024, 8192
    inp, dyv, dyup, hz, dfin = _case(batch, L, D, 16, "bf16", seed=11, h0=True, dfinal=True)
    t = {k: dev(inp.upload_array(k)) for k in ("u", "delta", "B", "C", "z")}
    _, _, cs = selective_scan_fwd_save(t["u"], t["delta"], dev(inp.A), t["B"], t["C"], dev(inp.Dskip), t["z"],
                                       dev(inp.delta_bias), True, initial_state=dev(hz))
    n = selective_scan_bwd_workspace_size(batch, L, D, 16, torch.bfloat16, saved=True)
    ws = torch.full((n,), 0x7f, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        g = selective_scan_bwd(t["u"], t["delta"], dev(inp.A), t["B"], t["C"], dev(dyup), dev(inp.Dskip), t["z"],
                               dev(inp.delta_bias), True, initial_state=dev(hz), dfinal_state=dev(dfin),
                               chunk_states=cs, workspace=ws)
        torch.cuda.synchronize()
        outs.append({k: host(v) for k, v in g.items()})
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dinitial_state"):
        assert np.array_equal(outs[0][k], outs[1][k]), k
    ref = _run_oracle_sliced(inp, dyv, hz, dfin)
    _compare(outs[1], ref, "bf16", "bwd saved reused workspace")


def test_bwd_saved_small_shape_is_the_plain_pass():
    # below 16384 channels the saved states are not read: the plain pass, bit for bit
    inp, dyv, dyup, hz, dfin = _case(2, 1100, 40, 16, "bf16", seed=2, h0=True, dfinal=True)
    _, _, _, got = _run_gpu_saved(inp, dyup, hz, dfin)
    plain = _run_gpu(inp, dyup, hz, dfin)
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dinitial_state"):
        assert np.array_equal(got[k], plain[k]), k
