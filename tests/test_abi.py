"""C-ABI tests that need no GPU: the library loads, exports every declared entry
point, and rejects bad arguments with the documented status before touching a
device.  Pointers here are fake addresses; no call reaches a kernel launch.
"""
import ctypes
import os
import re

import pytest

from selective_state_space_68_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

F = 0x10000          # fake, 64 KiB-aligned device addresses, never dereferenced
MB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    return _lib.load_library()


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert {"ssm_selective_scan_fwd", "ssm_selective_scan_workspace_size", "ssm_state_update",
            "ssm_status_string", "ssm_calib_copy"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"binding lacks {n}"


def test_version_and_status_strings(lib):
    assert lib.ssm_version() == 30100
    for s in range(5):
        assert lib.ssm_status_string(s).decode().startswith(("SSM_OK", "SSM_ERR"))
    assert b"unknown" in lib.ssm_status_string(99)


def _scan_args(**kw):
    a = dict(u=F, delta=F + 1 * 64 * MB, A=F + 2 * 64 * MB, B=F + 3 * 64 * MB, C=F + 4 * 64 * MB,
             Dskip=None, z=None, bias=None, softplus=1, h0=None, y=F + 5 * 64 * MB, final=F + 6 * 64 * MB,
             batch=1, L=64, D=16, N=4, dt=0, ws=None, ws_bytes=0, variant=0, kpl=0)
    a.update(kw)
    return a


def _scan(lib, **kw):
    a = _scan_args(**kw)
    return lib.ssm_selective_scan_fwd_variant(a["u"], a["delta"], a["A"], a["B"], a["C"], a["Dskip"], a["z"],
                                              a["bias"], a["softplus"], a["h0"], a["y"], a["final"], a["batch"],
                                              a["L"], a["D"], a["N"], a["dt"], a["ws"], a["ws_bytes"], None,
                                              a["variant"], a["kpl"])


def _scan_plain(lib, **kw):
    """ssm_selective_scan_fwd itself (no initial state, automatic kernel)."""
    a = _scan_args(**kw)
    return lib.ssm_selective_scan_fwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["Dskip"], a["z"], a["bias"],
                                      a["softplus"], a["y"], a["final"], a["batch"], a["L"], a["D"], a["N"],
                                      a["dt"], a["ws"], a["ws_bytes"], None)


def _scan_from_state(lib, **kw):
    a = _scan_args(**kw)
    return lib.ssm_selective_scan_fwd_from_state(a["u"], a["delta"], a["A"], a["B"], a["C"], a["Dskip"], a["z"],
                                                 a["bias"], a["softplus"], a["h0"], a["y"], a["final"],
                                                 a["batch"], a["L"], a["D"], a["N"], a["dt"], a["ws"],
                                                 a["ws_bytes"], None)


def _step(lib, **kw):
    a = dict(sin=F, sout=F + 1 * 64 * MB, u=F + 2 * 64 * MB, delta=F + 3 * 64 * MB, A=F + 4 * 64 * MB,
             B=F + 5 * 64 * MB, C=F + 6 * 64 * MB, Dskip=None, z=None, bias=None, softplus=1,
             y=F + 7 * 64 * MB, batch=4, D=8, N=16, dt=1)
    a.update(kw)
    return lib.ssm_state_update(a["sin"], a["sout"], a["u"], a["delta"], a["A"], a["B"], a["C"], a["Dskip"],
                                a["z"], a["bias"], a["softplus"], a["y"], a["batch"], a["D"], a["N"], a["dt"],
                                None)


@pytest.mark.parametrize("kw,status", [
    (dict(u=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(y=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(A=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(batch=-1), _lib.SSM_ERR_INVALID_ARG),
    (dict(L=-5), _lib.SSM_ERR_INVALID_ARG),
    (dict(N=0), _lib.SSM_ERR_UNSUPPORTED),
    (dict(N=65), _lib.SSM_ERR_UNSUPPORTED),
    (dict(dt=7), _lib.SSM_ERR_UNSUPPORTED),
    (dict(softplus=2), _lib.SSM_ERR_INVALID_ARG),
    (dict(variant=9), _lib.SSM_ERR_UNSUPPORTED),
    (dict(kpl=10), _lib.SSM_ERR_UNSUPPORTED),
    (dict(u=F + 2), _lib.SSM_ERR_INVALID_ARG),                       # misaligned f32
    (dict(dt=1, u=F + 1), _lib.SSM_ERR_INVALID_ARG),                 # misaligned bf16
    (dict(y=F), _lib.SSM_ERR_INVALID_ARG),                           # y aliases u
    (dict(y=F + 4 * 64 * MB + 128), _lib.SSM_ERR_INVALID_ARG),       # y overlaps C
    (dict(final=F + 2 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),         # final state aliases A
    (dict(final=F + 5 * 64 * MB + 64), _lib.SSM_ERR_INVALID_ARG),    # final state overlaps y
    (dict(batch=1 << 40, L=1 << 40), _lib.SSM_ERR_INVALID_ARG),      # size overflow
    (dict(B=F + 3 * 64 * MB + 2), _lib.SSM_ERR_INVALID_ARG),         # misaligned B
    (dict(final=F + 3 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),         # final state aliases B
    (dict(h0=F + 7 * 64 * MB + 2), _lib.SSM_ERR_INVALID_ARG),        # misaligned initial state
    (dict(h0=F + 5 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),            # initial state aliases y
    (dict(h0=F + 1 * 64 * MB + 64), _lib.SSM_ERR_INVALID_ARG),       # initial state overlaps delta
    (dict(h0=F + 6 * 64 * MB + 16), _lib.SSM_ERR_INVALID_ARG),       # partly overlaps the final state
    (dict(ws_bytes=1024), _lib.SSM_ERR_INVALID_ARG),                 # workspace size without a workspace
    (dict(ws=F + 7 * 64 * MB + 8, ws_bytes=1024), _lib.SSM_ERR_INVALID_ARG),   # workspace not 16-byte aligned
    (dict(ws=F + 3 * 64 * MB, ws_bytes=1024), _lib.SSM_ERR_INVALID_ARG),       # workspace aliases B
    (dict(ws=F + 5 * 64 * MB - 512, ws_bytes=1024), _lib.SSM_ERR_INVALID_ARG),  # workspace runs into y
])
def test_scan_argument_errors(lib, kw, status):
    assert _scan(lib, **kw) == status
    # the named entry points validate the same way (the initial state only where taken)
    if "h0" not in kw and "variant" not in kw and "kpl" not in kw:
        assert _scan_plain(lib, **kw) == status
    if "variant" not in kw and "kpl" not in kw:
        assert _scan_from_state(lib, **kw) == status


def test_scan_workspace_size(lib):
    ws = lib.ssm_selective_scan_workspace_size
    F32, BF16 = _lib.SSM_F32, _lib.SSM_BF16
    # every forward kernel keeps its carry in registers: no workspace at any shape
    for shape in ((1, 64, 16, 4), (2, 2048, 1536, 16), (8, 2048, 4096, 16), (1, 131072, 2560, 16), (1, 1, 1, 64)):
        assert ws(*shape, F32) == 0 and ws(*shape, BF16) == 0
    assert ws(1, 64, 16, 4, 7) == 0                                  # bad dtype
    assert ws(-1, 64, 16, 4, F32) == 0 and ws(1, 64, 16, 65, F32) == 0


def test_scan_empty_inputs_are_noops(lib):
    assert _scan(lib, batch=0) == _lib.SSM_OK
    assert _scan(lib, D=0) == _lib.SSM_OK
    assert _scan(lib, batch=0, u=None, delta=None, y=None, B=None, C=None) == _lib.SSM_OK
    assert _scan_plain(lib, batch=0) == _lib.SSM_OK
    assert _scan_from_state(lib, D=0) == _lib.SSM_OK


@pytest.mark.parametrize("kw,status", [
    (dict(sin=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(y=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(N=0), _lib.SSM_ERR_UNSUPPORTED),
    (dict(N=100), _lib.SSM_ERR_UNSUPPORTED),
    (dict(D=-1), _lib.SSM_ERR_INVALID_ARG),
    (dict(sout=F + 16), _lib.SSM_ERR_INVALID_ARG),                   # partial overlap of state
    (dict(y=F + 64), _lib.SSM_ERR_INVALID_ARG),                      # y inside the state
    (dict(sout=F + 2 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),          # state_out aliases u_t
    (dict(u=F + 2 * 64 * MB + 1), _lib.SSM_ERR_INVALID_ARG),         # misaligned bf16
    (dict(dt=5), _lib.SSM_ERR_UNSUPPORTED),
])
def test_state_update_argument_errors(lib, kw, status):
    assert _step(lib, **kw) == status


def _conv(lib, **kw):
    a = dict(x=F, w=F + 1 * 64 * MB, b=None, K=4, silu=1, out=F + 2 * 64 * MB, batch=2, D=8, L=64, dt=0)
    a.update(kw)
    return lib.ssm_causal_conv1d_fwd(a["x"], a["w"], a["b"], a["K"], a["silu"], a["out"], a["batch"], a["D"],
                                     a["L"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(w=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(K=0), _lib.SSM_ERR_UNSUPPORTED),
    (dict(K=5), _lib.SSM_ERR_UNSUPPORTED),
    (dict(silu=3), _lib.SSM_ERR_INVALID_ARG),
    (dict(out=F), _lib.SSM_ERR_INVALID_ARG),                         # in place is not allowed
    (dict(out=F + 2 * 64 * MB + 2), _lib.SSM_ERR_INVALID_ARG),       # misaligned
    (dict(L=-1), _lib.SSM_ERR_INVALID_ARG),
])
def test_conv_argument_errors(lib, kw, status):
    assert _conv(lib, **kw) == status


def _scan_conv(lib, **kw):
    a = dict(x=F, w=F + 7 * 64 * MB, cb=None, K=4, delta=F + 1 * 64 * MB, A=F + 2 * 64 * MB, B=F + 3 * 64 * MB,
             C=F + 4 * 64 * MB, Dskip=None, z=None, bias=None, softplus=1, h0=None, u_out=None,
             y=F + 5 * 64 * MB, final=F + 6 * 64 * MB, batch=1, L=64, D=16, N=4, dt=0, kpl=0)
    a.update(kw)
    return lib.ssm_selective_scan_fwd_conv(a["x"], a["w"], a["cb"], a["K"], a["delta"], a["A"], a["B"], a["C"],
                                           a["Dskip"], a["z"], a["bias"], a["softplus"], a["h0"], a["u_out"],
                                           a["y"], a["final"], a["batch"], a["L"], a["D"], a["N"], a["dt"], None,
                                           a["kpl"])


@pytest.mark.parametrize("kw,status", [
    (dict(w=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(K=7), _lib.SSM_ERR_UNSUPPORTED),
    (dict(kpl=12), _lib.SSM_ERR_UNSUPPORTED),
    (dict(u_out=F + 5 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),         # u_out aliases y
    (dict(u_out=F), _lib.SSM_ERR_INVALID_ARG),                       # u_out aliases x
    (dict(u_out=F + 7 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),         # u_out aliases the taps
    (dict(y=F + 7 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),             # y overlaps the taps
    (dict(x=None), _lib.SSM_ERR_INVALID_ARG),
])
def test_scan_conv_argument_errors(lib, kw, status):
    assert _scan_conv(lib, **kw) == status


def _bwd(lib, **kw):
    slots = ["u", "delta", "A", "B", "C", "Dskip", "z", "bias", "h0", "dy", "dfinal",
             "du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dbias", "dh0", "ws"]
    a = {k: F + i * 64 * MB for i, k in enumerate(slots)}
    a.update(Dskip=None, z=None, bias=None, h0=None, dfinal=None, dD=None, dz=None, dbias=None, dh0=None,
             softplus=1, batch=1, L=64, D=16, N=4, dt=0, ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = lib.ssm_selective_scan_bwd_workspace_size(a["batch"], a["L"], a["D"], a["N"], a["dt"])
    return lib.ssm_selective_scan_bwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["Dskip"], a["z"], a["bias"],
                                      a["softplus"], a["h0"], a["dy"], a["dfinal"], a["du"], a["ddelta"], a["dA"],
                                      a["dB"], a["dC"], a["dD"], a["dz"], a["dbias"], a["dh0"], a["batch"], a["L"],
                                      a["D"], a["N"], a["dt"], a["ws"], a["ws_bytes"], None)


def test_bwd_workspace_size(lib):
    ws = lib.ssm_selective_scan_bwd_workspace_size
    assert ws(0, 64, 16, 4, 0) == 0 and ws(1, 0, 16, 4, 0) == 0 and ws(1, 64, 0, 4, 0) == 0
    assert ws(1, 64, 16, 0, 0) == 0 and ws(1, 64, 16, 65, 0) == 0 and ws(1, 64, 16, 4, 5) == 0
    # at least the chunk states (3 x batch*chunks*D*N floats) and one float32 copy of
    # dB and dC (batch*2*N*L floats); the same for both activation dtypes
    for batch, L, D, N in ((2, 2048, 1536, 16), (1, 1000, 7, 5), (3, 100, 40, 20)):
        ch = 512 if N <= 16 else 256
        nc = -(-L // ch)
        floats = 3 * batch * nc * D * N + batch * 2 * N * L
        assert ws(batch, L, D, N, 0) >= 4 * floats
        assert ws(batch, L, D, N, 0) == ws(batch, L, D, N, 1)
        assert ws(batch, 2 * L, D, N, 0) > ws(batch, L, D, N, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(u=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(dy=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(du=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(ddelta=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(dA=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(dB=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(dC=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(ws=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(ws_bytes=64), _lib.SSM_ERR_INVALID_ARG),                 # workspace too small
    (dict(ws=F + 21 * 64 * MB + 8), _lib.SSM_ERR_INVALID_ARG),      # workspace not 16-byte aligned
    (dict(dz=F + 30 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),          # dz without z
    (dict(du=F), _lib.SSM_ERR_INVALID_ARG),                         # output aliases u
    (dict(dB=F + 11 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),          # output aliases another output
    (dict(ws=F + 9 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),           # workspace aliases dy
    (dict(dh0=F + 8 * 64 * MB, h0=F + 8 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),  # dh0 aliases h0
    (dict(dA=F + 13 * 64 * MB + 2), _lib.SSM_ERR_INVALID_ARG),      # misaligned float32 output
    (dict(dt=1, dB=F + 14 * 64 * MB + 1), _lib.SSM_ERR_INVALID_ARG),  # misaligned bf16 output
    (dict(N=0), _lib.SSM_ERR_UNSUPPORTED),
    (dict(N=65), _lib.SSM_ERR_UNSUPPORTED),
    (dict(dt=3), _lib.SSM_ERR_UNSUPPORTED),
    (dict(softplus=5), _lib.SSM_ERR_INVALID_ARG),
    (dict(L=-1), _lib.SSM_ERR_INVALID_ARG),
])
def test_bwd_argument_errors(lib, kw, status):
    assert _bwd(lib, **kw) == status


def _bwd_saved(lib, **kw):
    """ssm_selective_scan_bwd_saved: the _bwd arguments plus the saved chunk states."""
    slots = ["u", "delta", "A", "B", "C", "Dskip", "z", "bias", "h0", "dy", "dfinal",
             "du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dbias", "dh0", "ws"]
    a = {k: F + i * 64 * MB for i, k in enumerate(slots)}
    a.update(Dskip=None, z=None, bias=None, h0=None, dfinal=None, dD=None, dz=None, dbias=None, dh0=None,
             softplus=1, batch=1, L=64, D=16, N=4, dt=0, ws_bytes=None, cs=F + 22 * 64 * MB)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = lib.ssm_selective_scan_bwd_saved_workspace_size(a["batch"], a["L"], a["D"], a["N"],
                                                                        a["dt"])
    return lib.ssm_selective_scan_bwd_saved(a["u"], a["delta"], a["A"], a["B"], a["C"], a["Dskip"], a["z"],
                                            a["bias"], a["softplus"], a["h0"], a["dy"], a["dfinal"], a["cs"],
                                            a["du"], a["ddelta"], a["dA"], a["dB"], a["dC"], a["dD"], a["dz"],
                                            a["dbias"], a["dh0"], a["batch"], a["L"], a["D"], a["N"], a["dt"],
                                            a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(u=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(dy=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(ws=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(ws_bytes=64), _lib.SSM_ERR_INVALID_ARG),
    (dict(du=F), _lib.SSM_ERR_INVALID_ARG),
    (dict(cs=None), _lib.SSM_ERR_INVALID_ARG),                      # the saved states are required
    (dict(cs=F + 22 * 64 * MB + 2), _lib.SSM_ERR_INVALID_ARG),      # misaligned saved states
    (dict(cs=F + 11 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),          # saved states alias an output (du)
    (dict(cs=F + 20 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),          # ... or the workspace
    (dict(N=65), _lib.SSM_ERR_UNSUPPORTED),
    (dict(L=-1), _lib.SSM_ERR_INVALID_ARG),
])
def test_bwd_saved_argument_errors(lib, kw, status):
    assert _bwd_saved(lib, **kw) == status


def test_bwd_saved_workspace_size(lib):
    plain = lib.ssm_selective_scan_bwd_workspace_size
    saved = lib.ssm_selective_scan_bwd_saved_workspace_size
    # shapes that run the plain decomposition: the same size
    for shape in ((2, 2048, 1536, 16), (1, 1000, 7, 5), (8, 2048, 4096, 24)):
        assert saved(*shape, 1) == plain(*shape, 1)
    # the chunk walk (N <= 16 and batch * D >= 16384): at least the carried adjoints
    # (batch*D*N floats), the dA partials (batch*chunks*D*N) and one float32 dB, dC
    # copy (batch*2*N*L); no per-chunk entering states (batch*chunks*D*N)
    for batch, L, D, N in ((8, 2048, 4096, 16), (1, 1100, 16384, 16), (4, 2056, 4100, 5)):
        nc = -(-L // 512)
        assert saved(batch, L, D, N, 1) >= 4 * (batch * D * N + batch * nc * D * N + batch * 2 * N * L)
        assert saved(batch, L, D, N, 1) == saved(batch, L, D, N, 0)
    assert saved(0, 64, 16, 4, 0) == 0 and saved(1, 64, 16, 65, 0) == 0


def _scan_save(lib, **kw):
    a = _scan_args(**kw)
    a.setdefault("cs", F + 8 * 64 * MB)
    a.update({k: v for k, v in kw.items() if k == "cs"})
    return lib.ssm_selective_scan_fwd_save(a["u"], a["delta"], a["A"], a["B"], a["C"], a["Dskip"], a["z"],
                                           a["bias"], a["softplus"], a["h0"], a["y"], a["final"], a["cs"],
                                           a["batch"], a["L"], a["D"], a["N"], a["dt"], a["ws"], a["ws_bytes"],
                                           None)


@pytest.mark.parametrize("kw,status", [
    (dict(u=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(y=F), _lib.SSM_ERR_INVALID_ARG),
    (dict(cs=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(cs=F + 8 * 64 * MB + 8), _lib.SSM_ERR_INVALID_ARG),      # saved states not 16-byte aligned
    (dict(cs=F + 5 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),          # saved states alias y
    (dict(cs=F + 4 * 64 * MB + 64), _lib.SSM_ERR_INVALID_ARG),     # ... overlap C
    (dict(N=17), _lib.SSM_ERR_UNSUPPORTED),                        # saving covers up to 16 states
    (dict(N=0, cs=None), _lib.SSM_ERR_UNSUPPORTED),                # the state count is reported first
])
def test_scan_save_argument_errors(lib, kw, status):
    assert _scan_save(lib, **kw) == status


def test_bwd_empty_channels_is_noop(lib):
    assert _bwd(lib, D=0, u=None, delta=None, dy=None, du=None, ddelta=None, dA=None, ws=None) == _lib.SSM_OK


def _ssd(lib, **kw):
    slots = ["x", "dt", "A", "B", "C", "D", "bias", "h0", "y", "fs", "ws"]
    a = {k: F + i * 64 * MB for i, k in enumerate(slots)}
    a.update(D=None, bias=None, h0=None, fs=None, softplus=1, batch=1, L=128, H=2, P=64, N=64, dt_=1,
             ws_bytes=0, ws=None)
    a.update(kw)
    return lib.ssm_ssd_scan_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["bias"], a["softplus"], a["h0"],
                                a["y"], a["fs"], a["batch"], a["L"], a["H"], a["P"], a["N"], a["dt_"], a["ws"],
                                a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(y=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(A=None), _lib.SSM_ERR_INVALID_ARG),
    (dict(x=F + 8), _lib.SSM_ERR_INVALID_ARG),                     # x not 16-byte aligned
    (dict(y=F), _lib.SSM_ERR_INVALID_ARG),                         # y aliases x
    (dict(fs=F + 8 * 64 * MB), _lib.SSM_ERR_INVALID_ARG),           # final state aliases y
    (dict(ws=F + 10 * 64 * MB, ws_bytes=64 * MB + 1), _lib.SSM_ERR_INVALID_ARG),   # workspace runs into... nothing
    (dict(ws=None, ws_bytes=256), _lib.SSM_ERR_INVALID_ARG),        # size without a pointer
    (dict(ws=F + 1 * 64 * MB, ws_bytes=1024), _lib.SSM_ERR_INVALID_ARG),  # workspace aliases dt
    (dict(P=32), _lib.SSM_ERR_UNSUPPORTED),
    (dict(N=16), _lib.SSM_ERR_UNSUPPORTED),
    (dict(dt_=0), _lib.SSM_ERR_UNSUPPORTED),                       # float32 activations
    (dict(L=-1), _lib.SSM_ERR_INVALID_ARG),
    (dict(softplus=3), _lib.SSM_ERR_INVALID_ARG),
])
def test_ssd_argument_errors(lib, kw, status):
    st = _ssd(lib, **kw)
    if kw.get("ws_bytes") == 64 * MB + 1:
        assert st == _lib.SSM_ERR_HIP                               # a large, separate workspace is fine
    else:
        assert st == status


def test_ssd_workspace_size(lib):
    ws = lib.ssm_ssd_scan_workspace_size
    assert ws(2, 4096, 64, 64, 64, 1) > 0                          # 128 (batch, head) pairs: segments help
    assert ws(4, 2048, 80, 64, 64, 1) == 0                         # 320 pairs fill the chip: one segment
    assert ws(1, 64, 2, 64, 64, 1) == 0                            # a single chunk: nothing to split
    assert ws(4, 2048, 80, 64, 64, 0) == 0 and ws(4, 2048, 80, 32, 64, 1) == 0
    assert _ssd(lib) == _lib.SSM_ERR_HIP                            # valid arguments reach the device probe
    assert _ssd(lib, batch=0) == _lib.SSM_OK


@pytest.mark.parametrize("batch,L,H,N,segments", [
    (4, 2048, 80, 64, 1),     # the 2.7B-shaped workload: 320 workgroups already fill the chip
    (2, 4096, 64, 64, 4),     # 128 (batch, head) pairs: 4 segments of 16 chunks, 512 workgroups
    (1, 8192, 24, 64, 19),    # 128 chunks: 21 segments would be of 7, and 19 of 7 cover them
    (1, 8320, 24, 64, 19),    # 130 chunks: 19 segments of 7 (21 of 7 would leave 2 empty)
    (1, 2085, 2, 64, 7),      # 33 chunks: 7 segments of 5 (8 of 5 would leave the last empty)
    (1, 16384, 16, 64, 32),   # 256 chunks in 32 segments of 8
    (1, 8192, 8, 128, 32),    # N = 128 holds one workgroup per CU: 32 segments of 4
    (4, 2048, 80, 128, 3),    # N = 128 past one wave (320 pairs): about 768 workgroups, 3 segments
    (8, 2048, 80, 64, 1),     # N = 64 past one wave (640 pairs): one segment
])
def test_ssd_segments_never_empty(lib, batch, L, H, N, segments):
    # The workspace holds one P x N state and one decay per (batch, head, segment),
    # plus 256 bytes, so its size gives the segment count (no workspace: one
    # segment).  Every segment must hold a chunk: a segment starting at or past L
    # would have nothing to load.
    P = 64
    size = lib.ssm_ssd_scan_workspace_size(batch, L, H, P, N, 1)
    per_segment = batch * H * (P * N + 1) * 4
    if size == 0:
        nseg = 1
    else:
        assert (size - 256) % per_segment == 0
        nseg = (size - 256) // per_segment
    assert nseg == segments
    nch = (L + 63) // 64
    per = (nch + nseg - 1) // nseg
    assert (nseg - 1) * per < nch                                   # the last segment starts inside L


def test_scan_kernel_choice(lib):
    """The kernel query (host-only) follows the documented choice: the token-sequential
    kernel for N = 16 from 32768 channels, the chunked kernel otherwise, and the
    explicit variants as asked."""
    k = lib.ssm_selective_scan_fwd_kernel
    F32, BF16 = _lib.SSM_F32, _lib.SSM_BF16
    SEQ, CHK, TOK = _lib.SSM_SCAN_SEQUENTIAL, _lib.SSM_SCAN_CHUNKED, _lib.SSM_SCAN_TOKSEQ
    assert k(2, 2048, 1536, 16, F32, 1, 0, 0, 0, 0) == CHK                # 130M-shaped
    assert k(8, 2048, 4096, 16, BF16, 1, 0, 0, 0, 0) == TOK               # 1.4B-shaped: 32768 channels
    assert k(8, 2048, 4096, 16, F32, 1, 0, 0, 0, 0) == TOK
    assert k(16, 2048, 4096, 16, BF16, 1, 0, 0, 0, 0) == TOK              # 65536 channels
    assert k(2, 2048, 16383, 16, BF16, 1, 0, 0, 0, 0) == CHK              # 32766 channels
    assert k(16, 2048, 4096, 16, F32, 0, 0, 0, 0, 0) == TOK
    assert k(4, 2048, 4095, 16, BF16, 1, 0, 0, 0, 0) == CHK               # 16380 channels
    assert k(8, 2048, 4096, 8, BF16, 1, 0, 0, 0, 0) == CHK                # N != 16
    assert k(8, 2044, 4096, 16, BF16, 1, 0, 0, 0, 0) == CHK               # L % 8 != 0
    assert k(8, 2048, 4096, 16, BF16, 1, 0, 0, 0, 16) == CHK              # a chunked option pins the chunked kernel
    assert k(1, 64, 16, 4, F32, 0, 0, 0, SEQ, 0) == SEQ
    assert k(1, 64, 16, 16, F32, 0, 0, 0, TOK, 2) == TOK                  # asked for: any supported size
    assert k(1, 100, 16, 16, F32, 0, 0, 0, TOK, 0) == -_lib.SSM_ERR_UNSUPPORTED
    assert k(1, 64, 16, 16, F32, 0, 0, 0, TOK, 8) == -_lib.SSM_ERR_UNSUPPORTED   # states per lane: 2 or 4
    assert k(1, 64, 16, 16, BF16, 1, 0, 0, CHK, 12) == CHK                # 12 tokens per lane
    assert k(1, 64, 16, 16, BF16, 1, 0, 4, 0, 12) == -_lib.SSM_ERR_UNSUPPORTED   # not with the fused conv
    assert k(1, 64, 16, 16, BF16, 1, 1, 0, 0, 12) == -_lib.SSM_ERR_UNSUPPORTED   # nor the full ZOH
    assert k(1, 64, 16, 16, BF16, 1, 0, 0, CHK, 10) == -_lib.SSM_ERR_UNSUPPORTED
    assert k(1, 64, 16, 65, F32, 0, 0, 0, 0, 0) == -_lib.SSM_ERR_UNSUPPORTED
    assert k(1, 64, 16, 16, F32, 0, 0, 0, 7, 0) == -_lib.SSM_ERR_UNSUPPORTED
    # the arithmetic-progression flag does not change the kernel
    AP = _lib.SSM_SCAN_AP
    assert k(8, 2048, 4096, 16, BF16, 1, 0, 0, AP, 0) == TOK
    assert k(1, 131072, 2560, 16, BF16, 1, 0, 0, AP, 0) == CHK
    assert k(1, 64, 16, 16, F32, 0, 0, 0, TOK | AP, 2) == TOK
    assert k(1, 64, 16, 16, F32, 0, 0, 0, 7 | AP, 0) == -_lib.SSM_ERR_UNSUPPORTED
    assert k(0, 64, 16, 16, F32, 0, 0, 0, 0, 0) == -_lib.SSM_ERR_INVALID_ARG
    # the full zero-order hold: token-sequential at many channels, else chunked
    assert k(8, 2048, 4096, 16, BF16, 1, 1, 0, 0, 0) == TOK
    assert k(2, 2048, 1536, 16, F32, 1, 1, 0, 0, 0) == CHK
    assert k(8, 2048, 4096, 16, BF16, 1, 1, 0, CHK, 0) == -_lib.SSM_ERR_UNSUPPORTED   # the zoh entry chooses
    # the fused conv: as the plain scan
    assert k(8, 2048, 4096, 16, BF16, 1, 0, 4, 0, 0) == TOK
    assert k(2, 2048, 1536, 16, F32, 1, 0, 4, 0, 0) == CHK
    assert k(8, 2048, 4096, 16, BF16, 1, 0, 4, 0, 8) == CHK
    assert k(8, 2048, 4096, 16, BF16, 1, 0, 5, 0, 0) == -_lib.SSM_ERR_UNSUPPORTED


def test_state_update_empty_is_noop(lib):
    assert _step(lib, batch=0) == _lib.SSM_OK


def _no_gpu():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


@pytest.mark.skipif(not _no_gpu(), reason="forces the no-device path; only meaningful without a GPU")
def test_valid_call_without_device_reports_hip_error(lib):
    # Valid arguments reach the device probe, which fails cleanly (no launch happens).
    assert _scan(lib) == _lib.SSM_ERR_HIP
    assert _scan_plain(lib) == _lib.SSM_ERR_HIP                           # the named entry point
    assert _scan_plain(lib, ws=F + 7 * 64 * MB, ws_bytes=4096) == _lib.SSM_ERR_HIP   # a spare workspace is fine
    assert _scan_from_state(lib, h0=F + 7 * 64 * MB) == _lib.SSM_ERR_HIP
    assert _scan(lib, variant=1) == _lib.SSM_ERR_HIP                      # sequential kernel
    assert _scan(lib, h0=F + 7 * 64 * MB) == _lib.SSM_ERR_HIP             # from a given state
    assert _scan(lib, h0=F + 6 * 64 * MB) == _lib.SSM_ERR_HIP             # ... updated in place
    assert _conv(lib) == _lib.SSM_ERR_HIP
    assert _scan_conv(lib) == _lib.SSM_ERR_HIP
    assert _scan_conv(lib, u_out=F + 8 * 64 * MB, cb=F + 9 * 64 * MB) == _lib.SSM_ERR_HIP
    assert _step(lib, sout=F) == _lib.SSM_ERR_HIP          # exact in-place is valid
    assert _bwd(lib) == _lib.SSM_ERR_HIP
    zoh = (F, F + 64 * MB, F + 2 * 64 * MB, F + 3 * 64 * MB, F + 4 * 64 * MB, None, None, None, 1, None,
           F + 5 * 64 * MB, F + 6 * 64 * MB, 1, 64, 16, 4, 0, None)
    assert lib.ssm_selective_scan_fwd_zoh(*zoh) == _lib.SSM_ERR_HIP
    assert lib.ssm_selective_scan_fwd_zoh(None, *zoh[1:]) == _lib.SSM_ERR_INVALID_ARG
    assert lib.ssm_selective_scan_fwd_zoh(*zoh[:15], 0, *zoh[16:]) == _lib.SSM_ERR_UNSUPPORTED   # N = 0
    step = (F, F + 64 * MB, F + 2 * 64 * MB, F + 3 * 64 * MB, F + 4 * 64 * MB, F + 5 * 64 * MB, F + 6 * 64 * MB,
            None, None, None, 1, F + 7 * 64 * MB, 4, 8, 16, 1, None)
    assert lib.ssm_state_update_zoh(*step) == _lib.SSM_ERR_HIP
    assert lib.ssm_state_update_zoh(*step[:11], None, *step[12:]) == _lib.SSM_ERR_INVALID_ARG   # y_t NULL
    assert _bwd(lib, z=F + 6 * 64 * MB, dz=F + 17 * 64 * MB, h0=F + 8 * 64 * MB, dh0=F + 19 * 64 * MB,
                dfinal=F + 10 * 64 * MB, Dskip=F + 5 * 64 * MB, dD=F + 16 * 64 * MB) == _lib.SSM_ERR_HIP
    assert _bwd(lib, L=0) == _lib.SSM_ERR_HIP               # sums over no tokens still write zeros
    assert _bwd_saved(lib) == _lib.SSM_ERR_HIP
    assert _bwd_saved(lib, batch=1, L=1100, D=16384, N=16, dt=1) == _lib.SSM_ERR_HIP    # a chunk-walk shape
    assert _scan_save(lib) == _lib.SSM_ERR_HIP
    assert _scan_save(lib, N=16, L=1024) == _lib.SSM_ERR_HIP
    with pytest.raises(_lib.SsmError) as ei:
        _lib.check(_lib.SSM_ERR_HIP)
    assert ei.value.status == _lib.SSM_ERR_HIP


def test_missing_library_fails_loudly(tmp_path):
    saved = _lib._lib
    _lib._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            _lib.load_library(str(tmp_path / "nope.so"))
    finally:
        _lib._lib = saved
