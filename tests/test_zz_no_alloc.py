"""The allocation-free SSD entry point (ssm_ssd_scan_fwd_noalloc) against
ssm_ssd_scan_fwd given a workspace of the queried size, through the C ABI: two calls
in a row on segmented shapes, the second smaller (the library's scratch array keeps
the first call's contents), each equal to the workspace call bit for bit (both use
the same segments) and within the bfloat16 bar of the oracle."""
import ctypes

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


def _call(lib, fn, t, inp, y, fs, ws=None):
    import torch
    from selective_state_space_68_amd import _lib
    b, L, H, P = inp.x.shape
    N = inp.B.shape[2]
    ptr = lambda v: None if v is None else ctypes.c_void_p(v.data_ptr())
    args = [ptr(t["x"]), ptr(t["dt"]), ptr(t["A"]), ptr(t["B"]), ptr(t["C"]), ptr(t["D"]), ptr(t["bias"]), 1,
            ptr(t["h0"]), ptr(y), ptr(fs), b, L, H, P, N, _lib.SSM_BF16]
    if ws is not None:
        args += [ptr(ws), ws.numel()]
    st = fn(*args, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_ssd_matches_the_workspace_call_twice():
    import torch
    from selective_state_space_68_amd import _lib, load_library
    lib = load_library()
    assert lib.ssm_status_string(_lib.SSM_ERR_TOO_LARGE).decode().startswith("SSM_ERR_TOO_LARGE")
    # (batch, L, H, N): both shapes run in segments (nonzero workspace), the second smaller
    for shape in ((1, 8192, 24, 64), (1, 1100, 3, 128)):
        b, L, H, N = shape
        need = lib.ssm_ssd_scan_workspace_size(b, L, H, 64, N, _lib.SSM_BF16)
        assert need > 0 and need <= (64 << 20), need
        inp = synth.make_ssd_inputs(b, L, H, 64, N, "bf16", seed=L + H, with_h0=True)
        t = {k: dev(inp.dev[k]) for k in ("x", "dt", "B", "C")}
        t.update(A=dev(inp.A), D=dev(inp.D), bias=dev(inp.dt_bias), h0=dev(inp.h0))
        y0 = torch.full_like(t["x"], float("nan"))
        f0 = torch.full((b, H, 64, N), float("nan"), dtype=torch.float32, device="cuda")
        y1, f1 = torch.full_like(y0, 3.0), torch.full_like(f0, 3.0)
        ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")
        assert _call(lib, lib.ssm_ssd_scan_fwd, t, inp, y0, f0, ws) == _lib.SSM_OK
        assert _call(lib, lib.ssm_ssd_scan_fwd_noalloc, t, inp, y1, f1) == _lib.SSM_OK
        torch.cuda.synchronize()
        assert torch.equal(y0, y1) and torch.equal(f0, f1), shape
        ry, rf = oracle.ssd_scan(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.dt_bias, h0=inp.h0)
        ey = row_rel_err(host(y1).transpose(0, 2, 3, 1), ry.transpose(0, 2, 3, 1))
        ef = row_rel_err(host(f1), rf)
        print(f"noalloc ssd {shape}: {need} scratch bytes, y_err={ey:.2e} state_err={ef:.2e}", flush=True)
        assert ey <= TOL["bf16"] and ef <= TOL["bf16"]
    # argument errors come back before anything runs
    assert _call(lib, lib.ssm_ssd_scan_fwd_noalloc, dict(t, x=None), inp, y1, f1) == _lib.SSM_ERR_INVALID_ARG
