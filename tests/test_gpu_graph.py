"""Every entry point captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Each replay must equal the eager call bit for bit, also with eager library calls on
other inputs, unrelated device work and synchronizations between the replays, and
with the outputs overwritten with NaN before each replay (so a replay that skipped
a write would show).  The library launches only its own kernels (no memset, copy or
allocation), so its calls can be captured as they are.  Every buffer a graph
touches (inputs, outputs, workspaces) is kept referenced for the graph's lifetime:
torch.cuda.graph empties the allocator cache on entry, and memory freed while a
graph still uses it would be handed back to the driver.
"""
import numpy as np
import pytest

import synth
from gpu_util import dev, upload_scan

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_state_space_68_amd import load_library
    load_library()


def _replay_and_check(capture, outputs, refs, between, before=None):
    """capture(): the library calls to record, writing `outputs` (a dict of tensors);
    refs: the eager results under the same keys; between(): eager work run between
    replays; before(): eager set-up run before each replay (e.g. an in-place state)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture()
    for r in range(REPLAYS):
        for t in outputs.values():
            t.fill_(float("nan"))
        if before is not None:
            before()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, ref in refs.items():
            assert torch.equal(outputs[k], ref), (k, r)
        between()
        torch.cuda.synchronize()
    return g


def _other_work():
    import torch
    a = torch.randn(1 << 20, device="cuda")
    (a * 2.0 + 1.0).sum().item()


@pytest.mark.parametrize("kind", ["chunked", "tokseq", "zoh"])
def test_scan_graph_replays(kind):
    import torch
    from selective_state_space_68_amd import selective_scan_fwd
    dtype = "bf16" if kind == "tokseq" else "f32"
    inp = synth.make_scan_inputs(2, 1040, 40, 16, dtype, gate=True, seed=31, a_kind="lognormal")
    other = synth.make_scan_inputs(2, 1040, 40, 16, dtype, gate=True, seed=32, a_kind="lognormal")
    t, t2 = upload_scan(inp), upload_scan(other)
    # (the ZOH call runs the automatic choice: the chunked kernel at this size)
    kw = dict(discretization="zoh") if kind == "zoh" else dict(variant=3 if kind == "tokseq" else 2)

    def call(tt, **extra):
        return selective_scan_fwd(tt["u"], tt["delta"], tt["A"], tt["B"], tt["C"], tt["D"], tt["z"], tt["bias"],
                                  True, **kw, **extra)

    y_ref, f_ref = call(t)
    out = {"y": torch.empty_like(y_ref), "fs": torch.empty_like(f_ref)}
    _replay_and_check(lambda: call(t, y=out["y"], final_state=out["fs"]), out, {"y": y_ref, "fs": f_ref},
                      lambda: (call(t2), _other_work()))


def test_conv_graph_replays():
    import torch
    from selective_state_space_68_amd import causal_conv1d, selective_scan_fwd_conv
    inp = synth.make_scan_inputs(2, 1032, 24, 16, "bf16", gate=True, seed=33)
    t = upload_scan(inp)
    w, cb = synth.make_conv_params(24, 4, seed=34)
    tw, tcb = dev(w), dev(cb)
    y_ref, f_ref, u_ref = selective_scan_fwd_conv(t["u"], tw, tcb, t["delta"], t["A"], t["B"], t["C"], t["D"],
                                                  t["z"], t["bias"], return_u=True)
    c_ref = causal_conv1d(t["u"], tw, tcb)
    out = {"y": torch.empty_like(y_ref), "fs": torch.empty_like(f_ref), "u": torch.empty_like(u_ref),
           "c": torch.empty_like(c_ref)}

    def capture():
        selective_scan_fwd_conv(t["u"], tw, tcb, t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["bias"],
                                u_out=out["u"], y=out["y"], final_state=out["fs"])
        causal_conv1d(t["u"], tw, tcb, out=out["c"])

    _replay_and_check(capture, out, {"y": y_ref, "fs": f_ref, "u": u_ref, "c": c_ref},
                      lambda: (causal_conv1d(t["delta"], tw, tcb), _other_work()))


def test_decode_graph_replays():
    import torch
    from selective_state_space_68_amd import state_update
    S, D, N = 8, 128, 16
    A, Dsk, bias = synth.make_decode_params(S, D, N, seed=35)
    st0 = dev(synth.make_decode_state(S, D, N, seed=35))
    x = synth.make_decode_step(S, D, N, 0, "bf16", True, seed=35)
    tx = {k: dev(x.dev[k]) for k in ("u", "delta", "B", "C", "z")}
    tA, tD, tb = dev(A), dev(Dsk), dev(bias)
    ref_state = st0.clone()
    y_ref = state_update(ref_state, tx["u"], tx["delta"], tA, tx["B"], tx["C"], tD, tx["z"], tb, True)
    state = st0.clone()
    out = {"y": torch.empty_like(y_ref)}
    scratch_state = st0.clone()

    def capture():
        state_update(state, tx["u"], tx["delta"], tA, tx["B"], tx["C"], tD, tx["z"], tb, True, y=out["y"])

    # the step updates the state in place: every replay starts from the same state
    _replay_and_check(capture, out, {"y": y_ref}, lambda: (
        state_update(scratch_state, tx["delta"], tx["u"], tA, tx["C"], tx["B"], tD, tx["z"], tb, True),
        _other_work()), before=lambda: state.copy_(st0))
    assert torch.equal(state, ref_state)


def test_backward_graph_replays():
    import torch
    from selective_state_space_68_amd import selective_scan_bwd, selective_scan_bwd_workspace_size
    inp = synth.make_scan_inputs(2, 1100, 24, 16, "f32", gate=True, seed=36)
    _, dyup, dfin = synth.make_scan_cotangents(2, 1100, 24, 16, "f32", seed=36, with_dfinal=True)
    t = upload_scan(inp)
    dy, dF = dev(dyup), dev(dfin)
    ws = torch.empty(selective_scan_bwd_workspace_size(2, 1100, 24, 16, torch.float32), dtype=torch.uint8,
                     device="cuda")

    def call(**extra):
        return selective_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, t["D"], t["z"], t["bias"], True,
                                  dfinal_state=dF, workspace=ws, **extra)

    ref = {k: v for k, v in call().items() if v is not None}
    out = {k: torch.empty_like(v) for k, v in ref.items()}
    _replay_and_check(lambda: call(out=out), out, ref, lambda: (call(), _other_work()))


def test_ssd_graph_replays():
    import torch
    from selective_state_space_68_amd import ssd_scan_fwd, ssd_scan_workspace_size
    b, L, H, P, N = 1, 1100, 4, 64, 64
    inp = synth.make_ssd_inputs(b, L, H, P, N, "bf16", seed=37, with_h0=True)
    t = {k: dev(inp.dev[k]) for k in ("x", "dt", "B", "C")}
    A, Dk, bias, h0 = dev(inp.A), dev(inp.D), dev(inp.dt_bias), dev(inp.h0)
    nbytes = ssd_scan_workspace_size(b, L, H, P, N)
    assert nbytes > 0                                               # the segmented path is the one captured
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def call(**extra):
        return ssd_scan_fwd(t["x"], t["dt"], A, t["B"], t["C"], Dk, bias, True, initial_state=h0, workspace=ws,
                            **extra)

    y_ref, f_ref = call()
    out = {"y": torch.empty_like(y_ref), "fs": torch.empty_like(f_ref)}
    _replay_and_check(lambda: call(y=out["y"], final_state=out["fs"]), out, {"y": y_ref, "fs": f_ref},
                      lambda: (call(), _other_work()))
