"""Torch-facing wrappers of the C ABI: allocation, pointer and stream marshalling.

Torch is used for device memory and streams only; the arithmetic happens in
libssm.so.  Activations (u, delta, z, B, C and the outputs y) are float32 or
bfloat16 CUDA/HIP tensors of one dtype; A, D, delta_bias and states are float32.
Layouts: u, delta, z [batch, D, L]; B, C [batch, L, N]; A [D, N]; D, bias [D].

Every wrapper checks the shape of every tensor it is given, outputs included,
before it takes a single pointer: the library sees only pointers and sizes, so a
tensor smaller than its shape says would otherwise be read or written past its end.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return _lib.SSM_F32
    if t.dtype == torch.bfloat16:
        return _lib.SSM_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {t.dtype}")


def _shape(t, name: str, shape) -> None:
    """Raise ValueError unless `t` (a tensor, or None for an absent optional) has `shape`."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(int(s) for s in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _workspace(workspace, need: int, dev):
    """(pointer, bytes) of a caller's workspace tensor, or of one allocated here."""
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, {need} needed")
    return workspace.data_ptr(), nbytes


def _scan_shapes(u, delta, A, B, C, D, z, delta_bias, initial_state, y, final_state):
    """Shapes of a forward scan's tensors; returns (batch, D, L, N)."""
    if not isinstance(u, torch.Tensor) or not isinstance(A, torch.Tensor) or u.dim() != 3 or A.dim() != 2:
        raise ValueError("expected u [batch, D, L] and A [D, N]")
    batch, Dc, L = u.shape
    N = A.shape[1]
    _shape(delta, "delta", (batch, Dc, L))
    _shape(A, "A", (Dc, N))
    _shape(B, "B", (batch, L, N))
    _shape(C, "C", (batch, L, N))
    _shape(z, "z", (batch, Dc, L))
    _shape(D, "D", (Dc,))
    _shape(delta_bias, "delta_bias", (Dc,))
    _shape(initial_state, "initial_state", (batch, Dc, N))
    _shape(y, "y", (batch, Dc, L))
    _shape(final_state, "final_state", (batch, Dc, N))
    return batch, Dc, L, N


def selective_scan_workspace_size(batch, L, D, N, dtype=torch.float32) -> int:
    """Bytes of device workspace the forward scan needs for this shape (0: none)."""
    lib = _lib.load_library()
    dt = _lib.SSM_BF16 if dtype == torch.bfloat16 else _lib.SSM_F32
    return int(lib.ssm_selective_scan_workspace_size(int(batch), int(L), int(D), int(N), dt))


def selective_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, *,
                       initial_state=None, y=None, final_state=None, return_final_state=True, variant=0,
                       tokens_per_lane=0, discretization="simplified", workspace=None,
                       stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Selective scan forward.  Returns (y [batch, D, L], final_state [batch, D, N] or None).

    `initial_state` [batch, D, N] float32 starts the scan from a given state (zero
    when None); `final_state` may be the same tensor (updated in place).
    `discretization`: "simplified" (input term Delta*B*u) or "zoh" (the full
    zero-order hold, (exp(Delta*A) - 1)/A * B * u, Delta*B*u where A == 0).
    `workspace`: a device tensor of at least selective_scan_workspace_size(...)
    bytes, or None (allocated here when the size is nonzero).
    """
    if discretization not in ("simplified", "zoh"):
        raise ValueError(f"unknown discretization {discretization!r}")
    lib = _lib.load_library()
    batch, Dc, L, N = _scan_shapes(u, delta, A, B, C, D, z, delta_bias, initial_state, y, final_state)
    act = u.dtype
    dev = u.device
    if discretization == "zoh" and ((variant & ~_lib.SSM_SCAN_AP) or tokens_per_lane or workspace is not None):
        raise ValueError("the zoh scan runs the default kernel (variant=0, tokens_per_lane=0, no workspace)")
    if discretization != "zoh":
        ws_ptr, ws_bytes = _workspace(workspace, selective_scan_workspace_size(batch, L, Dc, N, act), dev)
    if y is None:
        y = torch.empty((batch, Dc, L), dtype=act, device=dev)
    if final_state is None and return_final_state:
        final_state = torch.empty((batch, Dc, N), dtype=torch.float32, device=dev)
    args = (_ptr(u, "u", act, dev), _ptr(delta, "delta", act, dev), _ptr(A, "A", torch.float32, dev),
            _ptr(B, "B", act, dev), _ptr(C, "C", act, dev), _ptr(D, "D", torch.float32, dev),
            _ptr(z, "z", act, dev), _ptr(delta_bias, "delta_bias", torch.float32, dev),
            1 if delta_softplus else 0, _ptr(initial_state, "initial_state", torch.float32, dev),
            _ptr(y, "y", act, dev), _ptr(final_state, "final_state", torch.float32, dev),
            batch, L, Dc, N, _dt(u))
    if discretization == "zoh":
        st = lib.ssm_selective_scan_fwd_zoh(*args, _stream(stream))
    else:
        st = lib.ssm_selective_scan_fwd_variant(*args, ws_ptr, ws_bytes, _stream(stream), int(variant),
                                                int(tokens_per_lane))
    _lib.check(st)
    return y, final_state


SAVE_CHUNK = 512   # tokens per saved chunk state (SSM_SAVE_CHUNK)


def selective_scan_fwd_save(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, *,
                            initial_state=None, y=None, final_state=None, chunk_states=None,
                            return_final_state=True, workspace=None, stream=None):
    """selective_scan_fwd that also stores the state entering every SAVE_CHUNK-token
    chunk, for selective_scan_bwd(..., chunk_states=...).  Returns (y, final_state or
    None, chunk_states [batch, D, ceil(L / SAVE_CHUNK), N] float32); entry 0 is the
    initial state (zeros when None).  N <= 16."""
    lib = _lib.load_library()
    batch, Dc, L, N = _scan_shapes(u, delta, A, B, C, D, z, delta_bias, initial_state, y, final_state)
    act = u.dtype
    dev = u.device
    nck = (L + SAVE_CHUNK - 1) // SAVE_CHUNK
    ws_ptr, ws_bytes = _workspace(workspace, selective_scan_workspace_size(batch, L, Dc, N, act), dev)
    if y is None:
        y = torch.empty((batch, Dc, L), dtype=act, device=dev)
    if final_state is None and return_final_state:
        final_state = torch.empty((batch, Dc, N), dtype=torch.float32, device=dev)
    if chunk_states is None:
        chunk_states = torch.empty((batch, Dc, nck, N), dtype=torch.float32, device=dev)
    _shape(chunk_states, "chunk_states", (batch, Dc, nck, N))
    st = lib.ssm_selective_scan_fwd_save(
        _ptr(u, "u", act, dev), _ptr(delta, "delta", act, dev), _ptr(A, "A", torch.float32, dev),
        _ptr(B, "B", act, dev), _ptr(C, "C", act, dev), _ptr(D, "D", torch.float32, dev),
        _ptr(z, "z", act, dev), _ptr(delta_bias, "delta_bias", torch.float32, dev), 1 if delta_softplus else 0,
        _ptr(initial_state, "initial_state", torch.float32, dev), _ptr(y, "y", act, dev),
        _ptr(final_state, "final_state", torch.float32, dev),
        _ptr(chunk_states, "chunk_states", torch.float32, dev),
        batch, L, Dc, N, _dt(u), ws_ptr, ws_bytes, _stream(stream))
    _lib.check(st)
    return y, final_state, chunk_states


SCAN_KERNELS = {_lib.SSM_SCAN_SEQUENTIAL: "scan_sequential_kernel", _lib.SSM_SCAN_CHUNKED: "scan_chunked_kernel",
                _lib.SSM_SCAN_TOKSEQ: "scan_tokseq_kernel"}


def selective_scan_fwd_kernel(batch, L, D, N, dtype=torch.float32, gate=True, discretization="simplified",
                              conv_width=0, variant=0, tokens_per_lane=0) -> str:
    """Name of the kernel selective_scan_fwd (or, with conv_width > 0,
    selective_scan_fwd_conv) runs for this shape (16-byte-aligned tensors, L > 0).
    Raises SsmError when such a call would be rejected."""
    lib = _lib.load_library()
    dt = _lib.SSM_BF16 if dtype == torch.bfloat16 else _lib.SSM_F32
    k = lib.ssm_selective_scan_fwd_kernel(int(batch), int(L), int(D), int(N), dt, 1 if gate else 0,
                                          1 if discretization == "zoh" else 0, int(conv_width), int(variant),
                                          int(tokens_per_lane))
    if k < 0:
        _lib.check(-k)
    return SCAN_KERNELS[k]


def selective_scan_bwd_workspace_size(batch, L, D, N, dtype=torch.float32, saved=False) -> int:
    """Bytes of device workspace selective_scan_bwd needs for this shape (saved: with
    chunk_states from selective_scan_fwd_save)."""
    lib = _lib.load_library()
    dt = _lib.SSM_BF16 if dtype == torch.bfloat16 else _lib.SSM_F32
    fn = lib.ssm_selective_scan_bwd_saved_workspace_size if saved else lib.ssm_selective_scan_bwd_workspace_size
    return int(fn(int(batch), int(L), int(D), int(N), dt))


def selective_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, delta_softplus=True, *,
                       initial_state=None, dfinal_state=None, chunk_states=None, want_dD=None,
                       want_ddelta_bias=None, want_dinitial_state=None, workspace=None, out=None,
                       stream=None) -> dict:
    """Backward pass of selective_scan_fwd (same inputs) for the output gradient dy
    [batch, D, L] and optionally the final-state gradient dfinal_state [batch, D, N].

    Returns a dict with du, ddelta (w.r.t. the raw delta), dA, dB, dC ([batch, L, N],
    the layout of B and C) and, where computed, dD, dz, ddelta_bias and
    dinitial_state (None otherwise).  dD, ddelta_bias and dinitial_state are computed
    when the matching input is given, unless the want_* flag says otherwise; dz
    whenever z is given.  `workspace` is a device tensor of at least
    selective_scan_bwd_workspace_size(...) bytes, or None to allocate one.  `out`
    may hold preallocated output tensors under the same keys (missing keys are
    allocated).  `chunk_states`: what selective_scan_fwd_save returned for these
    inputs; the pass then starts each chunk from the saved state
    (ssm_selective_scan_bwd_saved) and the workspace is
    selective_scan_bwd_workspace_size(..., saved=True) bytes.
    """
    lib = _lib.load_library()
    batch, Dc, L, N = _scan_shapes(u, delta, A, B, C, D, z, delta_bias, initial_state, None, None)
    _shape(dy, "dy", (batch, Dc, L))
    _shape(dfinal_state, "dfinal_state", (batch, Dc, N))
    act = u.dtype
    dev = u.device
    want_dD = D is not None if want_dD is None else want_dD
    want_db = delta_bias is not None if want_ddelta_bias is None else want_ddelta_bias
    want_dh0 = initial_state is not None if want_dinitial_state is None else want_dinitial_state
    f32 = torch.float32
    spec = {  # name: (shape, dtype, computed)
        "du": ((batch, Dc, L), act, True),
        "ddelta": ((batch, Dc, L), act, True),
        "dA": ((Dc, N), f32, True),
        "dB": ((batch, L, N), act, True),
        "dC": ((batch, L, N), act, True),
        "dD": ((Dc,), f32, want_dD),
        "dz": ((batch, Dc, L), act, z is not None),
        "ddelta_bias": ((Dc,), f32, want_db),
        "dinitial_state": ((batch, Dc, N), f32, want_dh0),
    }
    given = out or {}
    out = {}
    for k, (shape, dt_, computed) in spec.items():
        t = given.get(k)
        if t is not None and computed:
            _shape(t, f"out[{k!r}]", shape)
            if t.dtype != dt_:
                raise TypeError(f"out[{k!r}] must be {dt_}")
            out[k] = t
        else:
            out[k] = torch.empty(shape, dtype=dt_, device=dev) if computed else None
    saved = chunk_states is not None
    if saved:
        _shape(chunk_states, "chunk_states", (batch, Dc, (L + SAVE_CHUNK - 1) // SAVE_CHUNK, N))
    need = selective_scan_bwd_workspace_size(batch, L, Dc, N, act, saved)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = _workspace(workspace, need, dev)
    ins = (_ptr(u, "u", act, dev), _ptr(delta, "delta", act, dev), _ptr(A, "A", f32, dev),
           _ptr(B, "B", act, dev), _ptr(C, "C", act, dev), _ptr(D, "D", f32, dev),
           _ptr(z, "z", act, dev), _ptr(delta_bias, "delta_bias", f32, dev), 1 if delta_softplus else 0,
           _ptr(initial_state, "initial_state", f32, dev), _ptr(dy, "dy", act, dev),
           _ptr(dfinal_state, "dfinal_state", f32, dev))
    if saved:
        fn, ins = lib.ssm_selective_scan_bwd_saved, ins + (_ptr(chunk_states, "chunk_states", f32, dev),)
    else:
        fn = lib.ssm_selective_scan_bwd
    st = fn(
        *ins,
        _ptr(out["du"], "du"), _ptr(out["ddelta"], "ddelta"), _ptr(out["dA"], "dA"), _ptr(out["dB"], "dB"),
        _ptr(out["dC"], "dC"), _ptr(out["dD"], "dD"), _ptr(out["dz"], "dz"),
        _ptr(out["ddelta_bias"], "ddelta_bias"), _ptr(out["dinitial_state"], "dinitial_state"),
        batch, L, Dc, N, _dt(u), ws_ptr, ws_bytes, _stream(stream))
    _lib.check(st)
    return out


def ssd_scan_workspace_size(batch, L, H, P, N) -> int:
    """Bytes of workspace that let ssd_scan_fwd run sequences as parallel segments."""
    lib = _lib.load_library()
    return int(lib.ssm_ssd_scan_workspace_size(int(batch), int(L), int(H), int(P), int(N), _lib.SSM_BF16))


def ssd_scan_fwd(x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True, *, initial_state=None, y=None,
                 final_state=None, return_final_state=True, workspace="auto", stream=None):
    """Mamba-2 SSD scan.  x [batch, L, H, P] bf16; dt [batch, L, H] bf16; A [H] float32;
    B, C [batch, L, N] bf16; D, dt_bias [H] float32.  Returns (y [batch, L, H, P],
    final_state [batch, H, P, N] float32 or None).  `workspace`: a device tensor of at
    least ssd_scan_workspace_size(...) bytes, None (one segment per sequence), or
    "auto" (allocated here)."""
    lib = _lib.load_library()
    if not isinstance(x, torch.Tensor) or not isinstance(B, torch.Tensor) or x.dim() != 4 or B.dim() != 3:
        raise ValueError("expected x [batch, L, H, P] and B/C [batch, L, N]")
    batch, L, H, P = x.shape
    N = B.shape[2]
    _shape(dt, "dt", (batch, L, H))
    _shape(A, "A", (H,))
    _shape(B, "B", (batch, L, N))
    _shape(C, "C", (batch, L, N))
    _shape(D, "D", (H,))
    _shape(dt_bias, "dt_bias", (H,))
    _shape(initial_state, "initial_state", (batch, H, P, N))
    _shape(y, "y", (batch, L, H, P))
    _shape(final_state, "final_state", (batch, H, P, N))
    act, dev = x.dtype, x.device
    if y is None:
        y = torch.empty((batch, L, H, P), dtype=act, device=dev)
    if final_state is None and return_final_state:
        final_state = torch.empty((batch, H, P, N), dtype=torch.float32, device=dev)
    f32 = torch.float32
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"unknown workspace option {workspace!r}")
        ws_ptr, ws_bytes = _workspace(None, ssd_scan_workspace_size(batch, L, H, P, N), dev)
    elif workspace is None:
        ws_ptr, ws_bytes = None, 0
    else:
        ws_ptr, ws_bytes = _workspace(workspace, 0, dev)
    st = lib.ssm_ssd_scan_fwd(
        _ptr(x, "x", act, dev), _ptr(dt, "dt", act, dev), _ptr(A, "A", f32, dev), _ptr(B, "B", act, dev),
        _ptr(C, "C", act, dev), _ptr(D, "D", f32, dev), _ptr(dt_bias, "dt_bias", f32, dev),
        1 if dt_softplus else 0, _ptr(initial_state, "initial_state", f32, dev), _ptr(y, "y", act, dev),
        _ptr(final_state, "final_state", f32, dev), batch, L, H, P, N, _dt(x), ws_ptr, ws_bytes,
        _stream(stream))
    _lib.check(st)
    return y, final_state


def causal_conv1d(x, weight, bias=None, silu=True, *, out=None, stream=None) -> torch.Tensor:
    """Causal depthwise conv1d along L (+ SiLU).  x [batch, D, L]; weight [D, K] float32
    (K <= 4, weight[:, K-1] weighs the current token); bias [D] or None."""
    lib = _lib.load_library()
    if not isinstance(x, torch.Tensor) or not isinstance(weight, torch.Tensor) or x.dim() != 3 \
            or weight.dim() != 2 or weight.shape[0] != x.shape[1]:
        raise ValueError("expected x [batch, D, L] and weight [D, K]")
    batch, Dc, L = x.shape
    _shape(bias, "bias", (Dc,))
    _shape(out, "out", (batch, Dc, L))
    dev = x.device
    if out is None:
        out = torch.empty_like(x)
    st = lib.ssm_causal_conv1d_fwd(
        _ptr(x, "x", x.dtype, dev), _ptr(weight, "weight", torch.float32, dev),
        _ptr(bias, "bias", torch.float32, dev), int(weight.shape[1]), 1 if silu else 0,
        _ptr(out, "out", x.dtype, dev), batch, Dc, L, _dt(x), _stream(stream))
    _lib.check(st)
    return out


def selective_scan_fwd_conv(x, conv_weight, conv_bias, delta, A, B, C, D=None, z=None, delta_bias=None,
                            delta_softplus=True, *, initial_state=None, u_out=None, return_u=False, y=None,
                            final_state=None, return_final_state=True, tokens_per_lane=0,
                            stream=None):
    """Scan of u = SiLU(causal_conv1d(x)) with the convolution fused into the scan kernel.

    Returns (y, final_state, u) where u is the convolution output when `return_u`
    (or `u_out` is given), else None."""
    lib = _lib.load_library()
    batch, Dc, L, N = _scan_shapes(x, delta, A, B, C, D, z, delta_bias, initial_state, y, final_state)
    if not isinstance(conv_weight, torch.Tensor) or conv_weight.dim() != 2 or conv_weight.shape[0] != Dc:
        raise ValueError("conv_weight must be [D, K]")
    _shape(conv_bias, "conv_bias", (Dc,))
    _shape(u_out, "u_out", (batch, Dc, L))
    act = x.dtype
    dev = x.device
    if y is None:
        y = torch.empty((batch, Dc, L), dtype=act, device=dev)
    if final_state is None and return_final_state:
        final_state = torch.empty((batch, Dc, N), dtype=torch.float32, device=dev)
    if u_out is None and return_u:
        u_out = torch.empty((batch, Dc, L), dtype=act, device=dev)
    st = lib.ssm_selective_scan_fwd_conv(
        _ptr(x, "x", act, dev), _ptr(conv_weight, "conv_weight", torch.float32, dev),
        _ptr(conv_bias, "conv_bias", torch.float32, dev), int(conv_weight.shape[1]),
        _ptr(delta, "delta", act, dev), _ptr(A, "A", torch.float32, dev),
        _ptr(B, "B", act, dev), _ptr(C, "C", act, dev), _ptr(D, "D", torch.float32, dev),
        _ptr(z, "z", act, dev), _ptr(delta_bias, "delta_bias", torch.float32, dev),
        1 if delta_softplus else 0, _ptr(initial_state, "initial_state", torch.float32, dev),
        _ptr(u_out, "u_out", act, dev), _ptr(y, "y", act, dev),
        _ptr(final_state, "final_state", torch.float32, dev),
        batch, L, Dc, N, _dt(x), _stream(stream), int(tokens_per_lane))
    _lib.check(st)
    return y, final_state, u_out


def state_update(state, u_t, delta_t, A, B_t, C_t, D=None, z_t=None, delta_bias=None,
                 delta_softplus=True, *, out_state=None, y=None, discretization="simplified",
                 stream=None) -> torch.Tensor:
    """One decode step.  state [S, D, N] float32; u_t, delta_t, z_t [S, D]; A [D, N];
    B_t, C_t [S, N]; D, delta_bias [D].  Updates `out_state` (default: `state`, in
    place); returns y_t [S, D].  `discretization` as in selective_scan_fwd."""
    if discretization not in ("simplified", "zoh"):
        raise ValueError(f"unknown discretization {discretization!r}")
    lib = _lib.load_library()
    if not isinstance(state, torch.Tensor) or state.dim() != 3:
        raise ValueError("expected state [S, D, N]")
    S, Dc, N = state.shape
    _shape(u_t, "u_t", (S, Dc))
    _shape(delta_t, "delta_t", (S, Dc))
    _shape(z_t, "z_t", (S, Dc))
    _shape(A, "A", (Dc, N))
    _shape(B_t, "B_t", (S, N))
    _shape(C_t, "C_t", (S, N))
    _shape(D, "D", (Dc,))
    _shape(delta_bias, "delta_bias", (Dc,))
    _shape(out_state, "out_state", (S, Dc, N))
    _shape(y, "y", (S, Dc))
    act = u_t.dtype
    dev = state.device
    if out_state is None:
        out_state = state
    if y is None:
        y = torch.empty((S, Dc), dtype=act, device=dev)
    fn = lib.ssm_state_update_zoh if discretization == "zoh" else lib.ssm_state_update
    st = fn(
        _ptr(state, "state", torch.float32, dev), _ptr(out_state, "out_state", torch.float32, dev),
        _ptr(u_t, "u_t", act, dev), _ptr(delta_t, "delta_t", act, dev), _ptr(A, "A", torch.float32, dev),
        _ptr(B_t, "B_t", act, dev), _ptr(C_t, "C_t", act, dev), _ptr(D, "D", torch.float32, dev),
        _ptr(z_t, "z_t", act, dev), _ptr(delta_bias, "delta_bias", torch.float32, dev),
        1 if delta_softplus else 0, _ptr(y, "y", act, dev), S, Dc, N, _dt(u_t), _stream(stream))
    _lib.check(st)
    return y
