"""The five synthetic workloads: shapes, activation dtype and input recipe.

Shapes come from Mamba-style layer widths: the decode workload's D = 5120 and
N = 16 follow the Mamba-2.8B card (d_model 2560, expand 2, d_state 16) on the
interview-prep page's "Model Card" table; the long-context scan uses that
card's d_model as its channel count.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class ScanConfig:
    name: str
    batch: int
    L: int
    D: int
    N: int
    dtype: str          # activation dtype: "f32" or "bf16"
    gate: bool          # SiLU(z) output gate present
    d_skip: str         # "normal": D ~ N(0,1); "ones": D = 1
    seed: int = 0
    conv_k: int = 0     # > 0: the input is x and u = SiLU(causal conv1d of width conv_k) is fused in
    backward: bool = False  # the workload is the backward pass (gradients for dy) instead of the forward
    discretization: str = "simplified"   # or "zoh": the full zero-order-hold input term
    saved: bool = False  # backward: the forward pass's saved 512-token chunk states are read
    train: bool = False  # with saved: the step is the forward pass that saves them, then the backward

    @property
    def elements(self) -> int:
        return self.batch * self.L * self.D * self.N

    def algorithmic_bytes(self) -> int:
        """Each input read once and each output written once."""
        e = 4 if self.dtype == "f32" else 2
        per_tok = self.batch * self.L * self.D * e
        if self.backward:
            # reads u, delta, dy (+ z), B, C, A, D, bias; writes du, ddelta (+ dz), dB, dC, dA, dD, dbias
            n_act = 5 + (2 if self.gate else 0)
            saved = 4 * self.batch * self.D * (-(-self.L // 512)) * self.N if self.saved else 0
            if self.train:
                # plus the forward pass: u, delta (+ z) read again, y and the final
                # state written, the saved states written once more
                n_act += 3 + (1 if self.gate else 0)
                saved *= 2
                per_tok_extra = 2 * self.batch * self.L * self.N * e + 4 * self.batch * self.D * self.N
            else:
                per_tok_extra = 0
            return (per_tok * n_act + saved + per_tok_extra
                    + 4 * self.batch * self.L * self.N * e    # B, C read; dB, dC written
                    + 8 * self.D * self.N                     # A read, dA written
                    + 16 * self.D)                            # D skip, bias read; their gradients written
        n_act = 3 + (1 if self.gate else 0)          # u, delta, y (+ z)
        return (per_tok * n_act
                + 2 * self.batch * self.L * self.N * e  # B, C
                + 4 * self.D * self.N                   # A
                + 4 * self.D * 2                        # D skip + delta bias
                + 4 * self.batch * self.D * self.N     # final state
                + 4 * self.D * (self.conv_k + 1 if self.conv_k else 0))   # conv taps + bias


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int          # sequences S
    D: int
    N: int
    steps: int
    dtype: str = "bf16"
    gate: bool = True
    seed: int = 0

    @property
    def elements_per_step(self) -> int:
        return self.batch * self.D * self.N

    def algorithmic_bytes_per_step(self) -> int:
        e = 4 if self.dtype == "f32" else 2
        sd = self.batch * self.D
        return (8 * sd * self.N                        # state read + write
                + sd * e * (4 if self.gate else 3)     # u, delta, (z), y
                + 2 * self.batch * self.N * e          # B_t, C_t
                + 4 * self.D * self.N + 8 * self.D)    # A, D skip, bias


@dataclass(frozen=True)
class SSDConfig:
    """A Mamba-2 SSD scan workload (scalar decay per head, P x N state per head)."""
    name: str
    batch: int
    L: int
    H: int
    P: int
    N: int
    dtype: str = "bf16"
    seed: int = 0

    @property
    def elements(self) -> int:
        """Recurrence elements B*L*H*P*N (one state-entry update each)."""
        return self.batch * self.L * self.H * self.P * self.N

    def algorithmic_bytes(self) -> int:
        """x read and y written, dt, B, C read, A, D, bias read, the final state written."""
        e = 2
        return (2 * self.batch * self.L * self.H * self.P * e + self.batch * self.L * self.H * e
                + 2 * self.batch * self.L * self.N * e + 12 * self.H
                + 4 * self.batch * self.H * self.P * self.N)

    def flops(self, chunk: int = 64) -> int:
        """Matrix-core work of the chunked form per call: per (batch, head, chunk) the
        products C B^T (Q x Q x N), its masked product with x (Q x P x Q), the chunk's
        state contribution (N x P x Q) and the carried-state output (Q x P x N), 2 flops
        per multiply-add."""
        nch = -(-self.L // chunk)
        Q = chunk
        per = Q * Q * self.N + Q * self.P * Q + self.N * self.P * Q + Q * self.P * self.N
        return 2 * per * self.batch * self.H * nch


CONFIGS = {
    "tiny_f32": ScanConfig("tiny_f32", 1, 64, 16, 4, "f32", gate=False, d_skip="normal"),
    "mamba130m_f32": ScanConfig("mamba130m_f32", 2, 2048, 1536, 16, "f32", gate=True, d_skip="ones"),
    "mamba1p4b_bf16": ScanConfig("mamba1p4b_bf16", 8, 2048, 4096, 16, "bf16", gate=True, d_skip="ones"),
    "long131k_bf16": ScanConfig("long131k_bf16", 1, 131072, 2560, 16, "bf16", gate=True, d_skip="ones"),
    "decode_bf16": DecodeConfig("decode_bf16", 256, 5120, 16, 512),
    # the block's conv1d (d_conv = 4 on the interview-prep page's model card) fused into the scan
    "mamba130m_conv_f32": ScanConfig("mamba130m_conv_f32", 2, 2048, 1536, 16, "f32", gate=True, d_skip="ones",
                                     conv_k=4),
    "mamba1p4b_conv_bf16": ScanConfig("mamba1p4b_conv_bf16", 8, 2048, 4096, 16, "bf16", gate=True,
                                      d_skip="ones", conv_k=4),
    # the full zero-order-hold discretization at the forward workloads' shapes
    "zoh_mamba130m_f32": ScanConfig("zoh_mamba130m_f32", 2, 2048, 1536, 16, "f32", gate=True, d_skip="ones",
                                    discretization="zoh"),
    "zoh_mamba1p4b_bf16": ScanConfig("zoh_mamba1p4b_bf16", 8, 2048, 4096, 16, "bf16", gate=True, d_skip="ones",
                                     discretization="zoh"),
    # Mamba-2 SSD at a 2.7B-shaped layer: d_model 2560 (the prep page's model card),
    # expanded 2x to 5120 channels = 80 heads of 64, state 64 per head channel
    "ssd_2p7b_bf16": SSDConfig("ssd_2p7b_bf16", 4, 2048, 80, 64, 64),
    # the backward pass (training) at the forward workloads' shapes, for an output gradient dy
    "bwd_mamba130m_f32": ScanConfig("bwd_mamba130m_f32", 2, 2048, 1536, 16, "f32", gate=True, d_skip="ones",
                                    backward=True),
    "bwd_mamba1p4b_bf16": ScanConfig("bwd_mamba1p4b_bf16", 8, 2048, 4096, 16, "bf16", gate=True, d_skip="ones",
                                     backward=True),
    # ... with the forward pass's saved chunk states (the training pair)
    "bwd_saved_mamba1p4b_bf16": ScanConfig("bwd_saved_mamba1p4b_bf16", 8, 2048, 4096, 16, "bf16", gate=True,
                                           d_skip="ones", backward=True, saved=True),
    # the training pair: the forward pass saving chunk states, then the backward from them
    "train_mamba1p4b_bf16": ScanConfig("train_mamba1p4b_bf16", 8, 2048, 4096, 16, "bf16", gate=True, d_skip="ones",
                                       backward=True, saved=True, train=True),
    "bwd_long131k_bf16": ScanConfig("bwd_long131k_bf16", 1, 131072, 2560, 16, "bf16", gate=True, d_skip="ones",
                                    backward=True),
}
