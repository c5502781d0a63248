"""MI355X (gfx950) selective scan and recurrent decode step.

The kernels and the C ABI live in libssm.so (include/ssm.h); this package is a
thin binding over it.  Importing the package does not load the library; the
first call does, and raises if the library has not been built.
"""
from ._lib import SsmError, load_library, LIB_PATH  # noqa: F401
from ._lib import (SSM_SCAN_AUTO, SSM_SCAN_SEQUENTIAL, SSM_SCAN_CHUNKED, SSM_SCAN_TOKSEQ, SSM_SCAN_AP)  # noqa: F401
from .ops import (selective_scan_fwd, selective_scan_fwd_save, SAVE_CHUNK,  # noqa: F401
                  selective_scan_fwd_conv, selective_scan_fwd_kernel, selective_scan_bwd,
                  selective_scan_workspace_size, selective_scan_bwd_workspace_size, causal_conv1d, state_update,
                  ssd_scan_fwd, ssd_scan_workspace_size)

__all__ = ["selective_scan_fwd", "selective_scan_fwd_save", "SAVE_CHUNK", "selective_scan_fwd_conv", "selective_scan_fwd_kernel", "selective_scan_bwd",
           "selective_scan_workspace_size", "selective_scan_bwd_workspace_size", "causal_conv1d", "state_update",
           "ssd_scan_fwd", "ssd_scan_workspace_size", "SsmError", "load_library", "LIB_PATH",
           "SSM_SCAN_AUTO", "SSM_SCAN_SEQUENTIAL", "SSM_SCAN_CHUNKED", "SSM_SCAN_TOKSEQ", "SSM_SCAN_AP"]
