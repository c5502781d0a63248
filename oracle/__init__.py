"""CPU float64 oracle for the selective scan and the decode step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
package: only the tests, the smoke check and the benchmark's CPU-baseline leg use
it.  It shares no code with the HIP library and does not import it.
"""
from .ssm import (selective_scan, selective_scan_bwd, selective_scan_magnitude, state_update, softplus,  # noqa: F401
                  silu, causal_conv1d)
from .ssd import ssd_scan, ssd_step  # noqa: F401
