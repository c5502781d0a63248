"""Error metric used by every parity test.

The tolerance is a maximum relative error.  It is measured row by row: a row is
the series a tolerance naturally scales with (the time series y[b, d, :] of one
channel, one channel's state vector, or one decode channel's outputs over the
steps).  For each row, err = max|x - ref| / max|ref|; a row whose reference is
identically zero uses the absolute error.  The reported value is the max over rows.
A pure elementwise relative error is undefined where y cancels to ~0, which the
gated, skip-added readout does at many points.
"""
import numpy as np


def row_rel_err(x, ref, axis=-1):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if x.size == 0:
        return 0.0
    num = np.max(np.abs(x - ref), axis=axis)
    den = np.max(np.abs(ref), axis=axis)
    err = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    if not np.all(np.isfinite(x)):
        return float("inf")
    return float(np.max(err))
