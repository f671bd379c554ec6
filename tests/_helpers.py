"""Shared test plumbing: seeded parameters as fp64 arrays, parity metric."""
import numpy as np

import dit_inputs as DI


def params64(dims, dtype, prefix=None):
    """Every model parameter (seeded 1000 + k) as an fp64 numpy array."""
    return {n: t.double().numpy() for n, t in DI.iter_params(dims, dtype, prefix)}


def parity_err(got, ref):
    """max|got - ref| / sqrt(mean(ref^2)) in fp64 over the whole tensor."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r))
    return float(np.max(np.abs(g - r)) / rms)
