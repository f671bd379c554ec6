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


def parity_err_bf16_stored(got, ref):
    """parity_err for a bf16-stored result: each element may differ from the
    exact value by half a bf16 ulp of its magnitude just by being stored, so
    that half-ulp is taken off each element's error before the max."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    _, e = np.frexp(np.abs(r))            # |r| in [2^(e-1), 2^e): ulp = 2^(e-8)
    half_ulp = np.ldexp(1.0, e - 9)
    excess = np.maximum(np.abs(g - r) - half_ulp, 0.0)
    return float(np.max(excess) / np.sqrt(np.mean(r * r)))


def sampled_block_rows(Lt, L, n, seed):
    """Sorted joint-token rows (text first): n random text and n random image rows
    plus both streams' ends, the first image rows and tile edges after them."""
    g = np.random.default_rng(seed)
    fixed = [0, Lt - 1, Lt, Lt + 1, L - 1, L - 2, Lt + 127, Lt + 128, Lt + 255, Lt + 256]
    picks = np.concatenate([g.choice(Lt, n, replace=False), Lt + g.choice(L - Lt, n, replace=False),
                            [r for r in fixed if 0 <= r < L]])
    return np.unique(picks).astype(np.int64)
