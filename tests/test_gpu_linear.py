"""GPU parity of the plain linear entry point (y = x W^T + b) against the oracle.

Shapes are chosen to land on each GEMM kernel the library picks and to leave
ragged edges on every axis it tiles: M <= 64 (32 x 256 register-staged tiles),
mid-size M or N (128 x 128 register-staged tiles) and M, N >= 1024 (256 x 256
tiles fed by direct global->LDS loads, 128-byte K slabs), with M and N not
multiples of the tile and K from one slab to 48.

Bounds (max |gpu - oracle| / RMS(oracle)): fp32 output 1e-5 -- the only
difference is fp32 accumulation over K <= 3072 bf16 products, relative error
~ sqrt(K) * 2^-24 ~ 3e-6 at the maximum over 10^6 outputs; bf16 output: the
same after subtracting each element's half-ulp storage rounding.
"""
import sys

import numpy as np
import pytest
import torch

import dit_inputs as DI
import oracle as O
from _helpers import parity_err, parity_err_bf16_stored

pytestmark = pytest.mark.gpu

TOL_F32_OUT = 1e-5
TOL_BF16_OUT = 1e-5


@pytest.fixture(scope="module")
def dit():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from image_generation_amd import dit as D
    return D


LINEAR_CASES = [
    # M, K, N
    (7, 64, 264),          # small M
    (64, 128, 1028),       # small M, ragged N
    (300, 128, 520),       # mid-size, ragged M and N
    (1024, 64, 1024),      # large tiles, a single K slab
    (1100, 192, 1028),     # large tiles, ragged M (76 rows) and N (4 columns)
    (1024, 3072, 1280),    # large tiles, 48 K slabs
    (2049, 256, 1536),     # large tiles, one row past a tile boundary
]


@pytest.mark.parametrize("M,K,N", LINEAR_CASES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_linear_forward(dit, M, K, N, out_dtype):
    print(f"linear M={M} K={K} N={N} out={out_dtype}", flush=True)
    sys.stdout.flush()
    x = DI.randn((M, K), 91, 1.0, "bf16")
    w = DI.randn((N, K), 92, K ** -0.5, "bf16")
    b = DI.randn((N,), 93, 0.1, "f32")
    y = torch.empty((M, N), dtype=out_dtype, device="cuda")
    dit.dit_linear_forward(x.cuda(), w.cuda(), b.cuda(), y)
    torch.cuda.synchronize()
    ref = O.linear(O.to64(x), O.to64(w), O.to64(b))
    got = y.double().cpu().numpy()
    if out_dtype == torch.float32:
        err = parity_err(got, ref)
        tol = TOL_F32_OUT
    else:
        err = parity_err_bf16_stored(got, ref)
        tol = TOL_BF16_OUT
    print(f"  err {err:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err <= tol


@pytest.mark.parametrize("K,N", [(3072, 21504), (15360, 3072)])
def test_linear_forward_shard_shapes_sampled(dit, K, N):
    """One rank's linear1 and linear2 under 8-way sequence parallelism at the 2048px
    CFG pair (2 x 16896 / 8 = 4224 token rows), bf16 out, on sampled rows (tile
    edges and random rows).  The bound grows with the accumulation length like the
    fp32 rounding of the K-term sum, sqrt(K / 3072) x 1e-5."""
    M = 4224
    print(f"linear shard M={M} K={K} N={N}", flush=True)
    sys.stdout.flush()
    x = DI.randn((M, K), 94, 1.0, "bf16")
    w = DI.randn((N, K), 95, K ** -0.5, "bf16")
    b = DI.randn((N,), 96, 0.1, "f32")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dit.dit_linear_forward(x.cuda(), w.cuda(), b.cuda(), y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([rng.choice(M, 16, replace=False),
                                     [0, 1, 255, 256, 2047, 2048, 4095, 4096, M - 2, M - 1]]))
    ref = O.linear(O.to64(x)[rows], O.to64(w), O.to64(b))
    got = y[torch.from_numpy(rows).cuda()].double().cpu().numpy()
    err = parity_err_bf16_stored(got, ref)
    tol = TOL_BF16_OUT * (K / 3072) ** 0.5
    print(f"  err {err:.3e} (bound {tol:.1e})", flush=True)
    assert np.isfinite(got).all()
    assert err <= tol


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_linear_forward_epilogue_paths_agree(dit, out_dtype):
    """The tiled kernel's epilogue stores a pass wholly inside the problem through its
    batched path and a pass that crosses the last row one row at a time; both do the
    same arithmetic, so a row must come out bit-identical either way.  Rows 1024..1063
    of a 1064-row problem (per-row path: their pass runs to row 1087) are computed
    again as rows 0..39 of a 1024-row problem (batched path)."""
    print(f"linear epilogue paths out={out_dtype}", flush=True)
    sys.stdout.flush()
    K, N = 192, 1024
    x = DI.randn((1064, K), 94, 1.0, "bf16").cuda()
    w = DI.randn((N, K), 95, K ** -0.5, "bf16").cuda()
    b = DI.randn((N,), 96, 0.1, "f32").cuda()
    y_rag = torch.empty((1064, N), dtype=out_dtype, device="cuda")
    dit.dit_linear_forward(x, w, b, y_rag)
    x2 = torch.cat([x[1024:], x[:984]]).contiguous()
    y_full = torch.empty((1024, N), dtype=out_dtype, device="cuda")
    dit.dit_linear_forward(x2, w, b, y_full)
    torch.cuda.synchronize()
    assert torch.equal(y_rag[1024:], y_full[:40])
    assert torch.equal(y_rag[:984], y_full[40:])
