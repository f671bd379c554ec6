"""GPU parity of the MXFP4 (W4A4) path against the oracle.

Quantisation: every E2M1 code and every E8M0 block scale the kernel writes must
equal the oracle's (the decision is an exact power-of-two scaling followed by
comparisons, so there is nothing to round differently), padding rows of the scale
array read 2^0.

GEMM: the oracle quantises the same bf16 inputs, so both sides multiply the same
E2M1 values with the same scales; each product is exact in fp32 and only the fp32
accumulation order differs.  Bound: max |gpu - oracle| / RMS(oracle) <= 1e-5
(the accumulation error over K <= 3072 terms stays near 1e-6 of the RMS); a bf16
output first has its half-ulp storage rounding taken off.
"""
import sys

import numpy as np
import pytest
import torch

import dit_inputs as DI
import oracle as O
from _helpers import parity_err, parity_err_bf16_stored

pytestmark = pytest.mark.gpu

TOL_MX = 1e-5
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


@pytest.fixture(scope="module")
def dit():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from image_generation_amd import dit as D
    return D


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _decode(codes, scales, rows, width):
    """(E2M1 values [rows, width], block exponents [rows, width / 32], pad-row bytes)."""
    c = codes.cpu().numpy().astype(np.int64)
    nib = np.stack([c & 15, c >> 4], axis=-1).reshape(rows, width)
    val = E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    sc = scales.cpu().numpy().astype(np.int64)             # [width/256, pad, 8]
    order = [0, 2, 4, 6, 1, 3, 5, 7]                         # storage order of a row's 8 blocks
    blocks = np.empty((sc.shape[1], width // 32), dtype=np.int64)
    for slab in range(width // 256):
        for pos, blk in enumerate(order):
            blocks[:, slab * 8 + blk] = sc[slab, :, pos]
    return val, blocks[:rows] - 127, blocks[rows:]


def _special_rows(width, seed):
    """Rows with an all-zero block, a saturating block, tiny and huge magnitudes."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((4, width))
    x[0, :32] = 0.0
    x[1, :32] = np.linspace(-7.5, 7.5, 32)            # amax 7.5: e = 0, 7.5 and 6.5 saturate
    x[2] *= 1e-30
    x[3] *= 1e20
    return x


@pytest.mark.parametrize("rows,width", [(1, 256), (37, 768), (300, 3072), (257, 512)])
@pytest.mark.parametrize("src_dt", ["bf16", "f32"])
def test_quantize_mxfp4_exact(dit, rows, width, src_dt):
    _say(f"mxfp4 quantise rows={rows} width={width} src={src_dt}")
    x = DI.randn((rows, width), 71, 2.0, "f32")
    if rows >= 4:
        x[:4] = torch.from_numpy(_special_rows(width, 72)).float()
    x = x.to(torch.bfloat16) if src_dt == "bf16" else x
    codes, scales = dit.dit_quantize_mxfp4(x.cuda())
    torch.cuda.synchronize()
    val, e, pad = _decode(codes, scales, rows, width)
    q, e_ref = O.quantize_mxfp4(O.to64(x))
    np.testing.assert_array_equal(e, e_ref)
    np.testing.assert_array_equal(val, q)
    assert pad.size == 0 or np.all(pad == 127)           # padding rows: 2^0


@pytest.mark.parametrize("M,K,N", [(256, 256, 256), (1100, 768, 1028), (2049, 512, 1536),
                                   (1024, 3072, 1280)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_linear_mxfp4(dit, M, K, N, out_dtype):
    _say(f"mxfp4 linear M={M} K={K} N={N} out={out_dtype}")
    x = DI.randn((M, K), 73, 1.0, "bf16")
    w = DI.randn((N, K), 74, K ** -0.5, "bf16")
    b = DI.randn((N,), 75, 0.1, "f32")
    xq = dit.dit_quantize_mxfp4(x.cuda())
    wq = dit.dit_quantize_mxfp4(w.cuda())
    y = torch.empty((M, N), dtype=out_dtype, device="cuda")
    dit.dit_linear_mxfp4(xq, wq, b.cuda(), y)
    torch.cuda.synchronize()
    ref = O.linear_mxfp4(O.to64(x), O.to64(w), O.to64(b))
    got = y.double().cpu().numpy()
    err = parity_err(got, ref) if out_dtype == torch.float32 else parity_err_bf16_stored(got, ref)
    _say(f"  err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL_MX
