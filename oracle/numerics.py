"""Test infrastructure: number-format rounding used by the oracle (fp64 numpy).

Formats (from their public definitions, not from any page):
  * bfloat16: 1 sign, 8 exponent, 7 stored mantissa bits (fp32 exponent range).
  * IEEE binary16 (fp16): 1 sign, 5 exponent bits with bias 15, 10 stored
    mantissa bits; largest finite 65504, smallest normal 2^-14.
  * OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits, no infinities, the all-ones code S.1111.111 is NaN; largest finite
    magnitude 1.75 * 2^8 = 448, smallest normal 2^-6, smallest subnormal 2^-9.

  * OCP FP4 E2M1: 1 sign, 2 exponent bits with bias 1, 1 mantissa bit;
    magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (no infinities or NaN).
  * OCP MX block scaling (MXFP4): 32 consecutive elements share one E8M0 scale
    2^e (an 8-bit biased exponent, bias 127); the shared exponent is
    floor(log2(amax)) - 2, 2 being E2M1's largest exponent, and each element is
    x / 2^e rounded to E2M1, values beyond 6 saturating.

The fp8 W8A8 recipe the pages name ("FP8 W8A8 dynamic precision" in the
runinfra.ai image-generation runbook, Optimization stack table) fixes no
rounding rule; the reading used here is round-to-nearest-even with saturation
to +-448 and a scale of amax/448 (amax = 0 gives scale 1).  The 4-bit variant
(the pages compare NVFP4 checkpoints with BF16 in the VisualGen article on FLUX
Klein, and the diffusion-backend commit picks nvfp4 / fp8 / mxfp8 by GPU
generation) is taken as MXFP4, gfx950's block-scaled FP4, with
round-to-nearest-even.

Pins (tests/test_oracle_pins.py):
  round_bf16          test_bf16_rounding_vs_torch_cast
  round_fp16          test_fp16_rounding_vs_numpy_cast
  round_e4m3          test_e4m3_code_table_bruteforce (all 256 codes),
                      test_e4m3_golden_points (tests/golden/e4m3_points.txt),
                      test_e4m3_representable_values_are_fixed_points
  e4m3_tie_mask       test_e4m3_tie_mask_against_code_table
  quant_scale_f32,    test_quantize_rows_scale_and_roundtrip
  quantize_rows_e4m3
  round_e2m1          test_e2m1_rounding_cases, test_e2m1_value_set
  mx_block_exponent   test_mx_block_exponent_cases
  quantize_mxfp4,     test_mxfp4_reproduces_representable_blocks, test_mxfp4_error_bound
  dequantize_mxfp4
"""
from __future__ import annotations

import numpy as np

__all__ = ["round_bf16", "round_fp16", "e4m3_tie_mask", "round_e4m3", "E4M3_MAX", "quant_scale_f32",
           "quantize_rows_e4m3", "round_e2m1", "E2M1_MAX", "MX_BLOCK",
           "mx_block_exponent", "quantize_mxfp4", "dequantize_mxfp4"]

E2M1_MAX = 6.0
MX_BLOCK = 32

E4M3_MAX = 448.0


def _round_sig(x: np.ndarray, sig_bits: int, min_exp: int) -> np.ndarray:
    """Round to the nearest value with ``sig_bits`` significant bits, ties to even.

    Below 2**min_exp the spacing stays 2**(min_exp - sig_bits + 1) (gradual
    underflow).  Works in fp64, where every step below is exact.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    m, e = np.frexp(ax)                      # ax = m * 2**e, m in [0.5, 1)
    # exponent of the leading bit is e - 1; clamp to the subnormal range
    lead = np.maximum(e - 1, min_exp)
    ulp_exp = lead - (sig_bits - 1)
    q = np.rint(np.ldexp(ax, -ulp_exp))      # rint rounds half to even
    out = np.ldexp(q, ulp_exp)
    out = np.where(ax == 0, 0.0, out)
    return np.copysign(out, x)


def round_bf16(x) -> np.ndarray:
    """fp64 -> nearest bfloat16 value (as fp64), ties to even; overflow -> inf."""
    x = np.asarray(x, dtype=np.float64)
    out = _round_sig(x, 8, -126)
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    # halfway above max rounds to inf (ties-to-even lands on the next binade)
    out = np.where(np.abs(out) > bf16_max, np.copysign(np.inf, x), out)
    return np.where(np.isnan(x), np.nan, out)


def round_fp16(x) -> np.ndarray:
    """fp64 -> nearest binary16 value (as fp64), ties to even; overflow -> inf."""
    x = np.asarray(x, dtype=np.float64)
    out = _round_sig(x, 11, -14)
    fp16_max = (2.0 - 2.0 ** -10) * 2.0 ** 15
    out = np.where(np.abs(out) > fp16_max, np.copysign(np.inf, x), out)
    return np.where(np.isnan(x), np.nan, out)


def e4m3_tie_mask(y, rel):
    """(mask, step): mask marks the y (>= 0, <= 448) that lie within rel * y of
    an e4m3 rounding boundary (a midpoint between neighbouring codes), where a
    computation carried in a different precision may round the other way;
    step is the spacing of e4m3 values around y.  rel: a scalar or an array
    broadcast against y."""
    y = np.asarray(y, dtype=np.float64)
    _, e = np.frexp(y)
    step = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    mid = (np.floor(y / step) + 0.5) * step
    return np.abs(y - mid) <= rel * y, step


def round_e4m3(x) -> np.ndarray:
    """fp64 -> nearest OCP e4m3 value (as fp64), ties to even, saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    out = _round_sig(x, 4, -6)
    out = np.clip(out, -E4M3_MAX, E4M3_MAX)
    return np.where(np.isnan(x), np.nan, out)


def quant_scale_f32(amax) -> tuple:
    """Per-row scale and its reciprocal, both taken in fp32 as a kernel does.

    scale = amax / 448 and inv = 448 / amax, each one correctly rounded fp32
    division; amax == 0 gives scale = inv = 1.
    """
    a = np.asarray(amax, dtype=np.float32)
    safe = np.where(a > 0, a, np.float32(1.0))
    scale = np.where(a > 0, safe / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    inv = np.where(a > 0, np.float32(E4M3_MAX) / safe, np.float32(1.0)).astype(np.float32)
    return scale, inv


def quantize_rows_e4m3(x: np.ndarray):
    """Dynamic per-row (per-token) quantisation of a 2-D array.

    Returns (codes as fp64 values, scale [rows] fp32).  The value fed to the
    rounding is fp32(x) * inv in fp32, the precision a kernel takes the
    decision in.
    """
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    scale, inv = quant_scale_f32(amax)
    y = (x32 * inv[..., None]).astype(np.float32)
    return round_e4m3(y.astype(np.float64)), scale


def round_e2m1(x) -> np.ndarray:
    """fp64 -> nearest OCP E2M1 (FP4) value (as fp64), ties to even, saturating at +-6.

    Two significant bits, smallest normal exponent 0 (spacing 0.5 below 2): the
    magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
    """
    x = np.asarray(x, dtype=np.float64)
    out = _round_sig(x, 2, 0)
    return np.clip(out, -E2M1_MAX, E2M1_MAX)


def mx_block_exponent(amax) -> np.ndarray:
    """Shared MX exponent of a block: floor(log2(amax)) - 2, clamped to the E8M0
    range [-127, 127]; an all-zero block takes exponent 0."""
    a = np.asarray(amax, dtype=np.float64)
    _, k = np.frexp(np.where(a > 0, a, 1.0))       # a = m * 2^k, m in [0.5, 1)
    e = np.where(a > 0, k - 1 - 2, 0)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_mxfp4(x: np.ndarray):
    """MXFP4 quantisation along the last axis (a multiple of 32 long).

    Returns (q, e): q the E2M1 values (fp64, same shape as x) and e the shared
    exponent of each 32-element block ([..., K/32] int64); x ~ q * 2^e.  The
    value rounded is fp32(x) / 2^e, exact in fp32 as in a kernel.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    K = x.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("MXFP4: last axis must be a multiple of 32")
    xb = x.reshape(x.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    e = mx_block_exponent(np.max(np.abs(xb), axis=-1))
    q = round_e2m1(np.ldexp(xb, -e[..., None]))
    return q.reshape(x.shape), e


def dequantize_mxfp4(q: np.ndarray, e: np.ndarray) -> np.ndarray:
    """q * 2^e with each block's exponent broadcast over its 32 elements."""
    K = q.shape[-1]
    qb = np.asarray(q, dtype=np.float64).reshape(q.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    return np.ldexp(qb, np.asarray(e)[..., None]).reshape(q.shape)

