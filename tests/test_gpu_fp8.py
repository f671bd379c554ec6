"""GPU parity of the fp8 (W8A8, OCP e4m3) path against the fp64 oracle.

Quantisation is integer work once the fp32 product x * (448 / amax) is formed,
so codes and scales are compared bit for bit.  Attention, blocks and the step
use the fp8 bound: max|gpu - oracle| / RMS(oracle) <= 6e-2.
"""
import math
import sys

import numpy as np
import pytest
import torch

import dit_inputs as DI
import oracle as O
from oracle.numerics import quantize_rows_e4m3
from _helpers import parity_err, parity_err_bf16_stored, sampled_block_rows

pytestmark = pytest.mark.gpu

TOL_FP8 = 6e-2
# P codes: the kernel forms 448 P in fp32, so a code whose 448 P lies within the
# fp32 evaluation's error bound of an e4m3 rounding boundary may round either way;
# the oracle derives that bound score by score (p448_fp32_window) and returns the
# spread such codes can cause as a per-element slack


def _err_with_slack(got, ref, slack):
    """parity_err_bf16_stored with each element's error first reduced by the
    oracle's slack (the spread of equally valid roundings of near-tie codes)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    _, e = np.frexp(np.abs(r))
    excess = np.maximum(np.abs(g - r) - slack - np.ldexp(1.0, e - 9), 0.0)
    return float(np.max(excess) / np.sqrt(np.mean(r * r)))


@pytest.fixture(scope="module")
def dit():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from image_generation_amd import dit as D
    return D


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bf16(shape, seed, std=1.0):
    return DI.randn(shape, seed, std, "bf16")


def _decode(codes: torch.Tensor) -> np.ndarray:
    """e4m3 bytes -> fp64 values (torch's float8_e4m3fn decoder on the CPU)."""
    return codes.cpu().view(torch.float8_e4m3fn).double().numpy()


# ---------------------------------------------------------------- quantisation

@pytest.mark.parametrize("rows,width", [(1, 8), (37, 520), (300, 3072), (9, 4104), (64, 15360), (4, 589824)])
def test_quantize_rows_bit_exact(dit, rows, width):
    _say(f"quantize rows={rows} width={width}")
    x = _bf16((rows, width), 41, 3.0)
    if rows > 3:
        x[1] = 0.0                                    # zero row: scale 1, codes 0
        x[2, :] = x[2, :] * 1e-30                     # tiny row: scaled up into range
        x[3, 0] = 1e4                                 # one outlier sets the scale
    codes, scale = dit.dit_quantize_rows(x.cuda())
    torch.cuda.synchronize()
    ref_v, ref_s = quantize_rows_e4m3(O.to64(x))
    np.testing.assert_array_equal(scale.cpu().numpy(), ref_s)
    np.testing.assert_array_equal(_decode(codes), ref_v)


# ---------------------------------------------------------------- attention

def _fp8_operands(dit, q, k, v):
    """Per-(b, h) e4m3 codes and scales of q, k and v, quantised by the library
    (one row per head: the [L, d] slice; rows padded to a multiple of 8 values)."""
    B, H, L, d = q.shape
    out = []
    for t in (q, k, v):
        codes, sc = dit.dit_quantize_rows(t.reshape(B * H, L * d).cuda())
        out.append((codes.view(B, H, L, d), sc.view(B, H)))
    return out[0][0], out[1][0], out[2][0], out[0][1], out[1][1], out[2][1]


def _run_fp8_attention(dit, q, k, v):
    B, H, L, d = q.shape
    q8, k8, v8, sq, sk, sv = _fp8_operands(dit, q, k, v)
    o = torch.empty((B, L, H * d), dtype=torch.bfloat16, device="cuda")
    dit.dit_attention(q8, k8, v8, o, q_scale=sq, k_scale=sk, v_scale=sv)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy().reshape(B, L, H, d).transpose(0, 2, 1, 3)


@pytest.mark.parametrize("B,H,L,d", [(1, 1, 16, 128), (1, 2, 272, 128), (2, 1, 528, 64),
                                     (1, 3, 1040, 128), (1, 1, 1, 128), (2, 2, 37, 64),
                                     (1, 2, 333, 128), (1, 1, 4097, 64)])
def test_attention_fp8_small(dit, B, H, L, d):
    _say(f"attention fp8 B={B} H={H} L={L} d={d}")
    q, k, v = _bf16((B, H, L, d), 51), _bf16((B, H, L, d), 52), _bf16((B, H, L, d), 53)
    got = _run_fp8_attention(dit, q, k, v)
    ref, slack = O.attention_fp8(O.to64(q), O.to64(k), O.to64(v), tie_fp32=True)
    err = _err_with_slack(got, ref, slack)
    _say(f"  err {err:.3e} (without slack {parity_err_bf16_stored(got, ref):.3e})")
    assert err <= TOL_FP8


@pytest.mark.parametrize("L,d", [(208, 128), (99, 64)])
def test_attention_fp8_identical_keys(dit, L, d):
    B, H = 1, 2
    q = _bf16((B, H, L, d), 61)
    k = _bf16((B, H, 1, d), 62).expand(B, H, L, d).contiguous()
    v = _bf16((B, H, L, d), 63)
    got = _run_fp8_attention(dit, q, k, v)
    ref = O.attention_fp8(O.to64(q), O.to64(k), O.to64(v))    # = mean of dequantised V
    assert parity_err_bf16_stored(got, ref) <= TOL_FP8


@pytest.mark.parametrize("B,L,H", [(1, 4608, 24), (2, 16896, 24), (2, 16896, 3)])
def test_attention_fp8_full_size_sampled(dit, B, L, H):
    """Heads of 128 at 1024px (4608 tokens) and the 2048px CFG pair (16896): 24
    heads, and one rank's 3 heads under 8-way head sharding."""
    _say(f"attention fp8 full B={B} L={L} H={H}")
    d = 128
    q, k, v = _bf16((B, H, L, d), 71), _bf16((B, H, L, d), 72), _bf16((B, H, L, d), 73)
    got = _run_fp8_attention(dit, q, k, v)
    rng = np.random.default_rng(1)
    rows = np.sort(np.concatenate([rng.choice(L, 40, replace=False), [0, L - 1, 511, 512]]))
    ref, slack = O.attention_fp8(O.to64(q), O.to64(k), O.to64(v), rows=rows, tie_fp32=True)
    err = _err_with_slack(got[:, :, rows], ref, slack)
    _say(f"  err {err:.3e} (without slack {parity_err_bf16_stored(got[:, :, rows], ref):.3e})")
    assert err <= TOL_FP8


# ---------------------------------------------------------------- blocks

def _block_fp8_setup(dit, dims, w, kind, x_dtype):
    params = DI.block_params(dims, "bf16", kind)
    dev = {}
    for n, t in params.items():
        dev[n] = t.cuda() if n.endswith(".w") else t.float().cuda()
    dev8 = dit.quantize_block_params(dev)
    inp = DI.block_inputs(w, kind)
    blk = dit.make_double_block(dev8) if kind == "double" else dit.make_single_block(dev8)
    dd = dit.dims_of(w.B, w.Lt, w.grid_h, w.grid_w, dims.D, dims.H, dims.F)
    rope = dit.dit_rope_table(w.grid_h, w.grid_w, w.Lt, dims.d)
    ws = dit.workspace(dd, dit.DIT_WS_BLOCK)
    x = inp["x"].to(x_dtype).cuda()
    return params, dev8, inp, blk, dd, rope, ws, x


def _oracle_block_fp8(params, inp, w, dims, kind, fp8=True):
    P = {k: O.to64(v) for k, v in params.items()}
    x = O.to64(inp["x"])
    mod = O.to64(inp["mod"])
    ang = O.rope_table(O.image_positions(w.grid_h, w.grid_w, w.Lt), dims.d)
    if kind == "double":
        xt, xi = O.double_block(x[:, :w.Lt], x[:, w.Lt:], mod[:, :6], mod[:, 6:], P, ang, dims.H,
                                fp8=fp8)
        return np.concatenate([xt, xi], axis=1)
    return O.single_block(x, mod, P, ang, dims.H, fp8=fp8)


# The fp8 branch (x_out - x_in) end to end.  Each stage of an fp8 block agrees
# with the oracle on identical inputs (codes bit-exact, floats within 1e-4:
# test_gpu_fp8_stages.py); end to end the two differ only where near-tie codes
# (LN output, attention's P) were decided the other way and moved later
# quantisation inputs -- one such P code moves an fp8 attention output by up to
# ~0.2 of its RMS, so the largest element of the difference is not a stable
# measure (it varies by tens of percent between equally valid evaluations).  The
# branch is therefore held to RMS properties against the unquantised oracle
# branch E, like the MXFP4 blocks: RMS(kernel - oracle) <= FP8_TIE_SHARE x
# RMS(oracle - E), and RMS(kernel - E) <= 1.05 x RMS(oracle - E).  A wrong scale,
# a skipped quantisation or a mixed-up head fails both.
FP8_TIE_SHARE = 0.5


def _rms(a):
    return float(np.sqrt(np.mean(np.square(a))))


def _check_fp8_branch(got, ref8, exact, x0):
    b_gpu, b_orc, b_ex = got - x0, ref8 - x0, exact - x0
    q_orc = _rms(b_orc - b_ex)
    d_rms = _rms(b_gpu - b_orc)
    e_gpu = _rms(b_gpu - b_ex)
    _say(f"  branch RMS: kernel vs oracle fp8 {d_rms:.3e} ({d_rms / q_orc:.3f} of the fp8 effect "
         f"{q_orc:.3e}); kernel vs unquantised {e_gpu:.3e}; max-norm kernel vs oracle "
         f"{parity_err(b_gpu, b_orc):.3e}")
    assert d_rms <= FP8_TIE_SHARE * q_orc
    assert e_gpu <= 1.05 * q_orc


FP8_BLOCK_CASES = [
    # D, H, F, B, Lt, grid_h, grid_w, kind, x dtype   (L = Lt + grid_h * grid_w, a multiple of 16)
    (256, 2, 512, 2, 16, 6, 8, "double", torch.float32),
    (3072, 24, 12288, 1, 32, 12, 20, "double", torch.float32),
    (3072, 24, 12288, 2, 16, 8, 10, "double", torch.bfloat16),
    (256, 2, 512, 2, 16, 6, 8, "single", torch.float32),
    (3072, 24, 12288, 1, 32, 12, 20, "single", torch.float32),
    (256, 2, 512, 2, 0, 4, 8, "double", torch.float32),     # image tokens only
    # one 128-row GEMM wave tile runs from batch 1's image rows through batch 0's
    # text rows into batch 1's text rows (Li = 112, Lt = 16, B = 2)
    (256, 2, 512, 2, 16, 8, 14, "double", torch.float32),
]


@pytest.mark.parametrize("D,H,F,B,Lt,gh,gw,kind,xdt", FP8_BLOCK_CASES)
def test_block_forward_fp8(dit, D, H, F, B, Lt, gh, gw, kind, xdt):
    _say(f"fp8 block {kind} D={D} B={B} Lt={Lt} grid={gh}x{gw} x={xdt}")
    dims = DI.Dims(D=D, H=H, F=F, n_double=1, n_single=0)
    w = DI.Workload("t", dims, B=B, grid_h=gh, grid_w=gw, Lt=Lt, dtype="fp8")
    params, dev8, inp, blk, dd, rope, ws, x = _block_fp8_setup(dit, dims, w, kind, xdt)
    x_in = x.clone()
    dit.dit_block_forward(dd, blk, x, inp["mod"].cuda(), rope, ws, dtype=dit.DIT_FP8)
    torch.cuda.synchronize()
    ref = _oracle_block_fp8(params, inp, w, dims, kind)
    got = x.double().cpu().numpy()
    err = parity_err_bf16_stored(got, ref) if xdt == torch.bfloat16 else parity_err(got, ref)
    _say(f"  x_out err {err:.3e}")
    assert err <= TOL_FP8
    if xdt == torch.float32:
        exact = _oracle_block_fp8(params, inp, w, dims, kind, fp8=False)
        _check_fp8_branch(got, ref, exact, O.to64(inp["x"]))


@pytest.mark.parametrize("half", ["attention", "mlp"])
def test_block_forward_fp8_double_halves(dit, half):
    """Each half of the fp8 double block on its own (the other half's gates set
    to 0): the block output meets the fp8 bound and the branch is held to the
    share of the oracle's own quantisation effect described above."""
    _say(f"fp8 double block, {half} half only")
    dims = DI.Dims(D=3072, H=24, F=12288, n_double=1, n_single=0)
    w = DI.Workload("t", dims, B=1, grid_h=12, grid_w=20, Lt=32, dtype="fp8")
    params, dev8, inp, blk, dd, rope, ws, x = _block_fp8_setup(dit, dims, w, "double",
                                                               torch.float32)
    off = (5, 11) if half == "attention" else (2, 8)      # gate2 or gate1, image and text
    for i in off:
        inp["mod"][:, i] = 0.0
    dit.dit_block_forward(dd, blk, x, inp["mod"].cuda(), rope, ws, dtype=dit.DIT_FP8)
    torch.cuda.synchronize()
    x0 = O.to64(inp["x"])
    got = x.double().cpu().numpy()
    ref8 = _oracle_block_fp8(params, inp, w, dims, "double")
    P = {k: O.to64(v) for k, v in params.items()}
    mod = O.to64(inp["mod"])
    ang = O.rope_table(O.image_positions(w.grid_h, w.grid_w, w.Lt), dims.d)
    xt, xi = O.double_block(x0[:, :w.Lt], x0[:, w.Lt:], mod[:, :6], mod[:, 6:], P, ang, dims.H)
    exact = np.concatenate([xt, xi], axis=1)
    err = parity_err(got, ref8)
    _say(f"  x_out err {err:.3e}")
    _check_fp8_branch(got, ref8, exact, x0)
    assert err <= TOL_FP8


@pytest.mark.timeout(400)
def test_block_forward_fp8_flux_1024(dit):
    """The full fp8 double block at the 1024px shape (4096 image + 512 text tokens)."""
    _say("fp8 block double full 1024px")
    w = DI.WORKLOADS["block_1024"]
    dims = w.dims
    params, dev8, inp, blk, dd, rope, ws, x = _block_fp8_setup(dit, dims, w, "double",
                                                               torch.float32)
    dit.dit_block_forward(dd, blk, x, inp["mod"].cuda(), rope, ws, dtype=dit.DIT_FP8)
    torch.cuda.synchronize()
    got = x.double().cpu().numpy()
    del dev8, ws
    ref = _oracle_block_fp8(params, inp, w, dims, "double")
    err = parity_err(got, ref)
    _say(f"  x_out err {err:.3e}")
    assert err <= TOL_FP8
    exact = _oracle_block_fp8(params, inp, w, dims, "double", fp8=False)
    _check_fp8_branch(got, ref, exact, O.to64(inp["x"]))



@pytest.mark.timeout(600)        # the fp64 oracle's share takes ~2 min on 8 cores
def test_block_forward_fp8_2048_cfg_sampled(dit):
    """The fp8 double block at the 2048px CFG-pair shape of the fp8 model step
    (2 x (16384 image + 512 text) tokens, D 3072, fp32 residual stream, per-batch
    modulation), run whole on the GPU and compared on ~80 sampled rows per batch
    element.  Activation scales are per token and attention scales per (batch,
    head) over all rows, so the oracle's sampled rows equal its full block there."""
    dims = DI.Dims(D=3072, H=24, F=12288, n_double=1, n_single=0)
    w = DI.Workload("t", dims, B=2, grid_h=128, grid_w=128, Lt=512, dtype="fp8")
    _say(f"fp8 block double sampled 2048px B={w.B} L={w.L}")
    params, dev8, inp, blk, dd, rope, ws, x = _block_fp8_setup(dit, dims, w, "double",
                                                               torch.float32)
    dit.dit_block_forward(dd, blk, x, inp["mod"].cuda(), rope, ws, dtype=dit.DIT_FP8)
    torch.cuda.synchronize()
    rows = sampled_block_rows(w.Lt, w.L, 32, 2049)
    got = x[:, torch.from_numpy(rows).cuda()].double().cpu().numpy()
    del dev8, ws, x
    P = {k: O.to64(v) for k, v in params.items()}
    x64 = O.to64(inp["x"])
    m64 = O.to64(inp["mod"])
    ang = O.rope_table(O.image_positions(w.grid_h, w.grid_w, w.Lt), dims.d)
    ref = O.double_block_rows(x64[:, :w.Lt], x64[:, w.Lt:], m64[:, :6], m64[:, 6:], P, ang,
                              dims.H, rows, fp8=True)
    err = parity_err(got, ref)
    _say(f"  rows {len(rows)} x_out err {err:.3e}")
    assert err <= TOL_FP8
    exact = O.double_block_rows(x64[:, :w.Lt], x64[:, w.Lt:], m64[:, :6], m64[:, 6:], P, ang,
                                dims.H, rows)
    _check_fp8_branch(got, ref, exact, x64[:, rows])


# ---------------------------------------------------------------- full step

SMALL = DI.Dims(D=256, H=2, F=512, n_double=2, n_single=2)


@pytest.mark.parametrize("B,guidance", [(1, 0.0), (2, 3.5)])
def test_denoise_loop_fp8_teacher_forced(dit, B, guidance):
    w = DI.Workload("f", SMALL, B=B, grid_h=8, grid_w=8, Lt=32, dtype="fp8", steps=4, shift=3.0,
                    guidance=guidance)
    params = dict(DI.iter_params(SMALL, "bf16"))
    gm = dit.GPUModel(SMALL, w.B, w.Lt, w.grid_h, w.grid_w, params, guidance=w.guidance,
                      dtype=dit.DIT_FP8)
    P = {k: O.to64(v) for k, v in params.items()}
    sig = dit.dit_sigmas(w.steps, w.shift)
    mods = dit.dit_modulation(gm, sig[:-1])
    ws = dit.workspace(gm.model.dims, dit.DIT_WS_STEP)
    lat_g = DI.latents(w)[0].clone().cuda()
    txt = DI.text_tokens(w)
    errs = []
    for i in range(w.steps):
        x_in = lat_g.double().cpu().numpy()[None]
        dit.dit_denoise_step(gm, mods[i], txt.cuda(), lat_g, sig[i], sig[i + 1], None, ws)
        torch.cuda.synchronize()
        ref, _ = O.denoise_step(P, SMALL, w, x_in, O.to64(txt), i, np.array(sig), None, fp8=True)
        got = lat_g.double().cpu().numpy()[None]
        errs.append(parity_err(got - x_in, ref - x_in))
    _say(f"fp8 loop B={B} step-update errs {['%.2e' % e for e in errs]}")
    assert max(errs) <= TOL_FP8
