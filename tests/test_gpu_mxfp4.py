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


# ---------------------------------------------------------------- MXFP4 blocks
#
# The oracle's MXFP4 block quantises the same bf16 weights the same way and every
# linear input after rounding it to bf16, as the kernel stores it.  Where the two
# sides see the same bf16 input they take the same E2M1 / E8M0 decisions (the
# quantiser is bit-exact, the GEMM agrees to ~1e-7), so the MLP half of a double
# block (attention gates 0) must agree to fp32 accumulation level: x_out within
# 1e-5 of RMS(x), the branch within 1e-3 of its RMS.  Attention is not bit-exact
# (bf16 / fp16 storage of Q, K, V, P and O in the kernel, fp64 in the oracle), and
# a one-ulp change of a stored bf16 attention output flips the 4-bit code of the
# few values that sit on a rounding boundary by a whole grid step; those flips
# then move every later quantisation input.  In the oracle alone, rounding Q, K,
# V and O to their storage formats moves a 3072-wide MXFP4 block's branch by more
# than its RMS at the worst element, against 0.4% for the bf16 block.  The full
# block is therefore checked as a property: the kernel's branch is as far from
# the unquantised branch as the oracle's MXFP4 branch is (RMS, within 5%), and
# much closer to the oracle's MXFP4 branch than that (RMS, at most 35% of the
# MXFP4 error itself) -- a kernel that skipped the quantisation, used a wrong
# scale or mixed up a group fails one of the two.
TOL_MX4_HALF_X = 1e-5
TOL_MX4_HALF_BRANCH = 1e-3
MX4_SAME_ERROR = 1.05
MX4_CLOSER = 0.35

MX4_BLOCK_CASES = [
    # D, H, F, B, Lt, grid_h, grid_w, kind
    (256, 2, 512, 2, 16, 6, 8, "double"),
    (256, 2, 512, 2, 16, 6, 8, "single"),
    (256, 2, 512, 2, 0, 4, 8, "double"),          # image tokens only
    (256, 2, 512, 2, 24, 8, 14, "double"),        # text group starts at row 224
    (3072, 24, 12288, 1, 32, 12, 20, "double"),
    (3072, 24, 12288, 1, 32, 12, 20, "single"),
]


def _rms_rel(a, b):
    return float(np.sqrt(np.mean((a - b) ** 2)) / np.sqrt(np.mean(b ** 2)))


def _mx4_block(dit, dims, w, kind, zero_gates=(), attn8=False):
    """Run the MXFP4 block on the GPU -> (gpu, oracle MXFP4, oracle unquantised, x_in);
    attn8: e4m3 attention (DIT_MXFP4_FP8ATTN)."""
    params = DI.block_params(dims, "bf16", kind)
    dev = {n: (t.cuda() if n.endswith(".w") else t.float().cuda()) for n, t in params.items()}
    dev4 = dit.quantize_block_params_mx(dev)
    inp = DI.block_inputs(w, kind)
    for i in zero_gates:
        inp["mod"][:, i] = 0.0
    blk = dit.make_double_block(dev4) if kind == "double" else dit.make_single_block(dev4)
    dd = dit.dims_of(w.B, w.Lt, w.grid_h, w.grid_w, dims.D, dims.H, dims.F)
    rope = dit.dit_rope_table(w.grid_h, w.grid_w, w.Lt, dims.d)
    ws = dit.workspace(dd, dit.DIT_WS_BLOCK)
    x = inp["x"].float().cuda()
    dit.dit_block_forward(dd, blk, x, inp["mod"].cuda(), rope, ws,
                          dtype=dit.DIT_MXFP4_FP8ATTN if attn8 else dit.DIT_MXFP4)
    torch.cuda.synchronize()
    got = x.double().cpu().numpy()
    del dev, dev4, ws
    P = {k: O.to64(v) for k, v in params.items()}
    x0 = O.to64(inp["x"].float())
    mod = O.to64(inp["mod"])
    ang = O.rope_table(O.image_positions(w.grid_h, w.grid_w, w.Lt), dims.d)

    def oracle_block(mx4):
        if kind == "double":
            xt, xi = O.double_block(x0[:, :w.Lt], x0[:, w.Lt:], mod[:, :6], mod[:, 6:], P, ang,
                                    dims.H, mx4=mx4, attn8=attn8 and mx4)
            return np.concatenate([xt, xi], axis=1)
        return O.single_block(x0, mod, P, ang, dims.H, mx4=mx4, attn8=attn8 and mx4)

    return got, oracle_block(True), oracle_block(False), x0


def _check_mx4_property(got, ref4, exact, x0):
    e_gpu = _rms_rel(got - x0, exact - x0)
    e_orc = _rms_rel(ref4 - x0, exact - x0)
    e_go = _rms_rel(got - x0, ref4 - x0) * np.sqrt(np.mean((ref4 - x0) ** 2)) / \
        np.sqrt(np.mean((exact - x0) ** 2))
    _say(f"  branch RMS vs unquantised: kernel {e_gpu:.4f} oracle {e_orc:.4f}; "
         f"kernel vs oracle {e_go:.4f} ({e_go / e_orc:.2f} of the MXFP4 error)")
    assert np.isfinite(got).all()
    assert e_gpu <= MX4_SAME_ERROR * e_orc
    assert e_go <= MX4_CLOSER * e_orc


@pytest.mark.parametrize("attn8", [False, True])
@pytest.mark.parametrize("D,H,F,B,Lt,gh,gw,kind", MX4_BLOCK_CASES)
def test_block_forward_mxfp4(dit, D, H, F, B, Lt, gh, gw, kind, attn8):
    _say(f"mxfp4 block {kind} D={D} B={B} Lt={Lt} grid={gh}x{gw} e4m3 attention={attn8}")
    dims = DI.Dims(D=D, H=H, F=F, n_double=1, n_single=0)
    w = DI.Workload("t", dims, B=B, grid_h=gh, grid_w=gw, Lt=Lt, dtype="bf16")
    got, ref4, exact, x0 = _mx4_block(dit, dims, w, kind, attn8=attn8)
    _say(f"  x_out max err vs oracle {parity_err(got, ref4):.3e}")
    _check_mx4_property(got, ref4, exact, x0)


@pytest.mark.parametrize("D,H,F", [(256, 2, 512), (3072, 24, 12288)])
def test_block_forward_mxfp4_mlp_half(dit, D, H, F):
    """Attention gates 0: only the MLP half moves x, and its quantisation decisions
    are the oracle's."""
    _say(f"mxfp4 double block, MLP half only, D={D}")
    dims = DI.Dims(D=D, H=H, F=F, n_double=1, n_single=0)
    w = DI.Workload("t", dims, B=1, grid_h=12, grid_w=20, Lt=32, dtype="bf16")
    got, ref4, exact, x0 = _mx4_block(dit, dims, w, "double", zero_gates=(2, 8))
    err = parity_err(got, ref4)
    derr = parity_err(got - x0, ref4 - x0)
    _say(f"  x_out err {err:.3e} branch err {derr:.3e}")
    assert err <= TOL_MX4_HALF_X
    assert derr <= TOL_MX4_HALF_BRANCH


@pytest.mark.parametrize("attn8", [False, True])
def test_block_forward_mxfp4_flux_1024(dit, attn8):
    """The full MXFP4 double block at the 1024px shape (4096 image + 512 text tokens)."""
    _say(f"mxfp4 block double full 1024px, e4m3 attention={attn8}")
    w = DI.WORKLOADS["block_1024"]
    got, ref4, exact, x0 = _mx4_block(dit, w.dims, w, "double", attn8=attn8)
    _check_mx4_property(got, ref4, exact, x0)


@pytest.mark.parametrize("B,guidance,attn8", [(1, 0.0, False), (2, 3.5, False), (2, 3.5, True)])
def test_denoise_loop_mxfp4_teacher_forced(dit, B, guidance, attn8):
    """Four Euler steps of a small MXFP4 model (2 double + 2 single blocks), alone and
    as a CFG pair.  At the step level the unquantised final layer carries most of
    the update, so the MXFP4 effect is small next to the bf16 storage noise that
    both GPU paths share, and CFG multiplies that noise by the guidance scale where
    the two rows' roundings differ.  Each step, from the same latents: the GPU's
    MXFP4 update is no further from the oracle's MXFP4 update than the GPU's own
    bf16 update is from the exact one plus half the oracle's MXFP4 effect, and no
    further from the exact update than that bf16 noise plus 1.1 times the oracle's
    MXFP4 error (RMS over the update, relative to the exact update's RMS)."""
    small = DI.Dims(D=256, H=2, F=512, n_double=2, n_single=2)
    w = DI.Workload("m", small, B=B, grid_h=8, grid_w=8, Lt=32, dtype="bf16", steps=4, shift=3.0,
                    guidance=guidance)
    _say(f"mxfp4 loop B={B} guidance={guidance} e4m3 attention={attn8}")
    params = dict(DI.iter_params(small, "bf16"))
    q4 = dit.DIT_MXFP4_FP8ATTN if attn8 else dit.DIT_MXFP4
    gms = {dt: dit.GPUModel(small, w.B, w.Lt, w.grid_h, w.grid_w, params, guidance=w.guidance,
                            dtype=dt) for dt in (dit.DIT_BF16, q4)}
    P = {k: O.to64(v) for k, v in params.items()}
    sig = dit.dit_sigmas(w.steps, w.shift)
    mods = {dt: dit.dit_modulation(gm, sig[:-1]) for dt, gm in gms.items()}
    ws = dit.workspace(gms[q4].model.dims, dit.DIT_WS_STEP)
    lat = DI.latents(w)[0].clone().cuda()
    txt = DI.text_tokens(w)
    for i in range(w.steps):
        x_in = lat.double().cpu().numpy()[None]
        out = {}
        for dt, gm in gms.items():
            l2 = lat.clone()
            dit.dit_denoise_step(gm, mods[dt][i], txt.cuda(), l2, sig[i], sig[i + 1], None, ws)
            torch.cuda.synchronize()
            out[dt] = l2
        ref4, _ = O.denoise_step(P, small, w, x_in, O.to64(txt), i, np.array(sig), None, mx4=True,
                                 attn8=attn8)
        exact, _ = O.denoise_step(P, small, w, x_in, O.to64(txt), i, np.array(sig), None)
        g4 = out[q4].double().cpu().numpy()[None]
        g16 = out[dit.DIT_BF16].double().cpu().numpy()[None]
        n = np.sqrt(np.mean((exact - x_in) ** 2))
        e_b = np.sqrt(np.mean((g16 - exact) ** 2)) / n
        e_q = np.sqrt(np.mean((ref4 - exact) ** 2)) / n
        e_go = np.sqrt(np.mean((g4 - ref4) ** 2)) / n
        e_ge = np.sqrt(np.mean((g4 - exact) ** 2)) / n
        _say(f"  step {i}: bf16 noise {e_b:.4f}, oracle MXFP4 effect {e_q:.4f}, "
             f"kernel MXFP4 vs oracle {e_go:.4f}, vs exact {e_ge:.4f}")
        assert np.isfinite(g4).all()
        assert e_go <= e_b + 0.5 * e_q
        assert e_ge <= e_b + 1.1 * e_q
        lat = out[q4]
