"""GPU parity of the fp32 (reference-precision) path against the fp64 oracle.

The tiny fp32 model (2 double blocks, hidden 256, 4 heads of 64, MLP 1024,
16x16 patch grid + 32 text tokens, 4 Euler steps) runs every step in fp32.
Bound: max|gpu - oracle| / RMS(oracle) <= 1e-4 (fp32 arithmetic with fp32
accumulation over K <= 1280 stays near 1e-6 relative; the bound leaves room for
the transcendental approximations in GELU, SiLU and exp2).
"""
import math
import sys

import numpy as np
import pytest
import torch

import dit_inputs as DI
import oracle as O
from _helpers import parity_err

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4


@pytest.fixture(scope="module")
def dit():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from image_generation_amd import dit as D
    return D


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _f32(shape, seed, std=1.0):
    return DI.randn(shape, seed, std, "f32")


@pytest.mark.parametrize("B,H,L,d", [(1, 4, 288, 64), (2, 1, 100, 64), (1, 2, 7, 32),
                                     (1, 1, 1, 64), (2, 3, 130, 32)])
def test_attention_f32(dit, B, H, L, d):
    _say(f"attention fp32 B={B} H={H} L={L} d={d}")
    q, k, v = _f32((B, H, L, d), 81), _f32((B, H, L, d), 82), _f32((B, H, L, d), 83)
    o = torch.empty((B, L, H * d), dtype=torch.float32, device="cuda")
    dit.dit_attention(q.cuda(), k.cuda(), v.cuda(), o)
    torch.cuda.synchronize()
    got = o.cpu().double().numpy().reshape(B, L, H, d).transpose(0, 2, 1, 3)
    err = parity_err(got, O.attention(O.to64(q), O.to64(k), O.to64(v)))
    _say(f"  err {err:.3e}")
    assert err <= TOL_F32


def test_attention_f32_identical_keys(dit):
    B, H, L, d = 1, 2, 77, 64
    q = _f32((B, H, L, d), 84)
    k = _f32((B, H, 1, d), 85).expand(B, H, L, d).contiguous()
    v = _f32((B, H, L, d), 86)
    o = torch.empty((B, L, H * d), dtype=torch.float32, device="cuda")
    dit.dit_attention(q.cuda(), k.cuda(), v.cuda(), o)
    torch.cuda.synchronize()
    got = o.cpu().double().numpy().reshape(B, L, H, d).transpose(0, 2, 1, 3)
    mean = O.to64(v).mean(axis=2, keepdims=True)
    assert parity_err(got, np.broadcast_to(mean, got.shape)) <= TOL_F32


F32_BLOCK_CASES = [
    # D, H, F, B, Lt, grid_h, grid_w, kind
    (256, 4, 1024, 1, 32, 16, 16, "double"),
    (256, 4, 1024, 2, 8, 5, 8, "double"),
    (256, 4, 1024, 1, 32, 16, 16, "single"),
    (512, 16, 2048, 2, 16, 3, 8, "single"),
]


@pytest.mark.parametrize("D,H,F,B,Lt,gh,gw,kind", F32_BLOCK_CASES)
def test_block_forward_f32(dit, D, H, F, B, Lt, gh, gw, kind):
    _say(f"fp32 block {kind} D={D} H={H} B={B} Lt={Lt} grid={gh}x{gw}")
    dims = DI.Dims(D=D, H=H, F=F, n_double=1, n_single=0)
    w = DI.Workload("t", dims, B=B, grid_h=gh, grid_w=gw, Lt=Lt, dtype="f32")
    params = DI.block_params(dims, "f32", kind)
    dev = {n: t.cuda() for n, t in params.items()}
    inp = DI.block_inputs(w, kind)
    blk = dit.make_double_block(dev) if kind == "double" else dit.make_single_block(dev)
    dd = dit.dims_of(w.B, w.Lt, w.grid_h, w.grid_w, D, H, F)
    rope = dit.dit_rope_table(w.grid_h, w.grid_w, w.Lt, dims.d)
    ws = dit.workspace(dd, dit.DIT_WS_BLOCK)
    x = inp["x"].cuda()
    x_in = x.clone()
    dit.dit_block_forward(dd, blk, x, inp["mod"].cuda(), rope, ws, dtype=dit.DIT_F32)
    torch.cuda.synchronize()
    P = {k: O.to64(v) for k, v in params.items()}
    x0 = O.to64(inp["x"])
    mod = O.to64(inp["mod"])
    ang = O.rope_table(O.image_positions(w.grid_h, w.grid_w, w.Lt), dims.d)
    if kind == "double":
        xt, xi = O.double_block(x0[:, :Lt], x0[:, Lt:], mod[:, :6], mod[:, 6:], P, ang, H)
        ref = np.concatenate([xt, xi], axis=1)
    else:
        ref = O.single_block(x0, mod, P, ang, H)
    got = x.double().cpu().numpy()
    err = parity_err(got, ref)
    derr = parity_err(got - x_in.double().cpu().numpy(), ref - x0)
    _say(f"  x_out err {err:.3e} branch err {derr:.3e}")
    assert err <= TOL_F32 and derr <= TOL_F32


def _run_tiny(dit, threshold, enabled, teacher):
    w = DI.WORKLOADS["tiny_fp32"]
    dims = w.dims
    params = dict(DI.iter_params(dims, "f32"))
    gm = dit.GPUModel(dims, w.B, w.Lt, w.grid_h, w.grid_w, params, dtype=dit.DIT_F32)
    P = {k: O.to64(v) for k, v in params.items()}
    sig = dit.dit_sigmas(w.steps, w.shift)
    mods = dit.dit_modulation(gm, sig[:-1])
    ws = dit.workspace(gm.model.dims, dit.DIT_WS_STEP)
    lat = DI.latents(w)
    txt = DI.text_tokens(w)
    lat_g = lat[0].clone().cuda()
    cache = dit.FBCache(w.B, w.Li, dims.D, threshold, enabled)
    ocache = O.FBCacheState(enabled, threshold)
    olat = O.to64(lat)
    errs, dec = [], []
    for i in range(w.steps):
        x_in = lat_g.double().cpu().numpy()[None]
        rel, skip = dit.dit_denoise_step(gm, mods[i], txt.cuda(), lat_g, sig[i], sig[i + 1],
                                         cache, ws)
        torch.cuda.synchronize()
        start = x_in if teacher else olat
        olat_new, info = O.denoise_step(P, dims, w, start, O.to64(txt), i, np.array(sig),
                                        ocache if enabled else None,
                                        force_skip=skip if enabled else None)
        if enabled and np.isfinite(info["rel"]) and abs(info["rel"] - threshold) > 1e-3:
            assert skip == (info["rel"] < threshold), (i, rel, info["rel"])
        got = lat_g.double().cpu().numpy()[None]
        errs.append(parity_err(got - x_in, olat_new - start))
        dec.append((rel, info["rel"], skip))
        olat = olat_new
    return errs, dec, lat_g.double().cpu().numpy()[None], olat


@pytest.mark.parametrize("threshold,enabled", [(0.0, False), (0.12, True), (math.inf, True)])
def test_tiny_fp32_loop_teacher_forced(dit, threshold, enabled):
    errs, dec, _, _ = _run_tiny(dit, threshold, enabled, teacher=True)
    _say(f"tiny fp32 loop tau={threshold} step errs {['%.2e' % e for e in errs]} decisions {dec}")
    assert max(errs) <= TOL_F32


def test_tiny_fp32_loop_free_running(dit):
    errs, dec, got, ref = _run_tiny(dit, 0.0, False, teacher=False)
    e2e = parity_err(got, ref)
    _say(f"tiny fp32 free-running end-to-end err {e2e:.3e}")
    assert e2e <= TOL_F32


@pytest.mark.parametrize("warmup,max_skips,want", [(3, 2, "FFFSSFSS"), (0, 1, "FSFSFSFS")])
def test_tiny_fp32_loop_skip_policy(dit, warmup, max_skips, want):
    # tau = +inf: the pattern of skips is the policy's (warm-up, at most max_skips in
    # a row); each step is compared with the oracle step from the same latents
    import dataclasses
    w = dataclasses.replace(DI.WORKLOADS["tiny_fp32"], steps=8)
    dims = w.dims
    params = dict(DI.iter_params(dims, "f32"))
    gm = dit.GPUModel(dims, w.B, w.Lt, w.grid_h, w.grid_w, params, dtype=dit.DIT_F32)
    P = {k: O.to64(v) for k, v in params.items()}
    sig = dit.dit_sigmas(w.steps, w.shift)
    mods = dit.dit_modulation(gm, sig[:-1])
    ws = dit.workspace(gm.model.dims, dit.DIT_WS_STEP)
    lat_g = DI.latents(w)[0].clone().cuda()
    txt = DI.text_tokens(w)
    cache = dit.FBCache(w.B, w.Li, dims.D, math.inf, True, warmup_steps=warmup,
                        max_skips=max_skips)
    ocache = O.FBCacheState(True, math.inf, warmup_steps=warmup, max_skips=max_skips)
    got, errs = [], []
    for i in range(w.steps):
        x_in = lat_g.double().cpu().numpy()[None]
        _, skip = dit.dit_denoise_step(gm, mods[i], txt.cuda(), lat_g, sig[i], sig[i + 1],
                                       cache, ws)
        torch.cuda.synchronize()
        ref, info = O.denoise_step(P, dims, w, x_in, O.to64(txt), i, np.array(sig), ocache)
        assert skip == info["skip"], (i, skip, info["skip"])
        got.append("S" if skip else "F")
        errs.append(parity_err(lat_g.double().cpu().numpy()[None] - x_in, ref - x_in))
    _say(f"skip policy warmup={warmup} max={max_skips}: {''.join(got)} errs "
         f"{['%.1e' % e for e in errs]}")
    assert "".join(got) == want
    assert cache.steps_done == w.steps and cache.skip_run == ocache.skip_run
    assert max(errs) <= TOL_F32


def test_tiny_fp32_modulation(dit):
    w = DI.WORKLOADS["tiny_fp32"]
    params = dict(DI.iter_params(w.dims, "f32"))
    gm = dit.GPUModel(w.dims, w.B, w.Lt, w.grid_h, w.grid_w, params, dtype=dit.DIT_F32)
    P = {k: O.to64(v) for k, v in params.items()}
    sig = O.sigmas(w.steps, w.shift)[:-1]
    out = dit.dit_modulation(gm, list(sig)).double().cpu().numpy()
    c = O.time_embed(P, sig)
    names = [f"double{j}.{s}.mod" for j in range(2) for s in ("img", "txt")] + ["final.mod"]
    ref = np.concatenate([O.linear(O.silu(c), P[n + ".w"], P[n + ".b"]) for n in names], axis=1)
    err = parity_err(out, ref)
    _say(f"tiny fp32 modulation err {err:.3e}")
    assert err <= TOL_F32
