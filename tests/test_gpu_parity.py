"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerance (bf16 path): max|gpu - oracle| / RMS(oracle) <= 2e-2 over the compared
tensor.  Sizes span several tiles and ragged tails; the full FLUX block shape
(4096 + 512 tokens, D 3072) is compared whole.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import dit_inputs as DI
import oracle as O
from _helpers import parity_err, parity_err_bf16_stored, sampled_block_rows

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
# Branch-only check (x_out - x_in with an fp32 residual stream): the branch passes
# through about six bf16 roundings (LN out, Q/K/V, P, O, LN2 out, MLP hidden),
# each of relative RMS <= 2^-9/sqrt(3) ~ 1.1e-3 and independent, so the branch
# error has relative RMS ~ sqrt(6) * 1.1e-3 ~ 2.8e-3 and its maximum over ~10^6
# elements sits near 5 sigma ~ 1.4e-2 .. 3e-2.  Twice that is the bound.
TOL_BRANCH = 6e-2


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


# ---------------------------------------------------------------- attention

def _attn_ref_rows(q, k, v, rows):
    """fp64 softmax(q k^T / sqrt(d)) v for the selected query rows, all (b, h)."""
    d = q.shape[-1]
    out = np.empty(q.shape[:2] + (len(rows), d))
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            s = q[b, h, rows] @ k[b, h].T / math.sqrt(d)
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[b, h] = p @ v[b, h]
    return out


@pytest.mark.parametrize("B,H,L,d", [
    (1, 1, 1, 128), (1, 2, 7, 64), (1, 1, 8, 128), (2, 2, 65, 64), (1, 2, 264, 128),
    (2, 1, 520, 64), (1, 3, 1032, 128), (2, 2, 333, 128), (1, 1, 4097, 64), (1, 2, 4601, 128)])
def test_attention_small(dit, B, H, L, d):
    """Every tile path with ragged tails (L not a multiple of the 64-key tile or
    the 256-query tile, down to a single token) and both head sizes."""
    _say(f"attention B={B} H={H} L={L} d={d}")
    q = _bf16((B, H, L, d), 11)
    k = _bf16((B, H, L, d), 12)
    v = _bf16((B, H, L, d), 13)
    o = torch.empty((B, L, H * d), dtype=torch.bfloat16, device="cuda")
    dit.dit_attention(q.cuda(), k.cuda(), v.cuda(), o)
    torch.cuda.synchronize()
    ref = O.attention(O.to64(q), O.to64(k), O.to64(v))          # [B, H, L, d]
    got = o.float().cpu().double().numpy().reshape(B, L, H, d).transpose(0, 2, 1, 3)
    err = parity_err_bf16_stored(got, ref)
    _say(f"  err {err:.3e}")
    assert err <= TOL_BF16


@pytest.mark.parametrize("d", [64, 128])
def test_attention_identical_keys(dit, d):
    B, H, L = 1, 2, 200
    q = _bf16((B, H, L, d), 21)
    k = _bf16((B, H, 1, d), 22).expand(B, H, L, d).contiguous()
    v = _bf16((B, H, L, d), 23)
    o = torch.empty((B, L, H * d), dtype=torch.bfloat16, device="cuda")
    dit.dit_attention(q.cuda(), k.cuda(), v.cuda(), o)
    torch.cuda.synchronize()
    got = o.float().cpu().double().numpy().reshape(B, L, H, d).transpose(0, 2, 1, 3)
    mean = O.to64(v).mean(axis=2, keepdims=True)
    assert parity_err_bf16_stored(got, np.broadcast_to(mean, got.shape)) <= TOL_BF16


@pytest.mark.parametrize("B,L,H,d", [(1, 4608, 24, 128), (2, 16896, 24, 128),
                                     (2, 16896, 3, 128), (1, 4097, 24, 128), (1, 4601, 48, 64)])
def test_attention_full_size_sampled(dit, B, L, H, d):
    """FLUX head layout at 1024px (4608 tokens) and the 2048px CFG pair (16896),
    24 heads, and one rank's 3 heads of the latter under 8-way head sharding;
    ragged full-size lengths 4097 and 4601 (head dim 128 and 64)."""
    _say(f"attention full B={B} L={L} H={H} d={d}")
    q = _bf16((B, H, L, d), 31)
    k = _bf16((B, H, L, d), 32)
    v = _bf16((B, H, L, d), 33)
    o = torch.empty((B, L, H * d), dtype=torch.bfloat16, device="cuda")
    dit.dit_attention(q.cuda(), k.cuda(), v.cuda(), o)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.choice(L, 60, replace=False),
                                     [0, L - 1, 255, 256, 511, 512, L - 2]]))
    ref = _attn_ref_rows(O.to64(q), O.to64(k), O.to64(v), rows)
    got = o.float().cpu().double().numpy().reshape(B, L, H, d)[:, rows].transpose(0, 2, 1, 3)
    err = parity_err_bf16_stored(got, ref)
    _say(f"  err {err:.3e}")
    assert err <= TOL_BF16


# ---------------------------------------------------------------- blocks

def _block_setup(dit, dims, w, kind, x_dtype):
    params = DI.block_params(dims, "bf16", kind)
    dev = {}
    for n, t in params.items():
        dev[n] = t.cuda() if n.endswith(".w") else t.float().cuda()
    inp = DI.block_inputs(w, kind)
    blk = dit.make_double_block(dev) if kind == "double" else dit.make_single_block(dev)
    dd = dit.dims_of(w.B, w.Lt, w.grid_h, w.grid_w, dims.D, dims.H, dims.F)
    rope = dit.dit_rope_table(w.grid_h, w.grid_w, w.Lt, dims.d)
    ws = dit.workspace(dd, dit.DIT_WS_BLOCK)
    x = inp["x"].to(x_dtype).cuda()
    return params, dev, inp, blk, dd, rope, ws, x


def _oracle_block(params, inp, w, dims, kind):
    P = {k: O.to64(v) for k, v in params.items()}
    x = O.to64(inp["x"])
    mod = O.to64(inp["mod"])
    ang = O.rope_table(O.image_positions(w.grid_h, w.grid_w, w.Lt), dims.d)
    if kind == "double":
        xt, xi = O.double_block(x[:, :w.Lt], x[:, w.Lt:], mod[:, :6], mod[:, 6:], P, ang, dims.H)
        return np.concatenate([xt, xi], axis=1)
    return O.single_block(x, mod, P, ang, dims.H)


BLOCK_CASES = [
    # D, H, F, B, Lt, grid_h, grid_w, kind, x dtype
    (256, 2, 512, 2, 24, 6, 8, "double", torch.float32),
    (256, 2, 512, 1, 40, 12, 20, "double", torch.bfloat16),
    (3072, 24, 12288, 1, 40, 12, 20, "double", torch.float32),
    (3072, 24, 12288, 2, 16, 8, 10, "double", torch.bfloat16),
    (256, 2, 512, 2, 24, 6, 8, "single", torch.float32),
    (3072, 24, 12288, 1, 40, 12, 20, "single", torch.float32),
    # image tokens only (no text stream)
    (256, 2, 512, 2, 0, 6, 8, "double", torch.float32),
    (256, 2, 512, 1, 0, 5, 8, "single", torch.bfloat16),
]


@pytest.mark.parametrize("D,H,F,B,Lt,gh,gw,kind,xdt", BLOCK_CASES)
def test_block_forward_small(dit, D, H, F, B, Lt, gh, gw, kind, xdt):
    _say(f"block {kind} D={D} B={B} Lt={Lt} grid={gh}x{gw} x={xdt}")
    dims = DI.Dims(D=D, H=H, F=F, n_double=1, n_single=0)
    w = DI.Workload("t", dims, B=B, grid_h=gh, grid_w=gw, Lt=Lt, dtype="bf16")
    params, dev, inp, blk, dd, rope, ws, x = _block_setup(dit, dims, w, kind, xdt)
    x_in = x.clone()
    dit.dit_block_forward(dd, blk, x, inp["mod"].cuda(), rope, ws)
    torch.cuda.synchronize()
    ref = _oracle_block(params, inp, w, dims, kind)
    got = x.double().cpu().numpy()
    err = parity_err_bf16_stored(got, ref) if xdt == torch.bfloat16 else parity_err(got, ref)
    _say(f"  x_out err {err:.3e}")
    assert err <= TOL_BF16
    if xdt == torch.float32:
        derr = parity_err(got - x_in.double().cpu().numpy(), ref - O.to64(inp["x"]))
        _say(f"  branch err {derr:.3e}")
        assert derr <= TOL_BRANCH


def test_block_forward_flux_1024(dit):
    """The full double block of the 1024px FLUX shape: 4096 image + 512 text tokens."""
    _say("block double full 1024px")
    w = DI.WORKLOADS["block_1024"]
    dims = w.dims
    params, dev, inp, blk, dd, rope, ws, x = _block_setup(dit, dims, w, "double", torch.bfloat16)
    dit.dit_block_forward(dd, blk, x, inp["mod"].cuda(), rope, ws)
    torch.cuda.synchronize()
    got = x.double().cpu().numpy()
    del dev, ws
    ref = _oracle_block(params, inp, w, dims, "double")
    err = parity_err_bf16_stored(got, ref)
    _say(f"  err {err:.3e}")
    assert err <= TOL_BF16



@pytest.mark.timeout(300)        # the fp64 oracle's share takes ~1 min on 8 cores
def test_block_forward_2048_cfg_sampled(dit):
    """The double block at the 2048px CFG-pair shape, in the launch configuration
    the benchmark times (fp32 residual stream, per-batch modulation): 2 x (16384
    image + 512 text) tokens, D 3072.  The GPU runs the whole block; the oracle
    computes every token's Q, K, V and the complete output of ~80 sampled rows
    per batch element, which is exactly what the full block gives at those rows."""
    w = DI.WORKLOADS["block_2048_cfg"]
    dims = w.dims
    _say(f"block double sampled 2048px B={w.B} L={w.L} D={dims.D}")
    params = DI.block_params(dims, "bf16", "double")
    dev = {n: (t.cuda() if n.endswith(".w") else t.float().cuda()) for n, t in params.items()}
    blk = dit.make_double_block(dev)
    dd = dit.dims_of(w.B, w.Lt, w.grid_h, w.grid_w, dims.D, dims.H, dims.F)
    rope = dit.dit_rope_table(w.grid_h, w.grid_w, w.Lt, dims.d)
    ws = dit.workspace(dd, dit.DIT_WS_BLOCK)
    x_in = DI.randn((w.B, w.L, dims.D), DI.SEED_ACT, 1.0, "f32")
    mod = DI.randn((w.B, 12, dims.D), DI.SEED_MOD, DI.MOD_STD, "f32")
    x = x_in.cuda()
    dit.dit_block_forward(dd, blk, x, mod.cuda(), rope, ws)
    torch.cuda.synchronize()
    rows = sampled_block_rows(w.Lt, w.L, 32, 2048)
    got = x[:, torch.from_numpy(rows).cuda()].double().cpu().numpy()
    del dev, ws, x
    P = {k: O.to64(v) for k, v in params.items()}
    x64 = O.to64(x_in)
    m64 = O.to64(mod)
    ang = O.rope_table(O.image_positions(w.grid_h, w.grid_w, w.Lt), dims.d)
    ref = O.double_block_rows(x64[:, :w.Lt], x64[:, w.Lt:], m64[:, :6], m64[:, 6:], P, ang,
                              dims.H, rows)
    err = parity_err(got, ref)
    derr = parity_err(got - x64[:, rows], ref - x64[:, rows])
    _say(f"  rows {len(rows)} x_out err {err:.3e} branch err {derr:.3e}")
    assert err <= TOL_BF16
    assert derr <= TOL_BRANCH


# ---------------------------------------------------------------- First-Block-Cache

def test_fbcache_rel_and_decision(dit):
    B, Lt, Li, D = 2, 16, 200, 256
    g = torch.Generator().manual_seed(5)
    xa = torch.randn((B, Lt + Li, D), generator=g)
    xb = torch.randn((B, Li, D), generator=g)
    r = (xa[:, Lt:] - xb)
    anchor = r + 0.1 * torch.randn((B, Li, D), generator=g)
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    stg = torch.empty((B, Li, D), device="cuda")
    rel_ref = O.fbcache_rel(r.double().numpy(), anchor.double().numpy())
    rels = []
    for tau in (0.0, rel_ref * 0.99, rel_ref * 1.01, math.inf):
        rel, skip = dit.fbcache_should_skip(xa.cuda(), xb.cuda(), anchor.cuda(), stg, Lt, tau,
                                            True, ws)
        rels.append(rel)
        assert abs(rel - rel_ref) <= 1e-6 * rel_ref
        assert skip == (rel_ref < tau)
    assert len(set(rels)) == 1            # deterministic reduction
    np.testing.assert_array_equal(stg.cpu().numpy(), r.numpy())
    rel, skip = dit.fbcache_should_skip(xa.cuda(), xb.cuda(), None, stg, Lt, math.inf, False, ws)
    assert rel == math.inf and not skip
    anchor[0, 3, 5] = float("nan")
    with pytest.raises(dit.DitError) as ei:
        dit.fbcache_should_skip(xa.cuda(), xb.cuda(), anchor.cuda(), stg, Lt, math.inf, True, ws)
    assert ei.value.status == dit.DIT_ERR_NONFINITE


# ---------------------------------------------------------------- modulation and full step

def _model(dit, dims, w):
    params = dict(DI.iter_params(dims, "bf16"))
    gm = dit.GPUModel(dims, w.B, w.Lt, w.grid_h, w.grid_w, params, guidance=w.guidance)
    P = {k: O.to64(v) for k, v in params.items()}
    return params, gm, P


SMALL = DI.Dims(D=256, H=2, F=512, n_double=2, n_single=2)


def test_modulation_vectors(dit):
    w = DI.Workload("m", SMALL, B=1, grid_h=8, grid_w=8, Lt=32, dtype="bf16", steps=5, shift=3.0)
    params, gm, P = _model(dit, SMALL, w)
    sig = O.sigmas(5, 3.0)[:-1]
    out = dit.dit_modulation(gm, list(sig)).double().cpu().numpy()
    c = O.time_embed(P, sig)
    names = [f"double{j}.{s}.mod" for j in range(2) for s in ("img", "txt")]
    names += [f"single{j}.mod" for j in range(2)] + ["final.mod"]
    ref = np.concatenate([O.linear(O.silu(c), P[n + ".w"], P[n + ".b"]) for n in names], axis=1)
    err = parity_err(out, ref)
    _say(f"modulation err {err:.3e}")
    assert err <= TOL_BF16


def _run_loop(dit, dims, w, threshold, enabled, teacher=True):
    params, gm, P = _model(dit, dims, w)
    sig = dit.dit_sigmas(w.steps, w.shift)
    mods = dit.dit_modulation(gm, sig[:-1])
    ws = dit.workspace(gm.model.dims, dit.DIT_WS_STEP)
    lat = DI.latents(w)
    txt = DI.text_tokens(w)
    lat_g = lat[0].clone().cuda()
    txt_g = txt.cuda()
    cache = dit.FBCache(w.B, w.Li, dims.D, threshold, enabled)
    ocache = O.FBCacheState(enabled, threshold)
    olat = O.to64(lat)
    errs, decisions = [], []
    for i in range(w.steps):
        x_in = lat_g.double().cpu().numpy()[None]
        rel, skip = dit.dit_denoise_step(gm, mods[i], txt_g, lat_g, sig[i], sig[i + 1], cache, ws)
        torch.cuda.synchronize()
        start = x_in if teacher else olat
        # decision replay inside the +-1e-3 band around the threshold
        ref_rel_probe = None
        olat_new, info = O.denoise_step(P, dims, w, start, O.to64(txt), i, np.array(sig),
                                        ocache if enabled else None,
                                        force_skip=skip if enabled else None)
        if enabled:
            if abs(info["rel"] - threshold) > 1e-3 and np.isfinite(info["rel"]):
                assert skip == (info["rel"] < threshold), (i, rel, info["rel"])
            if not np.isfinite(info["rel"]):
                assert not np.isfinite(rel)
        got = lat_g.double().cpu().numpy()[None]
        errs.append(parity_err(got - x_in, olat_new - start))   # the step's update
        decisions.append((rel, info["rel"], skip))
        olat = olat_new
    return errs, decisions, lat_g.double().cpu().numpy()[None], olat


@pytest.mark.parametrize("threshold,enabled", [(0.0, False), (0.12, True), (math.inf, True)])
def test_denoise_loop_teacher_forced(dit, threshold, enabled):
    w = DI.Workload("s", SMALL, B=1, grid_h=8, grid_w=8, Lt=32, dtype="bf16", steps=4, shift=3.0)
    errs, dec, _, _ = _run_loop(dit, SMALL, w, threshold, enabled)
    _say(f"loop tau={threshold} step-update errs {['%.2e' % e for e in errs]} decisions {dec}")
    assert max(errs) <= TOL_BF16


def test_denoise_loop_cfg_free_running(dit):
    w = DI.Workload("c", SMALL, B=2, grid_h=8, grid_w=8, Lt=32, dtype="bf16", steps=4, shift=3.0,
                    guidance=3.5)
    errs, dec, got, ref = _run_loop(dit, SMALL, w, 0.2, True, teacher=False)
    e2e = parity_err(got, ref)
    _say(f"cfg loop step errs {['%.2e' % e for e in errs]} end-to-end {e2e:.3e} decisions {dec}")
    assert e2e <= TOL_BF16


def test_smoke_entry(dit):
    import importlib
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    ge = importlib.import_module("__graft_entry__")
    ge.smoke()
