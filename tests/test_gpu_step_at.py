"""dit_denoise_step_at (a step addressed by its index in the sigma table, computing
its own modulation row) against dit_denoise_step on the row dit_modulation
precomputes: the same kernels on the same inputs, so every step's latents, rel and
skip decision must be equal bit for bit, with and without the First-Block-Cache."""
import dataclasses
import math
import sys

import pytest
import torch

import dit_inputs as DI

pytestmark = pytest.mark.gpu

SMALL = DI.Dims(D=256, H=2, F=512, n_double=2, n_single=2)


@pytest.fixture(scope="module")
def dit():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from image_generation_amd import dit as D
    return D


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _setup(dit, kind, steps, B=1, guidance=0.0):
    if kind == "f32":
        w = dataclasses.replace(DI.WORKLOADS["tiny_fp32"], steps=steps)
        params = dict(DI.iter_params(w.dims, "f32"))
        gm = dit.GPUModel(w.dims, w.B, w.Lt, w.grid_h, w.grid_w, params, dtype=dit.DIT_F32)
    else:
        w = DI.Workload("g", SMALL, B=B, grid_h=8, grid_w=8, Lt=32, dtype=kind, steps=steps,
                        shift=3.0, guidance=guidance)
        params = dict(DI.iter_params(SMALL, "bf16"))
        gm = dit.GPUModel(SMALL, w.B, w.Lt, w.grid_h, w.grid_w, params, guidance=w.guidance,
                          dtype=dit.DIT_FP8 if kind == "fp8" else dit.DIT_BF16)
    sig = dit.dit_sigmas(w.steps, w.shift)
    txt = DI.text_tokens(w)
    txt = (txt.float() if kind == "f32" else txt.to(torch.bfloat16)).cuda()
    lat0 = DI.latents(w)[0].clone()
    return w, gm, sig, txt, lat0


@pytest.mark.parametrize("kind,B,guidance", [("f32", 1, 0.0), ("bf16", 2, 3.5), ("fp8", 1, 0.0)])
@pytest.mark.parametrize("enabled,tau,warmup", [(False, 0.0, 0), (True, math.inf, 2)])
def test_step_at_equals_step_on_the_precomputed_row(dit, kind, B, guidance, enabled, tau, warmup):
    _say(f"[step_at] {kind} B={B} cache={enabled} tau={tau} warmup={warmup}")
    w, gm, sig, txt, lat0 = _setup(dit, kind, 4, B, guidance)
    mods = dit.dit_modulation(gm, sig[:-1])
    ws = dit.workspace(gm.model.dims, dit.DIT_WS_STEP)
    ws_at = dit.step_at_workspace(gm)
    assert ws_at.numel() > ws.numel()
    D = gm.model.dims.D
    c_ref = dit.FBCache(w.B, w.Li, D, tau, enabled, warmup_steps=warmup)
    c_at = dit.FBCache(w.B, w.Li, D, tau, enabled, warmup_steps=warmup)
    lat_ref, lat_at = lat0.clone().cuda(), lat0.clone().cuda()
    skips = []
    for i in range(w.steps):
        r_ref = dit.dit_denoise_step(gm, mods[i], txt, lat_ref, sig[i], sig[i + 1], c_ref, ws)
        r_at = dit.dit_denoise_step_at(gm, txt, lat_at, i, sig, c_at, ws_at)
        torch.cuda.synchronize()
        assert torch.equal(lat_ref, lat_at), f"step {i}: latents differ"
        assert r_ref[1] == r_at[1], f"step {i}: skip decision differs"
        assert (r_ref[0] == r_at[0]) or (math.isinf(r_ref[0]) and math.isinf(r_at[0])), i
        skips.append(r_at[1])
    if enabled:
        # warm-up 2 then an infinite threshold: steps 2 and 3 are cached ones
        assert skips == [False, False, True, True]
    assert torch.isfinite(lat_at).all()


def test_step_at_rejects_a_step_outside_the_table(dit):
    w, gm, sig, txt, lat0 = _setup(dit, "bf16", 3)
    ws_at = dit.step_at_workspace(gm)
    lat = lat0.clone().cuda()
    for bad in (-1, 3):
        with pytest.raises(dit.DitError) as e:
            dit.dit_denoise_step_at(gm, txt, lat, bad, sig, None, ws_at)
        assert e.value.status == dit.DIT_ERR_INVALID_ARG
    with pytest.raises(dit.DitError) as e:
        dit.dit_denoise_step_at(gm, txt, lat, 0, sig, None, ws_at[:-256])
    assert e.value.status == dit.DIT_ERR_WORKSPACE
    assert torch.equal(lat.cpu(), lat0)
