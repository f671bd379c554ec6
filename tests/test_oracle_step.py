"""Whole-step pins of the oracle on the tiny fp32 model (16x16 grid + 32 text tokens)."""
import math

import numpy as np
import pytest

import dit_inputs as DI
import oracle as O
from _helpers import params64

W = DI.WORKLOADS["tiny_fp32"]


@pytest.fixture(scope="module")
def model():
    P = params64(W.dims, W.dtype)
    lat = O.to64(DI.latents(W))
    txt = O.to64(DI.text_tokens(W))
    return P, lat, txt


def _zero_gates(P, D, blocks):
    P = {k: v.copy() for k, v in P.items()}
    for j in blocks:
        for s in ("img", "txt"):
            for g in (2, 5):   # gate1, gate2 chunks of the 6-vector modulation
                P[f"double{j}.{s}.mod.w"][g * D:(g + 1) * D] = 0.0
                P[f"double{j}.{s}.mod.b"][g * D:(g + 1) * D] = 0.0
    return P


def test_step_with_identity_blocks_is_embed_final_euler(model):
    P, lat, txt = model
    D = W.dims.D
    Pz = _zero_gates(P, D, range(W.dims.n_double))
    sg = O.sigmas(W.steps, W.shift)
    new, info = O.denoise_step(Pz, W.dims, W, lat, txt, 1, sg)
    c = O.time_embed(Pz, np.array([sg[1]]))
    mf = O.modulation_vectors(c, Pz["final.mod.w"], Pz["final.mod.b"], D)
    h = O.linear(lat, Pz["img_in.w"], Pz["img_in.b"])
    v = O.final_layer(h, mf[:, 0:1], mf[:, 1:2], Pz["final.out.w"], Pz["final.out.b"])
    np.testing.assert_array_equal(info["v"], v)
    np.testing.assert_array_equal(new, O.euler_update(lat, v, sg[1], sg[2]))


def _loop(P, lat, txt, threshold, enabled=True):
    sg = O.sigmas(W.steps, W.shift)
    cache = O.FBCacheState(enabled, threshold)
    rels, skips, x = [], [], lat
    for i in range(W.steps):
        x, info = O.denoise_step(P, W.dims, W, x, txt, i, sg, cache)
        rels.append(info["rel"]); skips.append(info["skip"])
    return x, rels, skips


def test_fbcache_threshold_zero_never_skips_and_matches_disabled(model):
    P, lat, txt = model
    x0, rels, skips = _loop(P, lat, txt, 0.0)
    assert not any(skips) and rels[0] == math.inf and all(np.isfinite(rels[1:]))
    x1, _, _ = _loop(P, lat, txt, 0.0, enabled=False)
    np.testing.assert_array_equal(x0, x1)


def test_fbcache_threshold_inf_skips_every_step_after_first(model):
    P, lat, txt = model
    _, rels, skips = _loop(P, lat, txt, math.inf)
    assert skips == [False] + [True] * (W.steps - 1)


def _policy_loop(P, lat, txt, steps, warmup, max_skips):
    import dataclasses
    w = dataclasses.replace(W, steps=steps)
    sg = O.sigmas(steps, w.shift)
    cache = O.FBCacheState(True, math.inf, warmup_steps=warmup, max_skips=max_skips)
    skips, x = [], lat
    for i in range(steps):
        x, info = O.denoise_step(P, w.dims, w, x, txt, i, sg, cache)
        skips.append(info["skip"])
    return skips, cache


@pytest.mark.parametrize("warmup,max_skips,want", [
    # tau = +inf: every step with an anchor passes the rel test, so the pattern is the
    # policy's: step 0 has no anchor; warm-up steps compute; at most max_skips in a row
    (3, 2, "FFFSSFSS"),
    (0, 1, "FSFSFSFS"),
    (2, 0, "FFSSSSSS"),
])
def test_fbcache_policy_pattern(model, warmup, max_skips, want):
    P, lat, txt = model
    skips, cache = _policy_loop(P, lat, txt, 8, warmup, max_skips)
    assert "".join("S" if s else "F" for s in skips) == want
    assert cache.steps_done == 8 and cache.skip_run == len(want) - len(want.rstrip("S"))


def test_fbcache_identity_tail_skip_equals_full(model):
    # blocks after the first are identity: the cached residual is 0 and the
    # skip path must give exactly the full path's latents
    P, lat, txt = model
    Pz = _zero_gates(P, W.dims.D, range(1, W.dims.n_double))
    xs, _, skips = _loop(Pz, lat, txt, math.inf)
    xf, _, _ = _loop(Pz, lat, txt, 0.0)
    assert all(skips[1:])
    np.testing.assert_array_equal(xs, xf)


def test_fbcache_rel_is_direct_recomputation(model):
    # rel of step 1 recomputed from the two first-block residuals with a plain loop
    P, lat, txt = model
    sg = O.sigmas(W.steps, W.shift)
    D = W.dims.D
    res = []
    x = lat
    for i in range(2):
        c = O.time_embed(P, np.array([sg[i]]))
        ang = O.rope_table(O.image_positions(W.grid_h, W.grid_w, W.Lt), D // W.dims.H)
        h = O.linear(x, P["img_in.w"], P["img_in.b"])
        mi = O.modulation_vectors(c, P["double0.img.mod.w"], P["double0.img.mod.b"], D)
        mt = O.modulation_vectors(c, P["double0.txt.mod.w"], P["double0.txt.mod.b"], D)
        bp = {k[8:]: v for k, v in P.items() if k.startswith("double0.")}
        _, hi = O.double_block(txt, h, mi, mt, bp, ang, W.dims.H)
        res.append((hi - h).ravel().tolist())
        x, _ = O.denoise_step(P, W.dims, W, x, txt, i, sg)
    num = sum(abs(a - b) for a, b in zip(res[1], res[0]))
    den = sum(abs(b) for b in res[0])
    cache = O.FBCacheState(True, 0.0)
    y = lat
    for i in range(2):
        y, info = O.denoise_step(P, W.dims, W, y, txt, i, sg, cache)
    assert abs(info["rel"] - num / den) <= 1e-12 * (num / den)


def test_fbcache_repeated_step_has_zero_rel(model):
    P, lat, txt = model
    sg = O.sigmas(W.steps, W.shift)
    cache = O.FBCacheState(True, 1e-9)
    O.denoise_step(P, W.dims, W, lat, txt, 0, sg, cache)
    _, info = O.denoise_step(P, W.dims, W, lat, txt, 0, sg, cache)
    assert info["rel"] == 0.0 and info["skip"]


def test_cfg_identical_prompts_equals_single(model):
    P, lat, txt = model
    import dataclasses
    w2 = dataclasses.replace(W, B=2, guidance=3.5)
    sg = O.sigmas(W.steps, W.shift)
    a, _ = O.denoise_step(P, W.dims, w2, lat, np.concatenate([txt, txt]), 0, sg)
    b, _ = O.denoise_step(P, W.dims, W, lat, txt, 0, sg)
    np.testing.assert_allclose(a, b, atol=1e-12)
