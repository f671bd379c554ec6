"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names the mistake it is meant to catch.  CPU only.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from oracle.numerics import round_bf16, round_fp16, round_e4m3, quantize_rows_e4m3, e4m3_tie_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append([float(t) for t in line.split()])
    return rows


# ---------------------------------------------------------------- schedule

def test_sigmas_golden_shift3():
    want = np.array(_golden_rows("sigmas_shift3_n4.txt")[0])
    np.testing.assert_allclose(O.sigmas(4, 3.0), want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("n,s", [(4, 1.0), (28, 3.0), (50, 3.0), (7, 0.5)])
def test_sigmas_endpoints_monotone(n, s):
    sg = O.sigmas(n, s)
    assert sg[0] == 1.0 and sg[-1] == 0.0
    assert np.all(np.diff(sg) < 0)


def test_sigmas_shift1_is_linear():
    np.testing.assert_allclose(O.sigmas(10, 1.0), np.linspace(1, 0, 11), atol=1e-15)


def test_euler_constant_velocity_total_displacement():
    # sum of d(sigma) is exactly -1: a wrong sign or a dropped step shows here
    sg = O.sigmas(28, 3.0)
    x = np.array([0.3, -1.2])
    u = np.array([2.0, 0.5])
    for i in range(28):
        x = O.euler_update(x, u, sg[i], sg[i + 1])
    np.testing.assert_allclose(x, np.array([0.3, -1.2]) - u, atol=1e-13)


def test_euler_lands_on_target_for_exact_velocity():
    # v(x, sigma) = (x - x*) / sigma is the exact rectified-flow velocity of a
    # point mass at x*; Euler then hits x* at sigma = 0 for any schedule
    rng = np.random.default_rng(0)
    xs = rng.standard_normal(5)
    x = rng.standard_normal(5)
    sg = O.sigmas(13, 2.3)
    for i in range(13):
        x = O.euler_update(x, (x - xs) / sg[i], sg[i], sg[i + 1])
    np.testing.assert_allclose(x, xs, atol=1e-12)


def test_cfg_combine_cases():
    vp, vn = np.array([1.0, 2.0]), np.array([-1.0, 0.5])
    np.testing.assert_array_equal(O.cfg_combine(vp, vn, 1.0), vp)
    np.testing.assert_array_equal(O.cfg_combine(vp, vn, 0.0), vn)
    np.testing.assert_array_equal(O.cfg_combine(vp, vp, 3.5), vp)


# ---------------------------------------------------------------- embeddings

def test_timestep_sinusoid_t0():
    e = O.timestep_sinusoid(0.0)
    assert e.shape == (1, 256)
    np.testing.assert_array_equal(e[0, :128], 1.0)
    np.testing.assert_array_equal(e[0, 128:], 0.0)


def test_timestep_sinusoid_frequencies():
    # k = 0 turns once per unit of 1000 t; k = 64 at 10000^-0.5 = 1/100 of it
    t = math.pi / 2000.0          # 1000 t = pi/2
    e = O.timestep_sinusoid(t)[0]
    assert abs(e[0]) < 1e-15 and abs(e[128] - 1.0) < 1e-15
    np.testing.assert_allclose(e[64], math.cos(math.pi / 200.0), atol=1e-15)
    np.testing.assert_allclose(e[:128] ** 2 + e[128:] ** 2, 1.0, atol=1e-14)


# ---------------------------------------------------------------- LN / GELU

def test_layer_norm_vs_torch_and_moments():
    rng = np.random.default_rng(1)
    u = rng.standard_normal((7, 96)) * 3 + 1.5
    ln = O.layer_norm(u)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(u), (96,), eps=1e-6).numpy()
    np.testing.assert_allclose(ln, ref, atol=1e-12)
    np.testing.assert_allclose(ln.mean(-1), 0, atol=1e-13)
    var = u.var(-1)
    np.testing.assert_allclose(ln.var(-1), var / (var + 1e-6), rtol=1e-12)


def test_modulate_identity_and_affine():
    rng = np.random.default_rng(2)
    u = rng.standard_normal((3, 5, 64))
    z = np.zeros((1, 1, 64))
    np.testing.assert_array_equal(O.modulate(u, z, z), O.layer_norm(u))
    sh = rng.standard_normal((1, 1, 64))
    np.testing.assert_array_equal(O.modulate(u, sh, z - 1.0), np.broadcast_to(sh, u.shape))


def test_gelu_tanh_vs_torch_and_erf():
    x = np.linspace(-12, 12, 4001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_tanh(x), ref, atol=1e-14)
    exact = 0.5 * x * (1 + np.vectorize(math.erf)(x / math.sqrt(2)))
    assert np.max(np.abs(O.gelu_tanh(x) - exact)) < 1e-3   # tanh form is within ~5e-4
    assert O.gelu_tanh(np.array(0.0)) == 0.0
    np.testing.assert_allclose(O.gelu_tanh(np.array([30.0, -30.0])), [30.0, 0.0], atol=1e-12)


def test_silu_vs_torch():
    x = np.linspace(-20, 20, 801)
    np.testing.assert_allclose(O.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(),
                               atol=1e-14)


# ---------------------------------------------------------------- linear

def test_linear_vs_triple_loop():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 6))
    w = rng.standard_normal((5, 6))
    b = rng.standard_normal(5)
    y = O.linear(x, w, b)
    for i in range(4):
        for n in range(5):
            assert abs(y[i, n] - (sum(x[i, k] * w[n, k] for k in range(6)) + b[n])) < 1e-12


def test_linear_one_hot_weight_selects_column():
    x = np.arange(12.0).reshape(3, 4)
    w = np.zeros((2, 4))
    w[0, 2] = 1.0
    w[1, 0] = 1.0
    np.testing.assert_array_equal(O.linear(x, w, np.zeros(2)), x[:, [2, 0]])


# ---------------------------------------------------------------- RoPE

def _complex_rope(x, ang):
    z = x[..., 0::2] + 1j * x[..., 1::2]
    z = z * np.exp(1j * ang)
    out = np.empty_like(x)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def test_rope_matches_complex_rotation_and_keeps_pair_norms():
    rng = np.random.default_rng(4)
    pos = O.image_positions(5, 7, 3)
    ang = O.rope_table(pos, 64)
    x = rng.standard_normal((2, 3, pos.shape[0], 64))
    y = O.apply_rope(x, ang)
    np.testing.assert_allclose(y, _complex_rope(x, ang), atol=1e-13)
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    # text tokens sit at (0, 0): identity
    np.testing.assert_array_equal(y[:, :, :3], x[:, :, :3])


def test_rope_relative_position_per_axis():
    # <R(q, p + delta), R(k, p' + delta)> == <R(q, p), R(k, p')> for a shift
    # along either axis; a wrong frequency or pairing breaks it
    rng = np.random.default_rng(5)
    d = 128
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    for delta in ([3, 0], [0, 5], [2, 7]):
        p = np.array([[1.0, 4.0], [6.0, 2.0]])
        p2 = p + np.array(delta, dtype=float)
        a = O.rope_table(p, d)
        a2 = O.rope_table(p2, d)
        s1 = O.apply_rope(q[None], a[0:1])[0] @ O.apply_rope(k[None], a[1:2])[0]
        s2 = O.apply_rope(q[None], a2[0:1])[0] @ O.apply_rope(k[None], a2[1:2])[0]
        assert abs(s1 - s2) < 1e-10


def test_rope_axis_split():
    # moving along columns leaves the row pairs (p < d/4) untouched and vice versa
    d = 64
    a_row = O.rope_table(np.array([[3.0, 0.0]]), d)[0]
    a_col = O.rope_table(np.array([[0.0, 3.0]]), d)[0]
    assert np.all(a_row[:d // 4] != 0) and np.all(a_col[d // 4:] != 0)
    assert np.all(a_col[:d // 4] == 0)
    assert np.all(a_row[d // 4:] == 0)
    # pair j = 0 of each axis turns by exactly the position
    assert a_row[0] == 3.0 and a_col[d // 4] == 3.0


# ---------------------------------------------------------------- attention

def test_attention_rows_are_a_distribution():
    # with V = identity the output row is the softmax row itself
    rng = np.random.default_rng(6)
    L = 40
    q = rng.standard_normal((1, 2, L, 64)) * 2
    k = rng.standard_normal((1, 2, L, 64)) * 2
    v = np.broadcast_to(np.eye(L, 64), (1, 2, L, 64)).copy()
    p = O.attention(q, k, v)[..., :L]
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    assert np.all(p > 0)


def test_attention_identical_keys_gives_mean_of_v():
    rng = np.random.default_rng(7)
    L = 33
    q = rng.standard_normal((2, 2, L, 64))
    k = np.broadcast_to(rng.standard_normal((1, 1, 1, 64)), (2, 2, L, 64)).copy()
    v = rng.standard_normal((2, 2, L, 64))
    out = O.attention(q, k, v)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=2, keepdims=True), out.shape),
                               atol=1e-13)
    vv = np.broadcast_to(v[:, :, :1], v.shape).copy()
    np.testing.assert_allclose(O.attention(q, k, vv), vv, atol=1e-13)


def test_attention_dominant_key():
    rng = np.random.default_rng(8)
    L, d = 17, 64
    k = rng.standard_normal((1, 1, L, d))
    v = rng.standard_normal((1, 1, L, d))
    q = 200.0 * k[:, :, 5:6].repeat(L, axis=2)
    out = O.attention(q, k, v)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(v[0, 0, 5], (L, d)), atol=1e-8)


@pytest.mark.parametrize("B,H,L,d", [(1, 1, 7, 64), (2, 2, 33, 64), (1, 1, 9, 128)])
def test_attention_vs_naive_triple_loop(B, H, L, d):
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    np.testing.assert_allclose(O.attention(q, k, v), O.attention_naive(q, k, v), rtol=1e-9,
                               atol=1e-12)


def test_attention_vs_torch_sdpa():
    rng = np.random.default_rng(10)
    q, k, v = (rng.standard_normal((2, 3, 50, 64)) for _ in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(O.attention(q, k, v), ref, atol=1e-12)


# ---------------------------------------------------------------- blocks

def _tiny_double(rng, D=64, H=2, F=256, Lt=3, gh=2, gw=3, B=2):
    P = {}
    for s in ("img", "txt"):
        for name, shp in (("qkv", (3 * D, D)), ("proj", (D, D)), ("mlp1", (F, D)), ("mlp2", (D, F))):
            P[f"{s}.{name}.w"] = rng.standard_normal(shp) * 0.05
            P[f"{s}.{name}.b"] = rng.standard_normal(shp[0]) * 0.05
    x_txt = rng.standard_normal((B, Lt, D))
    x_img = rng.standard_normal((B, gh * gw, D))
    m_img = rng.standard_normal((B, 6, D)) * 0.1
    m_txt = rng.standard_normal((B, 6, D)) * 0.1
    ang = O.rope_table(O.image_positions(gh, gw, Lt), D // H)
    return P, x_txt, x_img, m_img, m_txt, ang, H


def test_double_block_zero_gates_is_identity():
    rng = np.random.default_rng(11)
    P, xt, xi, mi, mt, ang, H = _tiny_double(rng)
    for m in (mi, mt):
        m[:, 2] = 0.0
        m[:, 5] = 0.0
    ot, oi = O.double_block(xt, xi, mi, mt, P, ang, H)
    np.testing.assert_array_equal(ot, xt)
    np.testing.assert_array_equal(oi, xi)


def test_double_block_zero_value_weights():
    # W_v = b_v = 0 and mlp gate 0: the attention branch is exactly gate1 * b_o
    rng = np.random.default_rng(12)
    P, xt, xi, mi, mt, ang, H = _tiny_double(rng)
    D = xt.shape[-1]
    for s in ("img", "txt"):
        P[f"{s}.qkv.w"][2 * D:] = 0.0
        P[f"{s}.qkv.b"][2 * D:] = 0.0
    for m in (mi, mt):
        m[:, 5] = 0.0
    ot, oi = O.double_block(xt, xi, mi, mt, P, ang, H)
    np.testing.assert_allclose(oi, xi + mi[:, 2:3] * P["img.proj.b"], atol=1e-14)
    np.testing.assert_allclose(ot, xt + mt[:, 2:3] * P["txt.proj.b"], atol=1e-14)


def test_double_block_stream_isolation():
    # text gates 0: text rows unchanged, image rows still move
    rng = np.random.default_rng(13)
    P, xt, xi, mi, mt, ang, H = _tiny_double(rng)
    mt[:, 2] = 0.0
    mt[:, 5] = 0.0
    ot, oi = O.double_block(xt, xi, mi, mt, P, ang, H)
    np.testing.assert_array_equal(ot, xt)
    assert np.max(np.abs(oi - xi)) > 1e-3


@pytest.mark.parametrize("fp8,mx4", [(False, False), (True, False), (False, True)])
def test_double_block_rows_equals_full_block(fp8, mx4):
    # the row-sampled block is the full block restricted to the sampled rows (text,
    # image and boundary rows, out of order); fp8 included (its scales span heads)
    # and MXFP4 (its blocks lie along each row)
    rng = np.random.default_rng(15)
    P, xt, xi, mi, mt, ang, H = _tiny_double(rng, D=64, H=2, F=256, Lt=5, gh=4, gw=4, B=2)
    ot, oi = O.double_block(xt, xi, mi, mt, P, ang, H, fp8=fp8, mx4=mx4)
    full = np.concatenate([ot, oi], axis=1)
    rows = np.array([20, 0, 4, 5, 13, 2])
    got = O.double_block_rows(xt, xi, mi, mt, P, ang, H, rows, fp8=fp8, mx4=mx4)
    np.testing.assert_allclose(got, full[:, rows], rtol=0, atol=1e-12)


@pytest.mark.parametrize("attn8", [False, True])
def test_mx4_blocks_route_every_linear_through_mxfp4(monkeypatch, attn8):
    # every linear of an MXFP4 block (8 in a double block, 2 in a single one) goes
    # through the W4A4 linear, on an input already rounded to bf16, with the
    # expected (K, N); no full-precision or fp8 linear is left in the block; the
    # attention is the e4m3 one exactly when asked for, on Q, K held in bf16 and V
    # in fp16
    import oracle.dit_oracle as DO
    calls = []
    attn_calls = []
    real = DO.linear_mxfp4
    real_a, real_a8 = DO.attention, DO.attention_fp8

    def rec_a(q, k, v, *a, **kw):
        attn_calls.append("bf16")
        return real_a(q, k, v, *a, **kw)

    def rec_a8(q, k, v, *a, **kw):
        assert np.array_equal(O.round_bf16(q), q) and np.array_equal(O.round_bf16(k), k)
        assert np.array_equal(O.round_fp16(v), v)
        attn_calls.append("fp8")
        return real_a8(q, k, v, *a, **kw)

    monkeypatch.setattr(DO, "attention", rec_a)
    monkeypatch.setattr(DO, "attention_fp8", rec_a8)

    def rec(x, w, b):
        assert np.array_equal(O.round_bf16(x), x), "MXFP4 input not bf16-held"
        calls.append((w.shape[1], w.shape[0]))
        return real(x, w, b)

    def forbidden(*a, **k):
        raise AssertionError("a block linear bypassed MXFP4")

    monkeypatch.setattr(DO, "linear_mxfp4", rec)
    monkeypatch.setattr(DO, "linear", forbidden)
    monkeypatch.setattr(DO, "linear_fp8", forbidden)
    rng = np.random.default_rng(17)
    D, F = 64, 256
    P, xt, xi, mi, mt, ang, H = _tiny_double(rng, D=D, H=2, F=F)
    DO.double_block(xt, xi, mi, mt, P, ang, H, mx4=True, attn8=attn8)
    assert sorted(calls) == sorted([(D, 3 * D), (D, D), (D, F), (F, D)] * 2)
    assert attn_calls == ["fp8" if attn8 else "bf16"]
    calls.clear()
    attn_calls.clear()
    Ps = {"lin1.w": rng.standard_normal((3 * D + F, D)) * 0.05, "lin1.b": np.zeros(3 * D + F),
          "lin2.w": rng.standard_normal((D, D + F)) * 0.05, "lin2.b": np.zeros(D)}
    x = np.concatenate([xt, xi], axis=1)
    DO.single_block(x, mi[:, :3], Ps, ang, H, mx4=True, attn8=attn8)
    assert calls == [(D, 3 * D + F), (D + F, D)]
    assert attn_calls == ["fp8" if attn8 else "bf16"]


def test_mx4_double_block_zero_weights_keeps_biases_exact():
    # all weights zero: every MXFP4 linear returns its bias exactly (zero blocks
    # quantise to zero), so the block adds gate1 * b_proj + gate2 * b_mlp2
    rng = np.random.default_rng(18)
    P, xt, xi, mi, mt, ang, H = _tiny_double(rng)
    for k in P:
        if k.endswith(".w"):
            P[k] = np.zeros_like(P[k])
    ot, oi = O.double_block(xt, xi, mi, mt, P, ang, H, mx4=True)
    for got, x, m, s in ((oi, xi, mi, "img"), (ot, xt, mt, "txt")):
        ref = x + m[:, 2:3] * P[f"{s}.proj.b"]
        ref = ref + m[:, 5:6] * P[f"{s}.mlp2.b"]
        np.testing.assert_array_equal(got, ref)


def test_double_block_brute_force_small():
    # the joint attention written out token by token, no reshapes, no rope
    # helpers: catches a transposed head split or a swapped stream order
    rng = np.random.default_rng(14)
    D, H, F, Lt, gh, gw, B = 8, 2, 16, 2, 1, 3, 1
    P, xt, xi, mi, mt, ang, H = _tiny_double(rng, D, H, F, Lt, gh, gw, B)
    ot, oi = O.double_block(xt, xi, mi, mt, P, ang, H)
    d = D // H
    L = Lt + gh * gw
    x = np.concatenate([xt, xi], axis=1)[0]
    mods = [mt[0]] * Lt + [mi[0]] * (gh * gw)
    names = ["txt"] * Lt + ["img"] * (gh * gw)
    pos = [(0, 0)] * Lt + [(r, c) for r in range(gh) for c in range(gw)]

    def ln(u):
        mu = sum(u) / len(u)
        var = sum((t - mu) ** 2 for t in u) / len(u)
        return [(t - mu) / math.sqrt(var + 1e-6) for t in u]

    def lin(u, w, b):
        return [sum(u[k] * w[n][k] for k in range(len(u))) + b[n] for n in range(len(b))]

    def rot(vec, p):
        out = list(vec)
        for pr in range(d // 2):
            ax = 0 if pr < d // 4 else 1
            j = pr % (d // 4)
            th = p[ax] * 10000.0 ** (-j / (d // 4))
            a, b = vec[2 * pr], vec[2 * pr + 1]
            out[2 * pr] = a * math.cos(th) - b * math.sin(th)
            out[2 * pr + 1] = a * math.sin(th) + b * math.cos(th)
        return out

    qs, ks, vs = [], [], []
    for t in range(L):
        m = mods[t]
        u = [ln(list(x[t]))[c] * (1 + m[1][c]) + m[0][c] for c in range(D)]
        h = lin(u, P[f"{names[t]}.qkv.w"], P[f"{names[t]}.qkv.b"])
        qs.append(h[:D]); ks.append(h[D:2 * D]); vs.append(h[2 * D:])
    att = [[0.0] * D for _ in range(L)]
    for hh in range(H):
        sl = slice(hh * d, (hh + 1) * d)
        qh = [rot(qs[t][sl], pos[t]) for t in range(L)]
        kh = [rot(ks[t][sl], pos[t]) for t in range(L)]
        for t in range(L):
            s = [sum(a * b for a, b in zip(qh[t], kh[u])) / math.sqrt(d) for u in range(L)]
            mx = max(s)
            e = [math.exp(z - mx) for z in s]
            z = sum(e)
            for c in range(d):
                att[t][hh * d + c] = sum(e[u] * vs[u][sl][c] for u in range(L)) / z
    gelu = lambda z: 0.5 * z * (1 + math.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))
    out = []
    for t in range(L):
        m, nm = mods[t], names[t]
        y = lin(att[t], P[f"{nm}.proj.w"], P[f"{nm}.proj.b"])
        xr = [x[t][c] + m[2][c] * y[c] for c in range(D)]
        u = [ln(xr)[c] * (1 + m[4][c]) + m[3][c] for c in range(D)]
        hid = [gelu(z) for z in lin(u, P[f"{nm}.mlp1.w"], P[f"{nm}.mlp1.b"])]
        y2 = lin(hid, P[f"{nm}.mlp2.w"], P[f"{nm}.mlp2.b"])
        out.append([xr[c] + m[5][c] * y2[c] for c in range(D)])
    out = np.array(out)
    np.testing.assert_allclose(ot[0], out[:Lt], atol=1e-12)
    np.testing.assert_allclose(oi[0], out[Lt:], atol=1e-12)


def test_single_block_zero_gate_and_wiring():
    rng = np.random.default_rng(15)
    D, H, F, L, B = 32, 2, 64, 7, 2
    P = {"lin1.w": rng.standard_normal((3 * D + F, D)) * 0.1, "lin1.b": rng.standard_normal(3 * D + F) * 0.1,
         "lin2.w": rng.standard_normal((D, D + F)) * 0.1, "lin2.b": rng.standard_normal(D) * 0.1}
    x = rng.standard_normal((B, L, D))
    mod = rng.standard_normal((B, 3, D)) * 0.1
    ang = O.rope_table(O.image_positions(2, 3, 1), D // H)
    m0 = mod.copy(); m0[:, 2] = 0
    np.testing.assert_array_equal(O.single_block(x, m0, P, ang, H), x)
    # zero the attention half of lin2: the block reduces to a gated GELU MLP
    P2 = dict(P); P2["lin2.w"] = P["lin2.w"].copy(); P2["lin2.w"][:, :D] = 0
    u = O.modulate(x, mod[:, 0:1], mod[:, 1:2])
    mlp = O.gelu_tanh(u @ P["lin1.w"][3 * D:].T + P["lin1.b"][3 * D:]) @ P["lin2.w"][:, D:].T
    np.testing.assert_allclose(O.single_block(x, mod, P2, ang, H),
                               x + mod[:, 2:3] * (mlp + P["lin2.b"]), atol=1e-13)



def _single_block_by_hand(x, mod, P, H, pos, swap_qk=False):
    """The single-stream block written out token by token (R10): lin1's output
    columns are q | k | v | MLP-in, RoPE turns q and k only, lin2 reads
    [attention out, GELU(MLP-in)].  swap_qk plants the q/k column mix-up."""
    L, D = x.shape
    d = D // H

    def ln(u):
        mu = sum(u) / len(u)
        var = sum((t - mu) ** 2 for t in u) / len(u)
        return [(t - mu) / math.sqrt(var + 1e-6) for t in u]

    def lin(u, w, b):
        return [sum(u[k] * w[n][k] for k in range(len(u))) + b[n] for n in range(len(b))]

    def rot(vec, p):
        out = list(vec)
        for pr in range(d // 2):
            ax = 0 if pr < d // 4 else 1
            j = pr % (d // 4)
            th = p[ax] * 10000.0 ** (-j / (d // 4))
            a, b = vec[2 * pr], vec[2 * pr + 1]
            out[2 * pr] = a * math.cos(th) - b * math.sin(th)
            out[2 * pr + 1] = a * math.sin(th) + b * math.cos(th)
        return out

    gelu = lambda z: 0.5 * z * (1 + math.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))
    qs, ks, vs, ms = [], [], [], []
    for t in range(L):
        u = [ln(list(x[t]))[c] * (1 + mod[1][c]) + mod[0][c] for c in range(D)]
        h = lin(u, P["lin1.w"], P["lin1.b"])
        q, k = (h[D:2 * D], h[:D]) if swap_qk else (h[:D], h[D:2 * D])
        qs.append(q); ks.append(k); vs.append(h[2 * D:3 * D]); ms.append(h[3 * D:])
    att = [[0.0] * D for _ in range(L)]
    for hh in range(H):
        sl = slice(hh * d, (hh + 1) * d)
        qh = [rot(qs[t][sl], pos[t]) for t in range(L)]
        kh = [rot(ks[t][sl], pos[t]) for t in range(L)]
        for t in range(L):
            s = [sum(a * b for a, b in zip(qh[t], kh[u])) / math.sqrt(d) for u in range(L)]
            mx = max(s)
            e = [math.exp(z - mx) for z in s]
            z = sum(e)
            for c in range(d):
                att[t][hh * d + c] = sum(e[u] * vs[u][sl][c] for u in range(L)) / z
    out = []
    for t in range(L):
        y = lin(att[t] + [gelu(z) for z in ms[t]], P["lin2.w"], P["lin2.b"])
        out.append([x[t][c] + mod[2][c] * y[c] for c in range(D)])
    return np.array(out)


def test_single_block_brute_force_small():
    # the single-stream block's attention half written out by hand: catches a
    # q / k / v column mix-up in linear1, RoPE on v (or not on k), a wrong head
    # split or a swapped [attention, GELU] order in linear2's input
    rng = np.random.default_rng(16)
    D, H, F, Lt, gh, gw = 8, 2, 16, 2, 2, 2
    L = Lt + gh * gw
    P = {"lin1.w": rng.standard_normal((3 * D + F, D)) * 0.4,
         "lin1.b": rng.standard_normal(3 * D + F) * 0.1,
         "lin2.w": rng.standard_normal((D, D + F)) * 0.3,
         "lin2.b": rng.standard_normal(D) * 0.1}
    x = rng.standard_normal((1, L, D))
    mod = rng.standard_normal((1, 3, D)) * 0.3
    pos = [(0, 0)] * Lt + [(r, c) for r in range(gh) for c in range(gw)]
    ang = O.rope_table(O.image_positions(gh, gw, Lt), D // H)
    got = O.single_block(x, mod, P, ang, H)[0]
    ref = _single_block_by_hand(x[0], mod[0], P, H, pos)
    np.testing.assert_allclose(got, ref, atol=1e-12)
    # the hand version is sensitive to the planted q / k swap
    bad = _single_block_by_hand(x[0], mod[0], P, H, pos, swap_qk=True)
    assert np.max(np.abs(bad - ref)) > 1e-3


def test_time_embed_hand_derived():
    # one-hot rows pick single sinusoid entries, so the timestep MLP reduces to
    # closed forms: catches [sin, cos] order, a wrong frequency exponent or time
    # scale, and SiLU misplaced (after the second linear, or missing)
    D = 4
    w1 = np.zeros((D, 256)); b1 = np.array([0.5, 0.0, -0.25, 0.1])
    w1[0, 0] = 2.0        # cos, k = 0
    w1[1, 128] = -3.0     # sin, k = 0
    w1[2, 5] = 1.5        # cos, k = 5
    w1[3, 255] = 4.0      # sin, k = 127
    w2 = np.array([[0.0, 1.5, 0.0, 0.0],
                   [1.0, 0.0, -1.0, 0.0],
                   [0.0, 0.0, 0.0, 2.0],
                   [0.5, 0.5, 0.5, 0.5]])
    b2 = np.array([0.25, -0.5, 0.0, 1.0])
    P = {"time.w1": w1, "time.b1": b1, "time.w2": w2, "time.b2": b2}
    silu = lambda z: z / (1.0 + math.exp(-z))
    for t in (0.0, 0.3, 1.0):
        a0 = 1000.0 * t
        a5 = 1000.0 * t * 10000.0 ** (-5 / 128)
        a127 = 1000.0 * t * 10000.0 ** (-127 / 128)
        h = [silu(2.0 * math.cos(a0) + 0.5), silu(-3.0 * math.sin(a0)),
             silu(1.5 * math.cos(a5) - 0.25), silu(4.0 * math.sin(a127) + 0.1)]
        want = [1.5 * h[1] + 0.25, h[0] - h[2] - 0.5, 2.0 * h[3], 0.5 * sum(h) + 1.0]
        got = O.time_embed(P, np.array([t]))[0]
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_final_layer_hand_derived():
    # rows with a known LayerNorm: [1,-1,1,-1] normalises to itself / sqrt(1 + eps),
    # a constant row to zero.  One-hot output rows then read single modulated
    # entries: catches shift / scale swapped, a missing (1 + scale) and the
    # LN epsilon misplaced
    x = np.array([[[1.0, -1.0, 1.0, -1.0], [2.0, 2.0, 2.0, 2.0]]])
    shift = np.array([[[0.1, 0.2, 0.3, 0.4]]])
    scale = np.array([[[1.0, 0.0, -1.0, 0.5]]])
    w = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 0.0, 1.0, 0.0], [0.0, 0.0, 0.0, -2.0]])
    b = np.array([0.01, 0.02, 0.03])
    n = 1.0 / math.sqrt(1.0 + 1e-6)
    want = np.array([[[2.0 * n + 0.1 + 0.01, 0.0 * n + 0.3 + 0.02, -2.0 * (-1.0 * n * 1.5 + 0.4) + 0.03],
                      [0.1 + 0.01, 0.3 + 0.02, -2.0 * 0.4 + 0.03]]])
    got = O.final_layer(x, shift, scale, w, b)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_step_velocity_head_wiring_hand_derived():
    # a whole oracle step whose blocks are identities (every gate 0) and whose
    # final modulation is constant (weight 0, bias = [shift ; scale]): the
    # velocity is then a closed form of the embedded latents, which pins the
    # final layer's chunk order (shift first), its use of the image rows only
    # and the Euler update's sign and step
    import dit_inputs as DI
    dims = DI.Dims(D=4, H=1, F=8, n_double=1, n_single=1, C_in=4)
    w = DI.Workload("t", dims, B=1, grid_h=1, grid_w=2, Lt=2, dtype="f32", steps=2, shift=1.0)
    rng = np.random.default_rng(17)
    P = {}
    for name, t in DI.iter_params(dims, "f32"):
        P[name] = rng.standard_normal(tuple(t.shape)) * 0.1
    for s in ("img", "txt"):
        P[f"double0.{s}.mod.w"][:] = 0.0
        P[f"double0.{s}.mod.b"][:] = 0.0       # gates 0: the double block is the identity
    P["single0.mod.w"][:] = 0.0
    P["single0.mod.b"][:] = 0.0                # gate 0: so is the single block
    P["img_in.w"] = np.eye(4) * 2.0
    P["img_in.b"] = np.zeros(4)
    shift = np.array([0.1, 0.2, 0.3, 0.4]); scale = np.array([1.0, 0.0, -1.0, 0.5])
    P["final.mod.w"][:] = 0.0
    P["final.mod.b"] = np.concatenate([shift, scale])
    P["final.out.w"] = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0], [0, 0, 1.0, 0], [0, 0, 0, 1.0]])
    P["final.out.b"] = np.array([0.0, 0.5, 0.0, -0.5])
    lat = np.array([[[0.5, -0.5, 0.5, -0.5], [1.0, 1.0, 1.0, 1.0]]])     # [1, Li = 2, C_in]
    txt = rng.standard_normal((1, 2, 4))
    sg = O.sigmas(2, 1.0)                                               # 1, 0.5, 0
    new, info = O.denoise_step(P, dims, w, lat, txt, 0, sg)
    n = 1.0 / math.sqrt(1.0 + 1e-6)
    ln0 = np.array([n, -n, n, -n])                     # h = 2 lat = [1,-1,1,-1]
    v0 = ln0 * (1.0 + scale) + shift + P["final.out.b"]
    v1 = shift + P["final.out.b"]                       # constant row: LN = 0
    np.testing.assert_allclose(info["v"][0], [v0, v1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(new[0], lat[0] - 0.5 * np.array([v0, v1]), rtol=0, atol=1e-14)



@pytest.mark.parametrize("fp8,mx4", [(False, False), (True, False), (False, True)])
def test_single_block_rows_equals_full_block(fp8, mx4):
    rng = np.random.default_rng(18)
    D, H, F, Lt, gh, gw, B = 64, 2, 256, 3, 4, 8, 2
    L = Lt + gh * gw
    P = {"lin1.w": rng.standard_normal((3 * D + F, D)) * 0.05,
         "lin1.b": rng.standard_normal(3 * D + F) * 0.05,
         "lin2.w": rng.standard_normal((D, D + F)) * 0.05,
         "lin2.b": rng.standard_normal(D) * 0.05}
    x = rng.standard_normal((B, L, D))
    mod = rng.standard_normal((B, 3, D)) * 0.1
    ang = O.rope_table(O.image_positions(gh, gw, Lt), D // H)
    full = O.single_block(x, mod, P, ang, H, fp8=fp8, mx4=mx4)
    rows = np.array([0, 2, Lt, Lt + 5, L - 1])
    got = O.single_block_rows(x, mod, P, ang, H, rows, fp8=fp8, mx4=mx4)
    np.testing.assert_allclose(got, full[:, rows], rtol=0, atol=1e-12)


def test_modulation_vectors_hand_derived():
    # SiLU is applied to c before the modulation linear, and the output is cut
    # into D-wide chunks in order: catches a missing SiLU, SiLU after the linear
    # and a transposed [chunk, D] split
    D = 2
    c = np.array([[1.0, -2.0]])
    w = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, 0.0], [0.0, -1.0], [1.0, 1.0], [0.0, 0.0]])
    b = np.array([0.0, 0.0, 0.5, 0.0, 0.0, 0.25])
    s1 = 1.0 / (1.0 + math.exp(-1.0))             # SiLU(1)
    s2 = -2.0 / (1.0 + math.exp(2.0))             # SiLU(-2)
    want = np.array([[[s1, s2], [2 * s1 + 0.5, -s2], [s1 + s2, 0.25]]])
    got = O.modulation_vectors(c, w, b, D)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)



def test_attention_fp8_fp32_window_covers_fp32_decisions():
    # p448_fp32_window must bound the relative error of 448 P evaluated in fp32,
    # score by score: scores summed sequentially in fp32 from the exact e4m3
    # products (the worst ordering), the fp32 score scale, one fused multiply-add
    # against the fp32 reference, exp2 in fp32 -- so every P code such an
    # evaluation can decide differently lies inside the window.  Small and large
    # score magnitudes both occur.
    rng = np.random.default_rng(21)
    d, L = 128, 256
    worst = 0.0
    for trial in range(3):
        q = rng.standard_normal((1, 1, L, d)) * (1.0 + 2 * trial)
        k = rng.standard_normal((1, 1, L, d))
        qc, sq = quantize_rows_e4m3(q[0, 0].reshape(1, -1))
        kc, sk = quantize_rows_e4m3(k[0, 0].reshape(1, -1))
        qc = qc.reshape(L, d).astype(np.float32)
        kc = kc.reshape(L, d).astype(np.float32)
        s32 = np.zeros((L, L), dtype=np.float32)
        for c in range(d):                                # fp32, one rounding per add
            s32 = (s32 + np.outer(qc[:, c], kc[:, c]).astype(np.float32)).astype(np.float32)
        scale = 1.0 / math.sqrt(d)
        scale_log2 = np.float32(np.float32(scale) * np.float32(1.4426950408889634))
        cs = np.float32(np.float32(scale_log2 * sq[0]) * sk[0])
        qd = qc.astype(np.float64) * float(sq[0])
        kd = kc.astype(np.float64) * float(sk[0])
        t64 = qd @ kd.T * (scale / math.log(2.0))
        r = np.ceil(t64.max(axis=1, keepdims=True))
        moff = (r.astype(np.float32) - np.float32(math.log2(448.0))).astype(np.float32)
        arg = (s32.astype(np.float64) * float(cs) - moff.astype(np.float64)).astype(np.float32)
        y32 = np.exp2(arg).astype(np.float64)
        y64 = np.exp2(t64 - r) * 448.0
        T = np.abs(qd) @ np.abs(kd).T * (scale / math.log(2.0))
        rel = O.p448_fp32_window(t64, r, T, d)
        err = np.abs(y32 - y64) / y64
        worst = max(worst, float(np.max(err / rel)))
        assert np.all(err <= rel), (trial, float(np.max(err / rel)))
        # and the window stays narrow: a small share of codes lies inside it
        tie, _ = e4m3_tie_mask(y64, rel)
        assert tie.mean() < 0.02
    print(f"largest fp32 error / window: {worst:.3f}")
    assert worst > 1e-3            # the emulation's error is measured, not zero

# ---------------------------------------------------------------- FBC

def test_fbcache_rel_vs_python_loop():
    rng = np.random.default_rng(16)
    r = rng.standard_normal(1000)
    a = r + 0.05 * rng.standard_normal(1000)
    num = 0.0
    den = 0.0
    for x, y in zip(r.tolist(), a.tolist()):
        num += abs(x - y)
        den += abs(y)
    assert abs(O.fbcache_rel(r, a) - num / den) < 1e-12
    assert O.fbcache_rel(r, r) == 0.0
    assert O.fbcache_rel(r, np.zeros_like(r)) == math.inf
    assert not O.fbcache_decide(math.nan, 1.0)
    assert not O.fbcache_decide(0.12, 0.12)     # strict
    assert O.fbcache_decide(0.1199, 0.12)
    assert not O.fbcache_decide(0.0, 0.0)
    assert not O.fbcache_decide(math.inf, math.inf)


def test_fbcache_policy_cases():
    # (test says skip, steps done, warm-up steps, skips in a row, max skips) -> skip
    cases = [
        (False, 10, 0, 0, 0, False),   # the rel test decides first
        (True, 0, 0, 0, 0, True),      # no policy: the test alone
        (True, 2, 3, 0, 0, False),     # third step of a 3-step warm-up
        (True, 3, 3, 0, 0, True),      # first step after it
        (True, 9, 3, 1, 2, True),      # one skipped, two allowed
        (True, 9, 3, 2, 2, False),     # two skipped in a row: compute
        (True, 9, 0, 50, 0, True),     # max_skips 0: no limit
    ]
    for test, done, warm, run, mx, want in cases:
        assert O.fbcache_policy(test, done, warm, run, mx) == want, (test, done, warm, run, mx)


# ---------------------------------------------------------------- number formats

def _e4m3_table():
    vals = []
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 7
        if e == 15 and m == 7:
            continue
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals.append((s * v, code))
    return vals


def test_e4m3_code_table_bruteforce():
    table = _e4m3_table()
    pos = sorted((v, c) for v, c in table if v >= 0 and not (v == 0 and c & 0x80))
    assert len(pos) == 127 and pos[-1][0] == 448.0
    rng = np.random.default_rng(17)
    xs = np.concatenate([rng.standard_normal(4000) * 30, rng.standard_normal(2000) * 0.01,
                         [p[0] for p in pos],
                         [(pos[i][0] + pos[i + 1][0]) / 2 for i in range(126)]])
    vals = np.array([p[0] for p in pos])
    codes = np.array([p[1] for p in pos])
    for x in xs:
        ax = min(abs(x), 448.0)
        dist = np.abs(vals - ax)
        best = np.flatnonzero(dist == dist.min())
        if len(best) > 1:                   # tie: the even code
            best = [b for b in best if codes[b] % 2 == 0]
        want = math.copysign(vals[best[0]], x)
        assert round_e4m3(np.array(x)) == want, x


def test_e4m3_golden_points():
    for x, want in _golden_rows("e4m3_points.txt"):
        assert round_e4m3(np.array(x)) == want, (x, want)


def test_e4m3_representable_values_are_fixed_points():
    vals = np.array([v for v, _ in _e4m3_table()])
    np.testing.assert_array_equal(round_e4m3(vals), vals)


def test_bf16_rounding_vs_torch_cast():
    rng = np.random.default_rng(18)
    x32 = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 100,
                          (rng.standard_normal(2000) * 1e-39).astype(np.float32),
                          np.array([3.0e38, -3.0e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32)])
    want = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(round_bf16(x32.astype(np.float64)), want)


def test_quantize_rows_scale_and_roundtrip():
    # rows whose amax is 448 and whose entries are e4m3 values quantise exactly
    rng = np.random.default_rng(19)
    vals = np.array([v for v, _ in _e4m3_table()])
    x = rng.choice(vals, size=(6, 40))
    x[:, 0] = 448.0
    q, s = quantize_rows_e4m3(x)
    np.testing.assert_array_equal(s, np.float32(1.0))
    np.testing.assert_array_equal(q, x)
    z, sz = quantize_rows_e4m3(np.zeros((2, 5)))
    np.testing.assert_array_equal(sz, 1.0)
    np.testing.assert_array_equal(z, 0.0)


def test_linear_fp8_exact_on_representable_inputs():
    rng = np.random.default_rng(20)
    vals = np.array([v for v, _ in _e4m3_table()])
    vals = vals[np.abs(vals) <= 4]
    x = rng.choice(vals, size=(5, 32)); x[:, 0] = 448.0
    w = rng.choice(vals, size=(7, 32)); w[:, 0] = 448.0
    b = rng.standard_normal(7)
    np.testing.assert_allclose(O.linear_fp8(x, w, b), O.linear(x, w, b), rtol=1e-15)


def test_attention_fp8_identical_keys_mean_of_v():
    rng = np.random.default_rng(21)
    vals = np.array([v for v, _ in _e4m3_table()])
    L, d = 20, 64
    v = rng.choice(vals[np.abs(vals) < 100], size=(1, 1, L, d))
    v[0, 0, 0, :] = 448.0                  # head amax 448 -> scale 1
    k = np.broadcast_to(rng.standard_normal((1, 1, 1, d)), (1, 1, L, d)).copy()
    q = rng.standard_normal((1, 1, L, d))
    out = O.attention_fp8(q, k, v)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=2, keepdims=True), out.shape),
                               rtol=1e-14)


def test_fp16_rounding_vs_numpy_cast():
    rng = np.random.default_rng(30)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 5, 20000),
                        [0.0, -0.0, 65504.0, 65519.9, 65520.0, -70000.0, 2.0 ** -24,
                         2.0 ** -25, 3 * 2.0 ** -26, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11]])
    with np.errstate(over="ignore"):                 # overflow to inf is the point
        want = x.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(round_fp16(x), want)


def test_e4m3_tie_mask_against_code_table():
    # midpoints between consecutive non-negative e4m3 values, from the enumerated table
    vals = np.unique([v for v, _ in _e4m3_table() if v >= 0])
    mids = (vals[1:] + vals[:-1]) / 2
    rng = np.random.default_rng(31)
    y = np.concatenate([rng.uniform(0, 448, 5000), 2.0 ** rng.uniform(-10, 8.8, 5000),
                        mids, mids * (1 + 1e-5), mids * (1 - 3e-5)])
    y = y[y <= 448]
    rel = 2e-5
    want = np.min(np.abs(y[:, None] - mids[None, :]), axis=1) <= rel * y
    got, step = e4m3_tie_mask(y, rel)
    np.testing.assert_array_equal(got, want)
    # step: distance to the next code up from the code at or below y
    lo = vals[np.searchsorted(vals, y, side="right") - 1]
    hi = vals[np.minimum(np.searchsorted(vals, y, side="right"), len(vals) - 1)]
    inner = y < 448
    np.testing.assert_array_equal(step[inner], (hi - lo)[inner])


def test_attention_fp8_slack_grows_with_the_band():
    rng = np.random.default_rng(32)
    q, k, v = (rng.standard_normal((1, 2, 48, 64)) for _ in range(3))
    out0, s0 = O.attention_fp8(q, k, v, tie_rel=0.0)
    _, s1 = O.attention_fp8(q, k, v, tie_rel=1e-3)
    _, s2 = O.attention_fp8(q, k, v, tie_rel=1e-1)
    np.testing.assert_array_equal(out0, O.attention_fp8(q, k, v))
    assert np.all(s0 == 0) and np.all(s1 <= s2) and np.all(s2 >= 0) and s2.max() > 0


def test_attention_fp8_identical_values_returned_exactly():
    # the weights are normalised by the sum of the quantised P, so they sum to
    # one and a V whose rows are all equal (and representable) comes back as is
    rng = np.random.default_rng(24)
    vals = np.array([v for v, _ in _e4m3_table()])
    L, d = 40, 64
    row = rng.choice(vals[np.abs(vals) < 100], size=d)
    row[7] = 448.0
    v = np.broadcast_to(row, (1, 1, L, d)).copy()
    q, k = rng.standard_normal((1, 1, L, d)) * 2, rng.standard_normal((1, 1, L, d)) * 2
    np.testing.assert_allclose(O.attention_fp8(q, k, v), v, rtol=1e-14, atol=0)


def test_attention_fp8_exact_when_p_is_representable():
    # q = 0.875 e0, k_j = -(j mod 8) e0 and softmax scale ln 2 / 0.875 give
    # P_j = 2^-(j mod 8).  The head scales 0.875/448 = 2^-9, 7/448 = 2^-6 and
    # 448/448 are exact in fp32, Q, K, V quantise exactly and so does 448 P, so
    # the fp8 path equals exact attention on the same values
    rng = np.random.default_rng(23)
    vals = np.array([v for v, _ in _e4m3_table()])
    L, d = 16, 64
    q = np.zeros((1, 1, L, d)); q[..., 0] = 0.875
    k = np.zeros((1, 1, L, d)); k[0, 0, :, 0] = -(np.arange(L) % 8)
    v = rng.choice(vals[np.abs(vals) < 100], size=(1, 1, L, d))
    v[0, 0, 3, 5] = 448.0
    sc = math.log(2.0) / 0.875
    got = O.attention_fp8(q, k, v, scale=sc)
    np.testing.assert_allclose(got, O.attention(q, k, v, scale=sc), rtol=1e-13, atol=1e-13)


def test_attention_fp8_close_to_exact():
    # each P_j V_j term carries at most a few e4m3 half-ulps (2^-4 each) of
    # relative error, so the deviation is bounded by a small multiple of the
    # attention-weighted mean of |V| (the output itself can be much smaller)
    rng = np.random.default_rng(22)
    q, k, v = (rng.standard_normal((1, 2, 64, 64)) for _ in range(3))
    ex = O.attention(q, k, v)
    wabs = O.attention(q, k, np.abs(v))
    assert np.max(np.abs(O.attention_fp8(q, k, v) - ex) / wabs) < 0.3


# ---------------------------------------------------------------- MXFP4 (W4A4 variant)

def test_e2m1_rounding_cases():
    # (input, nearest E2M1 value; ties to the even mantissa; beyond 6 saturates)
    cases = [(0.0, 0.0), (0.25, 0.0), (0.26, 0.5), (0.75, 1.0), (1.25, 1.0), (1.3, 1.5),
             (1.75, 2.0), (2.5, 2.0), (2.51, 3.0), (3.5, 4.0), (5.0, 4.0), (5.01, 6.0),
             (6.0, 6.0), (7.0, 6.0), (1e9, 6.0), (-0.74, -0.5), (-5.5, -6.0)]
    got = O.round_e2m1(np.array([c[0] for c in cases]))
    np.testing.assert_array_equal(got, np.array([c[1] for c in cases]))


def test_e2m1_value_set():
    x = np.linspace(-10, 10, 200001)
    vals = set(np.unique(O.round_e2m1(x)).tolist())
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert vals == set(mags) | set(-m for m in mags)


def test_mx_block_exponent_cases():
    # floor(log2 amax) - 2: a block maximum in [4, 8) * 2^e
    amax = np.array([6.0, 7.99, 8.0, 0.5, 1.0, 3.0, 0.0, 2.0 ** -200])
    np.testing.assert_array_equal(O.mx_block_exponent(amax), [0, 0, 1, -3, -2, -1, 0, -127])


def test_mxfp4_reproduces_representable_blocks():
    # every 32-block holds E2M1 values times one power of two, with a +-4 or +-6
    # in it: quantisation returns the input and the W4A4 linear is the exact product
    rng = np.random.default_rng(5)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

    def make(rows, K):
        q = rng.choice(mags, size=(rows, K)) * rng.choice([-1.0, 1.0], size=(rows, K))
        q[:, ::32] = rng.choice([-6.0, -4.0, 4.0, 6.0], size=(rows, K // 32))
        e = rng.integers(-6, 6, size=(rows, K // 32))
        return O.dequantize_mxfp4(q, e), q, e

    x, qx, ex = make(5, 96)
    w, _, _ = make(7, 96)
    q2, e2 = O.quantize_mxfp4(x)
    np.testing.assert_array_equal(q2, qx)
    np.testing.assert_array_equal(e2, ex)
    b = rng.standard_normal(7)
    np.testing.assert_array_equal(O.linear_mxfp4(x, w, b), x @ w.T + b)


def test_mxfp4_error_bound():
    x = np.random.default_rng(6).standard_normal((64, 256)) * 3.0
    q, e = O.quantize_mxfp4(x)
    d = O.dequantize_mxfp4(q, e)
    scale = np.repeat(np.ldexp(1.0, e), 32, axis=-1)
    err = np.abs(x - d)
    assert np.all(err <= 2.0 * scale)                        # saturation above 6 * 2^e
    inside = np.abs(x) <= 6.0 * scale
    assert np.all(err[inside] <= 1.0 * scale[inside])        # half the top binade's spacing
    blk_max = np.abs(x).reshape(64, 8, 32).max(-1)
    s = np.ldexp(1.0, e)
    assert np.all((blk_max >= 4 * s) & (blk_max < 8 * s))
