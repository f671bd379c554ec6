"""Stage-by-stage replay of the fp8 (W8A8, OCP e4m3) blocks against the oracle.

A whole fp8 block is compared end to end elsewhere; here every stage of it is
recomputed by the oracle from the kernel's own inputs to that stage (the
intermediates the block leaves in its workspace, read through
dit_block_views_of), so a stage that disagrees on identical inputs is a kernel
error, and what remains end to end is the propagation of near-tie code
decisions through later quantisations.

  * integer work on identical inputs is compared bit for bit: the e4m3 codes
    and fp32 scales of Q / K / V (per (b, h)), of the attention output and of
    the GELU hidden (per row);
  * float work on identical inputs (the fp8 GEMMs with their epilogues, fp8
    attention) meets the fp8 bound, and the GEMM stages meet the bf16 bound of
    their stored bf16 outputs;
  * codes decided on values computed on each side (LN outputs) must agree
    except for near-ties, which are counted: at most a 1e-3 share of codes,
    each one e4m3 step from the oracle's.
"""
import sys

import numpy as np
import pytest
import torch

import dit_inputs as DI
import oracle as O
from oracle.numerics import quantize_rows_e4m3, round_bf16
from _helpers import parity_err, parity_err_bf16_stored

pytestmark = pytest.mark.gpu

TOL_FP8 = 6e-2
TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def dit():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from image_generation_amd import dit as D
    return D


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _codes(t: torch.Tensor) -> np.ndarray:
    """e4m3 bytes -> fp64 values (torch's float8_e4m3fn decoder on the CPU)."""
    return t.cpu().view(torch.float8_e4m3fn).double().numpy()


def _np(t):
    return t.cpu().double().numpy()


def _code_diffs(got, want):
    """(share of differing codes, largest step between differing codes in units
    of the e4m3 spacing at the oracle's value)."""
    diff = got != want
    if not diff.any():
        return 0.0, 0.0
    w = np.abs(want[diff])
    _, e = np.frexp(np.maximum(w, 2.0 ** -9))
    step = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    return float(diff.mean()), float(np.max(np.abs(got[diff] - want[diff]) / step))


def _check_ties(name, got_codes, got_scale, want_codes, want_scale):
    share, steps = _code_diffs(got_codes, want_codes)
    srel = float(np.max(np.abs(got_scale - want_scale) / want_scale))
    _say(f"  {name}: codes differing {share:.2e} (max {steps:.0f} step), scale rel diff {srel:.1e}")
    assert share <= 1e-3 and steps <= 1.0 and srel <= 1e-6


def _setup(dit, dims, w, kind):
    params = DI.block_params(dims, "bf16", kind)
    dev = {n: (t.cuda() if n.endswith(".w") else t.float().cuda()) for n, t in params.items()}
    dev8 = dit.quantize_block_params(dev)
    inp = DI.block_inputs(w, kind)
    blk = dit.make_double_block(dev8) if kind == "double" else dit.make_single_block(dev8)
    dd = dit.dims_of(w.B, w.Lt, w.grid_h, w.grid_w, dims.D, dims.H, dims.F)
    rope = dit.dit_rope_table(w.grid_h, w.grid_w, w.Lt, dims.d)
    ws = dit.workspace(dd, dit.DIT_WS_BLOCK)
    x = inp["x"].float().cuda()
    dit.dit_block_forward(dd, blk, x, inp["mod"].cuda(), rope, ws, dtype=dit.DIT_FP8)
    torch.cuda.synchronize()
    V = dit.block_views(dd, ws)
    P = {k: O.to64(v) for k, v in params.items()}
    ang = O.rope_table(O.image_positions(w.grid_h, w.grid_w, w.Lt), dims.d)
    return P, inp, V, _np(x), ang


def _heads(x, H):
    B, L, D = x.shape
    return x.reshape(B, L, H, D // H).transpose(0, 2, 1, 3)


def _merge(x):
    B, H, L, d = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B, L, H * d)


def _qkv_stages(V, q_ref, k_ref, v_ref, B, H):
    """Q / K / V against the oracle's, then their per-(b, h) codes and scales
    bit for bit from the kernel's own bf16 values; returns the kernel's Q, K, V."""
    kq, kk, kv = _np(V["q"]), _np(V["k"]), _np(V["v"])
    for name, got, ref in (("q", kq, q_ref), ("k", kk, k_ref), ("v", kv, v_ref)):
        err = parity_err_bf16_stored(got, ref)
        same = float(np.mean(got == round_bf16(ref)))
        _say(f"  {name}: err {err:.2e} (equal to the oracle's bf16 value: {same:.5f})")
        assert err <= TOL_BF16
    sc = _np(V["qkv_scale"])
    for i, (name, t) in enumerate((("q", kq), ("k", kk), ("v", kv))):
        codes = _codes(V[name + "8"])
        for b in range(B):
            for h in range(H):
                c, s = quantize_rows_e4m3(t[b, h].reshape(1, -1))
                np.testing.assert_array_equal(codes[b, h].reshape(1, -1), c, err_msg=f"{name}8 b{b} h{h}")
                assert sc[i, b, h] == s[0], (name, b, h)
    _say("  q / k / v codes and scales: bit-exact")
    return kq, kk, kv


def _attention_stage(kq, kk, kv, got):
    """fp8 attention on the kernel's own Q / K / V against the kernel's output."""
    ref, slack = O.attention_fp8(kq, kk, kv, tie_fp32=True)
    g = np.asarray(got)
    _, e = np.frexp(np.abs(ref))
    excess = np.maximum(np.abs(g - ref) - slack - np.ldexp(1.0, e - 9), 0.0)
    err = float(np.max(excess) / np.sqrt(np.mean(ref * ref)))
    _say(f"  attention: err {err:.2e} (without slack {parity_err_bf16_stored(g, ref):.2e}, "
         f"{float(np.mean(slack > 0)):.3f} of outputs near a P-code tie)")
    assert err <= TOL_FP8


@pytest.mark.parametrize("B,Lt,gh,gw", [(1, 32, 12, 20), (2, 16, 8, 10)])
def test_fp8_double_block_stages(dit, B, Lt, gh, gw):
    dims = DI.Dims(D=3072, H=24, F=12288, n_double=1, n_single=0)
    w = DI.Workload("t", dims, B=B, grid_h=gh, grid_w=gw, Lt=Lt, dtype="fp8")
    _say(f"fp8 double block stages B={B} Lt={Lt} grid={gh}x{gw}")
    P, inp, V, x_out, ang = _setup(dit, dims, w, "double")
    D, H, Li = dims.D, dims.H, w.Li
    x0 = O.to64(inp["x"])
    mod = O.to64(inp["mod"])
    streams = {"img": (x0[:, Lt:], mod[:, :6]), "txt": (x0[:, :Lt], mod[:, 6:])}

    def sm(rows_arr, s):         # stream-major rows of stream s -> [B, L_s, ...]
        if s == "img":
            return rows_arr[:B * Li].reshape(B, Li, -1)
        return rows_arr[B * Li:].reshape(B, Lt, -1)

    # QKV GEMM + RoPE from the LN of the (shared) block input
    qkv = {s: O.linear_fp8(O.modulate(x, m[:, 0:1], m[:, 1:2]), P[f"{s}.qkv.w"], P[f"{s}.qkv.b"])
           for s, (x, m) in streams.items()}
    cat = np.concatenate([qkv["txt"], qkv["img"]], axis=1)
    q_ref = O.apply_rope(_heads(cat[..., :D], H), ang)
    k_ref = O.apply_rope(_heads(cat[..., D:2 * D], H), ang)
    v_ref = _heads(cat[..., 2 * D:], H)
    kq, kk, kv = _qkv_stages(V, q_ref, k_ref, v_ref, B, H)

    # attention (kernel's Q / K / V); output rows are stream-major
    catk = _np(V["cat"])
    att = np.concatenate([sm(catk[:, :D], "txt"), sm(catk[:, :D], "img")], axis=1)
    _attention_stage(kq, kk, kv, _heads(att, H))

    # attention-output codes (per row over D) bit for bit
    c_att, s_att = quantize_rows_e4m3(catk[:, :D])
    cat8 = _codes(V["cat8"])
    np.testing.assert_array_equal(cat8[:, :D], c_att)
    np.testing.assert_array_equal(_np(V["att_scale"]), s_att)
    _say("  attention-output codes and scales: bit-exact")

    # projection + gated residual from the kernel's codes, then the second LN's codes
    x_mid, u2 = {}, {}
    for s, (x, m) in streams.items():
        y = O.linear_fp8_codes(sm(cat8[:, :D], s).reshape(-1, D), sm(s_att[:, None], s).reshape(-1),
                               P[f"{s}.proj.w"], P[f"{s}.proj.b"]).reshape(x.shape)
        x_mid[s] = x + m[:, 2:3] * y
        u2[s] = O.modulate(x_mid[s], m[:, 3:4], m[:, 4:5])
    u2_rows = np.concatenate([u2["img"].reshape(-1, D), u2["txt"].reshape(-1, D)], axis=0)
    c2, s2 = quantize_rows_e4m3(u2_rows)
    ln8, ln_s = _codes(V["ln8"]), _np(V["ln_scale"])
    _check_ties("second LN codes", ln8, ln_s, c2, s2.astype(np.float64))

    # MLP up-projection + GELU from the kernel's LN codes
    hid_k = catk[:, D:]
    for s, (x, m) in streams.items():
        rows = slice(0, B * Li) if s == "img" else slice(B * Li, B * (Li + Lt))
        h = O.gelu_tanh(O.linear_fp8_codes(ln8[rows], ln_s[rows], P[f"{s}.mlp1.w"],
                                           P[f"{s}.mlp1.b"]))
        err = parity_err_bf16_stored(hid_k[rows], h)
        same = float(np.mean(hid_k[rows] == round_bf16(h)))
        _say(f"  {s} GELU hidden: err {err:.2e} (equal to the oracle's bf16 value: {same:.5f})")
        assert err <= TOL_BF16

    # GELU-hidden codes bit for bit
    c_h, s_h = quantize_rows_e4m3(hid_k)
    np.testing.assert_array_equal(cat8[:, D:], c_h)
    np.testing.assert_array_equal(_np(V["hid_scale"]), s_h)
    _say("  GELU-hidden codes and scales: bit-exact")

    # down-projection + gated residual from the kernel's codes: the block output
    ref = {}
    for s, (x, m) in streams.items():
        y = O.linear_fp8_codes(sm(cat8[:, D:], s).reshape(-1, dims.F), sm(s_h[:, None], s).reshape(-1),
                               P[f"{s}.mlp2.w"], P[f"{s}.mlp2.b"]).reshape(x.shape)
        ref[s] = x_mid[s] + m[:, 5:6] * y
    ref_out = np.concatenate([ref["txt"], ref["img"]], axis=1)
    err = parity_err(x_out, ref_out)
    derr = parity_err(x_out - x0, ref_out - x0)
    _say(f"  block output from the kernel's stage inputs: x_out err {err:.2e}, branch err {derr:.2e}")
    assert derr <= TOL_FP8


@pytest.mark.parametrize("B,Lt,gh,gw", [(1, 32, 12, 20), (2, 16, 8, 10)])
def test_fp8_single_block_stages(dit, B, Lt, gh, gw):
    dims = DI.Dims(D=3072, H=24, F=12288, n_double=0, n_single=1)
    w = DI.Workload("t", dims, B=B, grid_h=gh, grid_w=gw, Lt=Lt, dtype="fp8")
    _say(f"fp8 single block stages B={B} Lt={Lt} grid={gh}x{gw}")
    P, inp, V, x_out, ang = _setup(dit, dims, w, "single")
    D, H, F, L = dims.D, dims.H, dims.F, w.L
    x0 = O.to64(inp["x"])
    mod = O.to64(inp["mod"])

    # the block's one LN: codes decided on each side's own fp32 / fp64 values
    u = O.modulate(x0, mod[:, 0:1], mod[:, 1:2])
    c1, s1 = quantize_rows_e4m3(u.reshape(-1, D))
    ln8, ln_s = _codes(V["ln8"]), _np(V["ln_scale"])
    _check_ties("LN codes", ln8, ln_s, c1, s1.astype(np.float64))

    # linear1 from the kernel's LN codes: Q, K (rotated), V and the GELU half
    h = O.linear_fp8_codes(ln8, ln_s, P["lin1.w"], P["lin1.b"]).reshape(B, L, -1)
    q_ref = O.apply_rope(_heads(h[..., :D], H), ang)
    k_ref = O.apply_rope(_heads(h[..., D:2 * D], H), ang)
    v_ref = _heads(h[..., 2 * D:3 * D], H)
    kq, kk, kv = _qkv_stages(V, q_ref, k_ref, v_ref, B, H)
    catk = _np(V["cat"])
    g_ref = O.gelu_tanh(h[..., 3 * D:]).reshape(-1, F)
    err = parity_err_bf16_stored(catk[:, D:], g_ref)
    _say(f"  GELU half: err {err:.2e} (equal: {float(np.mean(catk[:, D:] == round_bf16(g_ref))):.5f})")
    assert err <= TOL_BF16

    _attention_stage(kq, kk, kv, _heads(catk[:, :D].reshape(B, L, D), H))

    # linear2's input codes: one scale per joint row over [attention | GELU]
    c_cat, s_cat = quantize_rows_e4m3(catk)
    cat8 = _codes(V["cat8"])
    np.testing.assert_array_equal(cat8, c_cat)
    np.testing.assert_array_equal(_np(V["att_scale"]), s_cat)
    _say("  linear2 input codes and scales: bit-exact")

    y = O.linear_fp8_codes(cat8, s_cat, P["lin2.w"], P["lin2.b"]).reshape(B, L, D)
    ref_out = x0 + mod[:, 2:3] * y
    err = parity_err(x_out, ref_out)
    derr = parity_err(x_out - x0, ref_out - x0)
    _say(f"  block output from the kernel's stage inputs: x_out err {err:.2e}, branch err {derr:.2e}")
    assert derr <= TOL_FP8
