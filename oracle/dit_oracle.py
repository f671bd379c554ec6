"""Test infrastructure: plain fp64 CPU oracle of the DiT denoise step.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` import this module.  It shares no code with the HIP library.

What it computes, and which passage of the source pages each part follows:

* First-Block-Cache (FBC): the unsloth studio ``diffusion.py`` commit log,
  commit adding opt-in step caching (First-Block-Cache): the first block's
  residual is compared with the one cached from an earlier step; once it hardly
  moves, the remaining blocks are not run and their earlier contribution is
  added back instead; a quantised transformer gets a higher threshold.  The
  devotd.net VisualGen article (section on why the speed-ups differ, Cache-DiT
  paragraph) describes the same kind of test as a threshold on the change of a
  residual.
* Fused QKV projection: same commit log, speed-profile commit ("fused QKV").
* RoPE as its own step: the vflash "Optimization ledger" page, table
  "Accepted or exposed" (strict Triton RoPE row).
* Flow-matching schedule with a flow shift and an Euler solver: the ledger
  page, section "Fewer steps require a new contract" (scheduler, flow shift,
  solver tuned together).
* CFG with scale 3.5 on a positive/negative prompt pair: the VisualGen
  article, stage-latency table conditions.
* fp8 W8A8 with dynamic activation scales: runinfra.ai image-gen runbook,
  "Optimization stack" table, first row.

The pages give no formulas, so every formula below is a reading; each one
carries its reading number (R1..R32) as listed in the design notes.

Everything is fp64 numpy.  Parameters are ``dict[str, ndarray]`` with weights
in ``torch.nn.Linear`` layout ``[out, in]``: ``y = x @ W.T + b``.

Pins: each function, and the CPU test (``tests/test_oracle_pins.py`` unless
another file is named) that fails on a plausible mistake in it -- a dropped
term, a wrong sign or index, a transposed operand:

  sigmas              test_sigmas_golden_shift3 (hand-derived values),
                      test_sigmas_endpoints_monotone, test_sigmas_shift1_is_linear
  timestep_sinusoid   test_timestep_sinusoid_t0, test_timestep_sinusoid_frequencies
  silu, gelu_tanh     test_silu_vs_torch, test_gelu_tanh_vs_torch_and_erf
  linear              test_linear_vs_triple_loop, test_linear_one_hot_weight_selects_column
  time_embed          test_time_embed_hand_derived
  modulation_vectors  test_modulation_vectors_hand_derived
  layer_norm          test_layer_norm_vs_torch_and_moments
  modulate            test_modulate_identity_and_affine, test_final_layer_hand_derived
  image_positions,    test_rope_matches_complex_rotation_and_keeps_pair_norms,
  rope_table,         test_rope_relative_position_per_axis, test_rope_axis_split
  apply_rope
  attention           test_attention_rows_are_a_distribution,
                      test_attention_identical_keys_gives_mean_of_v,
                      test_attention_dominant_key, test_attention_vs_naive_triple_loop,
                      test_attention_vs_torch_sdpa
  attention_naive     the textbook triple loop itself; agrees with torch's SDPA
                      through test_attention_vs_torch_sdpa / _vs_naive_triple_loop
  linear_fp8,         test_linear_fp8_exact_on_representable_inputs,
  linear_fp8_codes    test_quantize_rows_scale_and_roundtrip
  linear_mxfp4        test_mx4_blocks_route_every_linear_through_mxfp4,
                      test_mx4_double_block_zero_weights_keeps_biases_exact,
                      test_mxfp4_reproduces_representable_blocks
  p448_fp32_window    test_attention_fp8_fp32_window_covers_fp32_decisions (an fp32
                      evaluation emulated on the CPU flips only codes inside it)
  attention_fp8       test_attention_fp8_identical_keys_mean_of_v,
                      test_attention_fp8_identical_values_returned_exactly,
                      test_attention_fp8_exact_when_p_is_representable,
                      test_attention_fp8_close_to_exact, test_attention_fp8_slack_grows_with_the_band
  double_block        test_double_block_brute_force_small, test_double_block_zero_gates_is_identity,
                      test_double_block_zero_value_weights, test_double_block_stream_isolation
  double_block_rows   test_double_block_rows_equals_full_block
  single_block        test_single_block_brute_force_small (with a planted q / k swap
                      that the hand version rejects), test_single_block_zero_gate_and_wiring
  single_block_rows   test_single_block_rows_equals_full_block
  final_layer         test_final_layer_hand_derived
  fbcache_rel         test_fbcache_rel_vs_python_loop;
                      tests/test_oracle_step.py::test_fbcache_rel_is_direct_recomputation
  fbcache_decide,     test_fbcache_policy_cases; tests/test_oracle_step.py (threshold 0
  fbcache_policy,     never skips, +inf skips every step after the first, warm-up / cap
  FBCacheState        patterns, identity tail: skip == full)
  euler_update        test_euler_constant_velocity_total_displacement,
                      test_euler_lands_on_target_for_exact_velocity
  cfg_combine         test_cfg_combine_cases;
                      tests/test_oracle_step.py::test_cfg_identical_prompts_equals_single
  denoise_step        test_step_velocity_head_wiring_hand_derived; tests/test_oracle_step.py
  to64                a cast (exact for bf16 and fp32 inputs)
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from .numerics import (quantize_rows_e4m3, round_e4m3, quant_scale_f32, E4M3_MAX, round_bf16,
                       e4m3_tie_mask, quantize_mxfp4, dequantize_mxfp4)

__all__ = [
    "sigmas", "timestep_sinusoid", "silu", "gelu_tanh", "layer_norm", "modulate",
    "linear", "rope_table", "apply_rope", "attention", "attention_naive",
    "double_block", "double_block_rows", "single_block", "single_block_rows", "final_layer", "fbcache_rel",
    "fbcache_decide", "fbcache_policy", "euler_update", "cfg_combine", "time_embed",
    "modulation_vectors", "denoise_step", "FBCacheState", "to64",
    "linear_fp8", "linear_fp8_codes", "linear_mxfp4", "attention_fp8", "p448_fp32_window", "image_positions",
]

LN_EPS = 1e-6
ROPE_THETA = 10000.0
TIME_PERIOD = 10000.0
TIME_SCALE = 1000.0


def to64(t) -> np.ndarray:
    """torch tensor / array -> fp64 ndarray (exact for bf16 and fp32 inputs)."""
    if hasattr(t, "detach"):
        t = t.detach().to("cpu").double().numpy()
    return np.asarray(t, dtype=np.float64)


# --------------------------------------------------------------------------
# schedule and embeddings
# --------------------------------------------------------------------------

def sigmas(num_steps: int, shift: float) -> np.ndarray:
    """Shifted flow-matching sigmas (R14): tau_i = 1 - i/N, sigma = s*tau / (1 + (s-1)*tau)."""
    tau = 1.0 - np.arange(num_steps + 1, dtype=np.float64) / num_steps
    return shift * tau / (1.0 + (shift - 1.0) * tau)


def timestep_sinusoid(t, dim: int = 256) -> np.ndarray:
    """[cos(1000 t w_k), sin(1000 t w_k)], w_k = 10000^(-k/(dim/2)) (R5). t: [M] -> [M, dim]."""
    t = np.atleast_1d(np.asarray(t, dtype=np.float64))
    half = dim // 2
    w = TIME_PERIOD ** (-np.arange(half, dtype=np.float64) / half)
    arg = TIME_SCALE * t[:, None] * w[None, :]
    return np.concatenate([np.cos(arg), np.sin(arg)], axis=1)


def silu(x):
    return x / (1.0 + np.exp(-x))


def gelu_tanh(x):
    """GELU, tanh approximation (R9)."""
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def linear(x, w, b):
    """y = x W^T + b over the last axis."""
    return x @ w.T + b


def time_embed(P: Dict[str, np.ndarray], t) -> np.ndarray:
    """Timestep MLP (R5): c = W2 SiLU(W1 e + b1) + b2."""
    e = timestep_sinusoid(t)
    h = silu(linear(e, P["time.w1"], P["time.b1"]))
    return linear(h, P["time.w2"], P["time.b2"])


def modulation_vectors(c: np.ndarray, w: np.ndarray, b: np.ndarray, D: int) -> np.ndarray:
    """mu = W SiLU(c) + b, split into D-wide chunks (R4, R6). c: [M, D] -> [M, k, D]."""
    mu = linear(silu(c), w, b)
    return mu.reshape(mu.shape[0], -1, D)


# --------------------------------------------------------------------------
# normalisation, modulation, RoPE
# --------------------------------------------------------------------------

def layer_norm(u: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis, no affine, biased variance (R3)."""
    mu = u.mean(axis=-1, keepdims=True)
    var = ((u - mu) ** 2).mean(axis=-1, keepdims=True)
    return (u - mu) / np.sqrt(var + eps)


def modulate(u, shift, scale):
    """LN(u) * (1 + scale) + shift (R3, R4); shift/scale broadcast over tokens."""
    return layer_norm(u) * (1.0 + scale) + shift


def image_positions(grid_h: int, grid_w: int, Lt: int) -> np.ndarray:
    """(row, col) of every joint token: text tokens at (0, 0), image row-major (R7, R8)."""
    pos = np.zeros((Lt + grid_h * grid_w, 2), dtype=np.float64)
    ii = np.arange(grid_h * grid_w)
    pos[Lt:, 0] = ii // grid_w
    pos[Lt:, 1] = ii % grid_w
    return pos


def rope_table(pos: np.ndarray, d: int, theta: float = ROPE_THETA) -> np.ndarray:
    """Angles [L, d/2] of the 2-D RoPE (R7).

    Pair p < d/4 rotates with the row coordinate, pair p >= d/4 with the column;
    inside an axis, pair j turns at theta^(-j/(d/4)) radians per position.
    """
    q = d // 4
    p = np.arange(d // 2)
    j = p % q
    freq = theta ** (-j / q)
    axis = (p >= q).astype(np.int64)
    return pos[:, axis] * freq[None, :]


def apply_rope(x: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Rotate interleaved pairs (x[2p], x[2p+1]) by ang[t, p].  x: [..., L, d]."""
    a = x[..., 0::2]
    b = x[..., 1::2]
    c = np.cos(ang)
    s = np.sin(ang)
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def attention(q, k, v, scale: Optional[float] = None) -> np.ndarray:
    """softmax(q k^T * scale) v per (batch, head), no mask (R8).  q,k,v: [B, H, L, d]."""
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    B, H, L, _ = q.shape
    out = np.empty_like(q)
    for bi in range(B):
        for h in range(H):
            s = (q[bi, h] @ k[bi, h].T) * scale
            s = s - s.max(axis=1, keepdims=True)     # exact shift; softmax unchanged
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[bi, h] = p @ v[bi, h]
    return out


def attention_naive(q, k, v, scale: Optional[float] = None) -> np.ndarray:
    """Triple-loop attention for tiny shapes (a brute-force second opinion)."""
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    B, H, L, _ = q.shape
    Lk = k.shape[2]
    out = np.zeros_like(q)
    for bi in range(B):
        for h in range(H):
            for i in range(L):
                s = [sum(q[bi, h, i, c] * k[bi, h, j, c] for c in range(d)) * scale
                     for j in range(Lk)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                for c in range(d):
                    out[bi, h, i, c] = sum(e[j] * v[bi, h, j, c] for j in range(Lk)) / z
    return out


def _heads(x, H):
    """[B, L, D] -> [B, H, L, d]."""
    B, L, D = x.shape
    return x.reshape(B, L, H, D // H).transpose(0, 2, 1, 3)


def _merge(x):
    """[B, H, L, d] -> [B, L, D]."""
    B, H, L, d = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B, L, H * d)


# --------------------------------------------------------------------------
# fp8 W8A8 (R24-R28)
# --------------------------------------------------------------------------

def linear_mxfp4(x, w, b):
    """W4A4 linear with MXFP4 operands (see ``numerics``): activations x [..., K]
    and weights w [N, K] are both quantised along K in blocks of 32 with a shared
    power-of-two scale each; the product of the dequantised operands is taken in
    fp64, plus the bias."""
    shp = x.shape
    x2 = np.asarray(x).reshape(-1, shp[-1])
    qx, ex = quantize_mxfp4(x2)
    qw, ew = quantize_mxfp4(np.asarray(w))
    y = dequantize_mxfp4(qx, ex) @ dequantize_mxfp4(qw, ew).T + b
    return y.reshape(shp[:-1] + (w.shape[0],))


def linear_fp8(x, w, b):
    """fp8 linear: per-token e4m3 activations x per-channel e4m3 weights (R25, R26).

    Both operands are quantised with scale amax/448 and the product is taken
    on the dequantised values in fp64.
    """
    shp = x.shape
    x2 = x.reshape(-1, shp[-1])
    qx, sx = quantize_rows_e4m3(x2)
    y = linear_fp8_codes(qx, sx, w, b)
    return y.reshape(*shp[:-1], w.shape[0])


def linear_fp8_codes(qx, sx, w, b):
    """The product half of ``linear_fp8``: activations already quantised (e4m3
    values qx [M, K] with row scales sx [M]) times the per-channel e4m3 weight,
    dequantised, in fp64, plus the bias."""
    qw, sw = quantize_rows_e4m3(w)
    return (np.asarray(qx, np.float64) @ qw.T) * np.asarray(sx, np.float64)[:, None] \
        * sw.astype(np.float64)[None, :] + b


def p448_fp32_window(t, r, T, d):
    """Relative error bound of 448 P = 2^(t - r + log2 448) formed in fp32 (R43):
    t the score in log2 units, r the integer row reference, T the same score
    with every product taken in magnitude (sum_c |q_c k_c| scale log2 e), d the
    number of products.  Terms: the score summed in fp32 from exact products
    (d roundings of partial sums no larger than T), the fp32 score scale (4
    roundings of |t|), the fp32 reference minus log2 448 (the constant within
    2^-21, one rounding), one fused multiply-add and exp2 within 2 ulps; an
    error e in the exponent is a relative error ln 2 e of 448 P."""
    u = 2.0 ** -24
    l448 = math.log2(E4M3_MAX)
    arg = t - r + l448
    return math.log(2.0) * (d * u * T + 4 * u * np.abs(t) + u * np.abs(r - l448) + 2.0 ** -21
                            + u * np.abs(arg)) + 2 * u


def attention_fp8(q, k, v, scale: Optional[float] = None, rows=None,
                  tie_rel: Optional[float] = None, tie_fp32: bool = False):
    """fp8 attention (R27).

    Q, K and V each get one e4m3 scale per (batch, head), taken over that head's
    whole [L, d] slice, so the scales factor out of both products.  Scores use
    the dequantised operands.  With t = s * log2(e) and the row reference
    r = ceil(max_j t_j) (the row max rounded up to an integer in log2 units),
    P = 2^(t - r) lies in (0, 1] with its largest entry above 1/2; P enters the
    P V product as e4m3(448 P) / 448 and the normaliser is the row sum of that
    quantised P, so every row of weights sums to one.  A power-of-two reference
    makes the quantised weights independent of which integer r is used (short
    of e4m3's subnormal range).  Identical keys give equal weights, so the
    output is then the mean of the dequantised V.  ``rows`` restricts the
    output to those query rows (each row is independent of the others).

    Slack (returned as (out, slack) when a window is asked for): a first-order
    bound on how far the output moves when every P code whose 448 P lies within
    its window of an e4m3 rounding boundary rounds the other way -- the spread
    of equally valid results that an evaluation of 448 P in fp32 can give.  The
    window is either the constant relative width ``tie_rel``, or, with
    ``tie_fp32``, each score's own bound on the relative error of 448 P formed
    in fp32 (R43): the score summed from exact e4m3 products in fp32 (at most d
    roundings, each within u = 2^-24 of a partial sum no larger than
    sum_c |q_c k_c|), times the fp32 score scale (4 roundings of |t|), minus the
    reference shifted by log2 448 (an fp32 constant within 2^-21, one rounding
    of |r - log2 448|), one fused multiply-add (u |arg|) and an exp2 within 2
    ulps: rel = ln 2 (d u T + 4 u |t| + u |r - 8.8| + 2^-21 + u |arg|) + 2 u,
    T = scale log2(e) sum_c |q_c k_c| in the dequantised values.
    """
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    B, H, L, _ = q.shape
    sel = np.arange(L) if rows is None else np.asarray(rows)
    out = np.empty((B, H, len(sel), d))
    want_slack = tie_rel is not None or tie_fp32
    slack = np.zeros_like(out) if want_slack else None

    def deq(t):
        codes, sc = quantize_rows_e4m3(t.reshape(1, -1))
        return (codes * float(sc[0])).reshape(t.shape)

    for bi in range(B):
        for h in range(H):
            qd, kd, vd = deq(q[bi, h]), deq(k[bi, h]), deq(v[bi, h])
            t = (qd[sel] @ kd.T) * (scale / math.log(2.0))
            r = np.ceil(t.max(axis=1, keepdims=True))
            p = np.exp2(t - r)
            pq = round_e4m3(p * E4M3_MAX) / E4M3_MAX
            lq = pq.sum(axis=1, keepdims=True)
            out[bi, h] = (pq @ vd) / lq
            if want_slack:
                if tie_fp32:
                    T = (np.abs(qd[sel]) @ np.abs(kd).T) * (scale / math.log(2.0))
                    rel = p448_fp32_window(t, r, T, d)
                else:
                    rel = tie_rel
                # moving one weight by a step changes the output by step * (v_j - out) / l
                tie, step = e4m3_tie_mask(p * E4M3_MAX, rel)
                w = np.where(tie, step / E4M3_MAX, 0.0)
                slack[bi, h] = (w @ np.abs(vd) + w.sum(axis=1, keepdims=True)
                                * np.abs(out[bi, h])) / lq
    return out if slack is None else (out, slack)


# --------------------------------------------------------------------------
# blocks
# --------------------------------------------------------------------------

def _held(x, fp8):
    """fp8 blocks (R33): every activation between two steps of a bf16 model is
    stored in bf16, so one that is quantised to e4m3 later (Q, K, V, attention
    output, GELU output) is rounded to bf16 first and each e4m3 code is decided
    on that stored value."""
    return round_bf16(x) if fp8 else x


def _lin(x, P, name, fp8, mx4=False):
    if mx4:
        # MXFP4 blocks (R38): the input is stored bf16 before it is quantised
        return linear_mxfp4(round_bf16(x), P[name + ".w"], P[name + ".b"])
    if fp8:
        return linear_fp8(x, P[name + ".w"], P[name + ".b"])
    return linear(x, P[name + ".w"], P[name + ".b"])


def double_block(x_txt, x_img, mod_img, mod_txt, P, ang, H, fp8=False, mx4=False,
                 attn8=False):
    """Double-stream block (R1, R2, R4, R8): separate weights per stream, joint attention.

    x_txt [B, Lt, D], x_img [B, Li, D]; mod_* [B or 1, 6, D] in the order
    shift1, scale1, gate1, shift2, scale2, gate2; P keys "img.qkv.w" etc.;
    ang: RoPE angles [Lt + Li, d/2].  Returns the updated (x_txt, x_img).
    """
    a8 = fp8 or attn8        # e4m3 attention (R27), alone with MXFP4 linears (R40)
    attn_fn = attention_fp8 if a8 else attention
    Lt = x_txt.shape[1]
    streams = {"txt": (x_txt, mod_txt), "img": (x_img, mod_img)}
    qkv = {}
    for s, (x, m) in streams.items():
        u = modulate(x, m[:, 0:1], m[:, 1:2])
        qkv[s] = _lin(u, P, f"{s}.qkv", fp8, mx4)
    D = x_img.shape[-1]
    q = np.concatenate([qkv["txt"][..., :D], qkv["img"][..., :D]], axis=1)
    k = np.concatenate([qkv["txt"][..., D:2 * D], qkv["img"][..., D:2 * D]], axis=1)
    v = np.concatenate([qkv["txt"][..., 2 * D:], qkv["img"][..., 2 * D:]], axis=1)
    q = _held(apply_rope(_heads(q, H), ang), a8)
    k = _held(apply_rope(_heads(k, H), ang), a8)
    a = _held(_merge(attn_fn(q, k, _held(_heads(v, H), a8))), a8)
    out = {}
    for s, (x, m) in streams.items():
        a_s = a[:, :Lt] if s == "txt" else a[:, Lt:]
        x = x + m[:, 2:3] * _lin(a_s, P, f"{s}.proj", fp8, mx4)
        u = modulate(x, m[:, 3:4], m[:, 4:5])
        hdn = _held(gelu_tanh(_lin(u, P, f"{s}.mlp1", fp8, mx4)), fp8)
        x = x + m[:, 5:6] * _lin(hdn, P, f"{s}.mlp2", fp8, mx4)
        out[s] = x
    return out["txt"], out["img"]


def double_block_rows(x_txt, x_img, mod_img, mod_txt, P, ang, H, rows, fp8=False, mx4=False,
                      attn8=False):
    """The double block's output for the joint token rows ``rows`` only (text rows
    first, 0 <= row < Lt + Li) -> [B, len(rows), D].

    Every token's Q, K, V is computed (attention needs all keys and values, and
    fp8 scales span whole heads); attention, projection and MLP then run for the
    selected query rows alone: each row's update depends on its own row and the
    keys and values only, so the result equals ``double_block`` at those rows.
    """
    a8 = fp8 or attn8        # e4m3 attention (R27), alone with MXFP4 linears (R40)
    attn_fn = attention_fp8 if a8 else attention
    Lt = x_txt.shape[1]
    D = x_img.shape[-1]
    rows = np.asarray(rows)
    streams = {"txt": (x_txt, mod_txt), "img": (x_img, mod_img)}
    qkv = {}
    for s, (x, m) in streams.items():
        u = modulate(x, m[:, 0:1], m[:, 1:2])
        qkv[s] = _lin(u, P, f"{s}.qkv", fp8, mx4)
    q = np.concatenate([qkv["txt"][..., :D], qkv["img"][..., :D]], axis=1)
    k = np.concatenate([qkv["txt"][..., D:2 * D], qkv["img"][..., D:2 * D]], axis=1)
    v = np.concatenate([qkv["txt"][..., 2 * D:], qkv["img"][..., 2 * D:]], axis=1)
    q = _held(apply_rope(_heads(q, H), ang), a8)
    k = _held(apply_rope(_heads(k, H), ang), a8)
    vh = _held(_heads(v, H), a8)
    if a8:
        a = attn_fn(q, k, vh, rows=rows)
    else:
        a = attn_fn(q[:, :, rows], k, vh)
    a = _held(_merge(a), a8)                                  # [B, R, D]
    B = x_img.shape[0]
    out = np.empty((B, len(rows), D))
    for s, (x, m) in streams.items():
        sel = np.nonzero(rows < Lt)[0] if s == "txt" else np.nonzero(rows >= Lt)[0]
        if len(sel) == 0:
            continue
        tok = rows[sel] if s == "txt" else rows[sel] - Lt
        xs = x[:, tok]
        xs = xs + m[:, 2:3] * _lin(a[:, sel], P, f"{s}.proj", fp8, mx4)
        u = modulate(xs, m[:, 3:4], m[:, 4:5])
        hdn = _held(gelu_tanh(_lin(u, P, f"{s}.mlp1", fp8, mx4)), fp8)
        out[:, sel] = xs + m[:, 5:6] * _lin(hdn, P, f"{s}.mlp2", fp8, mx4)
    return out


def single_block(x, mod, P, ang, H, fp8=False, mx4=False, attn8=False):
    """Single-stream block (R10): one modulated LN feeding attention and MLP in parallel.

    x [B, L, D]; mod [B or 1, 3, D] = shift, scale, gate; P keys "lin1.w" ...
    """
    a8 = fp8 or attn8        # e4m3 attention (R27), alone with MXFP4 linears (R40)
    attn_fn = attention_fp8 if a8 else attention
    D = x.shape[-1]
    u = modulate(x, mod[:, 0:1], mod[:, 1:2])
    h = _lin(u, P, "lin1", fp8, mx4)
    q = _held(apply_rope(_heads(h[..., :D], H), ang), a8)
    k = _held(apply_rope(_heads(h[..., D:2 * D], H), ang), a8)
    v = _held(_heads(h[..., 2 * D:3 * D], H), a8)
    a = _merge(attn_fn(q, k, v))
    cat = _held(np.concatenate([a, gelu_tanh(h[..., 3 * D:])], axis=-1), fp8)
    return x + mod[:, 2:3] * _lin(cat, P, "lin2", fp8, mx4)


def single_block_rows(x, mod, P, ang, H, rows, fp8=False, mx4=False, attn8=False):
    """The single-stream block's output for the joint token rows ``rows`` only
    -> [B, len(rows), D].

    Every token's linear1 output is computed (attention needs all keys and
    values, and fp8 Q / K / V scales span whole heads); attention, the GELU half
    and linear2 then run for the selected rows alone.  A row's update depends on
    its own row and on the keys and values only, so the result equals
    ``single_block`` at those rows.
    """
    a8 = fp8 or attn8
    attn_fn = attention_fp8 if a8 else attention
    D = x.shape[-1]
    rows = np.asarray(rows)
    u = modulate(x, mod[:, 0:1], mod[:, 1:2])
    h = _lin(u, P, "lin1", fp8, mx4)
    q = _held(apply_rope(_heads(h[..., :D], H), ang), a8)
    k = _held(apply_rope(_heads(h[..., D:2 * D], H), ang), a8)
    v = _held(_heads(h[..., 2 * D:3 * D], H), a8)
    a = attn_fn(q, k, v, rows=rows) if a8 else attn_fn(q[:, :, rows], k, v)
    cat = _held(np.concatenate([_merge(a), gelu_tanh(h[:, rows, 3 * D:])], axis=-1), fp8)
    return x[:, rows] + mod[:, 2:3] * _lin(cat, P, "lin2", fp8, mx4)


def final_layer(x_img, shift, scale, w, b):
    """Velocity head (R11): Mod(x_img) W_out^T + b_out, image tokens only."""
    return linear(modulate(x_img, shift, scale), w, b)


# --------------------------------------------------------------------------
# First-Block-Cache (R18-R22), Euler (R14-R17)
# --------------------------------------------------------------------------

def fbcache_rel(r: np.ndarray, anchor: np.ndarray) -> float:
    """Relative L1 change of the first block's residual (R20), in fp64.

    sum|r - a| / sum|a|; a zero denominator gives +inf (never skips).
    """
    num = float(np.sum(np.abs(np.asarray(r, np.float64) - np.asarray(anchor, np.float64))))
    den = float(np.sum(np.abs(np.asarray(anchor, np.float64))))
    if den == 0.0:
        return math.inf if num == num else math.nan
    return num / den


def fbcache_decide(rel: float, threshold: float) -> bool:
    """Skip iff rel < threshold, strictly; NaN never skips (R20, R21)."""
    return bool(rel < threshold)


def fbcache_policy(test_skips: bool, steps_done: int, warmup_steps: int, skip_run: int,
                   max_skips: int) -> bool:
    """Skip policy on top of the rel test (R34, R35): a step whose test says skip
    still computes in full while it is one of the first ``warmup_steps`` steps taken
    with the cache, or when ``max_skips`` (> 0) steps in a row were just skipped."""
    if not test_skips:
        return False
    if steps_done < warmup_steps:
        return False
    if max_skips > 0 and skip_run >= max_skips:
        return False
    return True


def euler_update(x, v, sigma_i, sigma_next):
    """x <- x + (sigma_{i+1} - sigma_i) v, integrating sigma from 1 to 0 (R16)."""
    return x + (sigma_next - sigma_i) * v


def cfg_combine(v_pos, v_neg, g):
    """v_neg + g (v_pos - v_neg) (R17)."""
    return v_neg + g * (v_pos - v_neg)


class FBCacheState:
    """Caller-held First-Block-Cache state (anchor residual + cached tail residual,
    and the skip policy's counters)."""

    def __init__(self, enabled: bool, threshold: float, warmup_steps: int = 0,
                 max_skips: int = 0):
        self.enabled = enabled
        self.threshold = threshold
        self.has_anchor = False
        self.anchor = None     # first block's residual at the last full step
        self.cached = None     # final image hidden - image hidden after block 0
        self.warmup_steps = warmup_steps
        self.max_skips = max_skips
        self.steps_done = 0    # steps taken with the cache enabled
        self.skip_run = 0      # consecutive skipped steps ending at the last one


def _block_params(P, prefix):
    n = len(prefix) + 1
    return {k[n:]: v for k, v in P.items() if k.startswith(prefix + ".")}


def denoise_step(P, dims, w, lat, txt, i, sig, cache: Optional[FBCacheState] = None,
                 force_skip: Optional[bool] = None, fp8: bool = False,
                 mx4: bool = False, attn8: bool = False):
    """One flow-matching Euler step of the whole model (steps 1-11 of the oracle definition).

    P: parameters keyed as in ``dit_inputs.param_specs`` (fp64 arrays);
    w: the workload (B, grid, Lt, guidance); lat [1, Li, C_in]; txt [B, Lt, D].
    ``force_skip`` replays a decision taken elsewhere (decision replay).
    Returns (new latents, info dict with rel / skip / velocity).
    """
    D, H = dims.D, dims.H
    B = txt.shape[0]
    t = sig[i]
    c = time_embed(P, np.array([t]))                           # [1, D]
    ang = rope_table(image_positions(w.grid_h, w.grid_w, w.Lt), D // H)
    h_img = linear(lat, P["img_in.w"], P["img_in.b"])         # [1, Li, D]
    x_img = np.broadcast_to(h_img, (B,) + h_img.shape[1:]).copy()
    x_txt = txt.copy()
    before = x_img.copy()

    def mods(prefix, k):
        return modulation_vectors(c, P[prefix + ".mod.w"], P[prefix + ".mod.b"], D)

    info = {"rel": math.inf, "skip": False}
    for j in range(dims.n_double):
        bp = _block_params(P, f"double{j}")
        m_img = mods(f"double{j}.img", 6)
        m_txt = mods(f"double{j}.txt", 6)
        x_txt, x_img = double_block(x_txt, x_img, m_img, m_txt, bp, ang, H, fp8, mx4, attn8)
        if j == 0 and cache is not None and cache.enabled:
            r = x_img - before
            rel = fbcache_rel(r, cache.anchor) if cache.has_anchor else math.inf
            skip = fbcache_policy(fbcache_decide(rel, cache.threshold), cache.steps_done,
                                  cache.warmup_steps, cache.skip_run, cache.max_skips)
            if force_skip is not None:
                skip = bool(force_skip)
            info["rel"], info["skip"] = rel, skip
            cache.steps_done += 1
            cache.skip_run = cache.skip_run + 1 if skip else 0
            after0 = x_img.copy()
            if skip:
                break
    if info["skip"]:
        x_img = after0 + cache.cached
    else:
        if dims.n_single:
            x = np.concatenate([x_txt, x_img], axis=1)
            for j in range(dims.n_single):
                x = single_block(x, mods(f"single{j}", 3), _block_params(P, f"single{j}"),
                                 ang, H, fp8, mx4, attn8)
            x_img = x[:, w.Lt:]
        if cache is not None and cache.enabled:
            cache.cached = x_img - after0
            cache.anchor = r
            cache.has_anchor = True
    mf = mods("final", 2)
    v = final_layer(x_img, mf[:, 0:1], mf[:, 1:2], P["final.out.w"], P["final.out.b"])
    if B == 2 and w.guidance:
        v = cfg_combine(v[0:1], v[1:2], w.guidance)
    info["v"] = v
    return euler_update(lat, v, sig[i], sig[i + 1]), info
