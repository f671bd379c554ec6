"""ctypes binding of libdit (include/dit.h): argument marshalling only.

Every function here checks shapes and dtypes of torch tensors, turns them into
pointers and calls the C entry point of the same name.  All arithmetic runs in
the HIP kernels of libdit.so; importing this module fails if the library is
missing (build it with ``python -m image_generation_amd.build``).
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import POINTER, Structure, c_double, c_float, c_int, c_long, c_size_t, c_void_p
from typing import List, Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdit.so")

DIT_OK = 0
DIT_ERR_INVALID_ARG = -1
DIT_ERR_UNSUPPORTED = -2
DIT_ERR_WORKSPACE = -3
DIT_ERR_HIP = -4
DIT_ERR_NONFINITE = -5

DIT_F32, DIT_BF16, DIT_FP8, DIT_MXFP4, DIT_MXFP4_FP8ATTN = 0, 1, 2, 3, 4
DIT_BLOCK_DOUBLE, DIT_BLOCK_SINGLE = 0, 1
DIT_WS_ATTENTION, DIT_WS_BLOCK, DIT_WS_STEP, DIT_WS_MODULATION, DIT_WS_FBCACHE = range(5)
DIT_MOD_STATIC_BYTES = 8 << 20   # static scratch of dit_modulation_static (include/dit.h)


class DitDims(Structure):
    _fields_ = [("B", c_int), ("Lt", c_int), ("grid_h", c_int), ("grid_w", c_int),
                ("D", c_int), ("H", c_int), ("F", c_int)]


class DitLinear(Structure):
    _fields_ = [("w", c_void_p), ("b", c_void_p), ("w_scale", c_void_p), ("w_mx", c_void_p)]


class DitBlock(Structure):
    _fields_ = [("kind", c_int), ("qkv", DitLinear * 2), ("proj", DitLinear * 2),
                ("mlp1", DitLinear * 2), ("mlp2", DitLinear * 2),
                ("lin1", DitLinear), ("lin2", DitLinear)]


class DitBlockViews(Structure):
    _fields_ = [(n, c_void_p) for n in ("ln", "ln8", "ln_scale", "q", "k", "v", "q8", "k8", "v8",
                                        "qkv_scale", "cat", "cat8", "att_scale", "hid_scale")]


class DitModel(Structure):
    _fields_ = [("dims", DitDims), ("n_double", c_int), ("n_single", c_int),
                ("blocks", POINTER(DitBlock)), ("time1", DitLinear), ("time2", DitLinear),
                ("img_in", DitLinear), ("final_out", DitLinear), ("mod", DitLinear),
                ("C_in", c_int), ("guidance", c_float), ("dtype", c_int)]


class DitFBCache(Structure):
    _fields_ = [("enabled", c_int), ("threshold", c_float), ("has_anchor", c_int),
                ("anchor", c_void_p), ("cached", c_void_p), ("warmup_steps", c_int),
                ("max_skips", c_int), ("steps_done", c_int), ("skip_run", c_int)]


class DitStepInfo(Structure):
    _fields_ = [("rel", c_double), ("skipped", c_int)]


class DitKernelTimer(Structure):
    _fields_ = [("site_mask", ctypes.c_uint), ("capacity", c_int), ("count", c_int),
                ("sites", POINTER(c_int)), ("start", POINTER(c_void_p)),
                ("stop", POINTER(c_void_p))]


SITES = ("attention", "gemm_qkv", "gemm_resid", "gemm_gelu", "gemm_lin1", "gemm_f32",
         "gemm_silu", "ln", "fbc", "other", "quant")


class DitError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libdit status {status}: {msg}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m image_generation_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P = c_void_p
    sig = {
        "dit_status_string": (ctypes.c_char_p, [c_int]),
        "dit_last_error": (ctypes.c_char_p, []),
        "dit_workspace_bytes": (c_size_t, [POINTER(DitDims), c_int, c_int]),
        "dit_sigmas": (c_int, [c_int, c_double, POINTER(c_double)]),
        "dit_rope_table": (c_int, [c_int, c_int, c_int, c_int, c_double, P, P]),
        "dit_attention": (c_int, [P, P, P, P, P, P, P, c_int, c_int, c_int, c_int, c_int, c_float,
                                  P]),
        "dit_quantize_rows": (c_int, [P, c_int, c_int, c_int, c_int, P, c_int, P, P]),
        "dit_block_forward": (c_int, [POINTER(DitDims), POINTER(DitBlock), c_int, P, c_int, P,
                                      c_long, P, P, c_size_t, P]),
        "dit_modulation": (c_int, [POINTER(DitModel), POINTER(c_double), c_int, P, P, c_size_t, P]),
        "fbcache_should_skip": (c_int, [P, P, P, P, c_int, c_int, c_int, c_int, c_float, c_int,
                                        P, c_size_t, P, POINTER(c_double), POINTER(c_int)]),
        "dit_denoise_step": (c_int, [POINTER(DitModel), P, P, P, c_double, c_double,
                                     POINTER(DitFBCache), P, c_size_t, P, POINTER(DitStepInfo)]),
        "dit_denoise_step_at": (c_int, [POINTER(DitModel), P, P, c_int, c_int, POINTER(c_double),
                                        POINTER(DitFBCache), P, c_size_t, P,
                                        POINTER(DitStepInfo)]),
        "dit_step_at_workspace_bytes": (c_size_t, [POINTER(DitModel)]),
        "dit_set_kernel_timer": (c_int, [POINTER(DitKernelTimer)]),
        "dit_linear_forward": (c_int, [P, c_int, c_int, POINTER(DitLinear), c_int, P, c_int, P]),
        "dit_quantize_mxfp4": (c_int, [P, c_int, c_int, c_int, c_int, P, P, P]),
        "dit_mx_rows": (c_int, [c_int]),
        "dit_linear_mxfp4": (c_int, [P, P, c_int, c_int, P, P, P, c_int, P, c_int, P]),
        "dit_loop_state_bytes": (c_size_t, [POINTER(DitModel), c_int]),
        "dit_loop_graph_create": (c_int, [POINTER(DitModel), P, P, P, POINTER(c_double), c_int,
                                          POINTER(DitFBCache), P, c_size_t, P, c_size_t, P,
                                          POINTER(P)]),
        "dit_loop_graph_run": (c_int, [P, c_int, P]),
        "dit_loop_graph_sync": (c_int, [P, POINTER(DitFBCache), POINTER(DitStepInfo), c_int, P,
                                        POINTER(c_int)]),
        "dit_loop_graph_reset": (c_int, [P, POINTER(DitFBCache), c_int, P]),
        "dit_loop_graph_destroy": (c_int, [P]),
        "dit_modulation_static": (c_int, [POINTER(DitModel), POINTER(c_double), c_int, P, P]),
        "dit_block_views_of": (c_int, [POINTER(DitDims), P, c_size_t, POINTER(DitBlockViews)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()
EXPORTED = ("dit_status_string", "dit_last_error", "dit_workspace_bytes", "dit_sigmas",
            "dit_rope_table", "dit_attention", "dit_block_forward", "dit_modulation",
            "fbcache_should_skip", "dit_denoise_step", "dit_set_kernel_timer", "dit_linear_forward",
            "dit_quantize_rows", "dit_quantize_mxfp4", "dit_mx_rows", "dit_linear_mxfp4",
            "dit_loop_state_bytes", "dit_loop_graph_create", "dit_loop_graph_run",
            "dit_loop_graph_sync", "dit_loop_graph_reset", "dit_loop_graph_destroy",
            "dit_modulation_static", "dit_block_views_of", "dit_denoise_step_at",
            "dit_step_at_workspace_bytes")


def _check(rc: int) -> None:
    if rc != DIT_OK:
        raise DitError(rc, LIB.dit_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libdit must be contiguous")
    return t.data_ptr()


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t: torch.Tensor, dtype: torch.dtype, shape: Sequence[int], name: str) -> None:
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_cuda:
        raise ValueError(f"{name}: expected {dtype} {tuple(shape)} on the GPU, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def dims_of(B: int, Lt: int, grid_h: int, grid_w: int, D: int, H: int, F: int) -> DitDims:
    return DitDims(B, Lt, grid_h, grid_w, D, H, F)


# ------------------------------------------------------------------ helpers

def dit_workspace_bytes(dims: DitDims, purpose: int, n_steps: int = 0) -> int:
    return int(LIB.dit_workspace_bytes(ctypes.byref(dims), purpose, n_steps))


def workspace(dims: DitDims, purpose: int, n_steps: int = 0, device="cuda") -> torch.Tensor:
    n = dit_workspace_bytes(dims, purpose, n_steps)
    if n == 0 and purpose != DIT_WS_ATTENTION:
        raise DitError(DIT_ERR_INVALID_ARG, "invalid dims for the workspace query")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def dit_sigmas(n_steps: int, shift: float) -> List[float]:
    out = (c_double * (n_steps + 1))()
    _check(LIB.dit_sigmas(n_steps, float(shift), out))
    return list(out)


def dit_rope_table(grid_h: int, grid_w: int, Lt: int, head_dim: int, theta: float = 10000.0,
                   device="cuda", stream=None) -> torch.Tensor:
    tab = torch.empty((Lt + grid_h * grid_w, head_dim // 2, 2), dtype=torch.float32, device=device)
    _check(LIB.dit_rope_table(grid_h, grid_w, Lt, head_dim, float(theta), _ptr(tab),
                              _stream(stream)))
    return tab


# ------------------------------------------------------------------ entry points

def _codes(t: torch.Tensor, shape, name: str) -> None:
    """e4m3 codes: uint8 (raw bytes) or torch.float8_e4m3fn."""
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn) or tuple(t.shape) != tuple(shape) \
            or not t.is_cuda:
        raise ValueError(f"{name}: expected e4m3 codes (uint8) {tuple(shape)} on the GPU, "
                         f"got {t.dtype} {tuple(t.shape)}")


def dit_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                  softmax_scale: Optional[float] = None, q_scale: Optional[torch.Tensor] = None,
                  k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """q, k, v [B, H, L, d] (any L >= 1), o [B, L, H*d] (written).
    bf16: q, k, v bf16, d 64 or 128, o bf16.
    fp8: q, k, v e4m3 codes (d 64 or 128), scales fp32 [B, H], o bf16.
    fp32: q, k, v fp32 (d 32 or 64), o fp32."""
    B, H, L, d = q.shape
    fp8 = q.dtype in (torch.uint8, torch.float8_e4m3fn)
    f32 = q.dtype == torch.float32
    if f32:
        for n_, t_ in (("q", q), ("k", k), ("v", v)):
            _need(t_, torch.float32, (B, H, L, d), n_)
        _need(o, torch.float32, (B, L, H * d), "o")
    elif fp8:
        for n_, t_ in (("q", q), ("k", k), ("v", v)):
            _codes(t_, (B, H, L, d), n_)
        for n_, t_ in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
            if t_ is None:
                raise ValueError(f"{n_} is required for fp8 attention")
            _need(t_, torch.float32, (B, H), n_)
    else:
        for n_, t_ in (("q", q), ("k", k), ("v", v)):
            _need(t_, torch.bfloat16, (B, H, L, d), n_)
    if not f32:
        _need(o, torch.bfloat16, (B, L, H * d), "o")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    _check(LIB.dit_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(q_scale), _ptr(k_scale),
                             _ptr(v_scale), B, H, L, d,
                             DIT_F32 if f32 else DIT_FP8 if fp8 else DIT_BF16,
                             float(softmax_scale), _stream(stream)))
    return o


def dit_quantize_rows(src: torch.Tensor, stream=None):
    """Per-row e4m3 quantisation of a bf16 [rows, width] tensor -> (codes uint8, scale fp32 [rows])."""
    if src.dim() != 2 or src.dtype != torch.bfloat16 or not src.is_cuda:
        raise ValueError("src: bf16 [rows, width] on the GPU")
    rows, width = src.shape
    codes = torch.empty((rows, width), dtype=torch.uint8, device=src.device)
    scale = torch.empty((rows,), dtype=torch.float32, device=src.device)
    _check(LIB.dit_quantize_rows(_ptr(src), DIT_BF16, width, rows, width, _ptr(codes), width,
                                 _ptr(scale), _stream(stream)))
    return codes, scale


def dit_quantize_mxfp4(src: torch.Tensor, stream=None):
    """MXFP4 quantisation of a bf16 or fp32 [rows, width] tensor along its rows ->
    (codes uint8 [rows, width / 2], scales uint8 [width / 256, dit_mx_rows(rows), 8])."""
    if src.dim() != 2 or src.dtype not in (torch.bfloat16, torch.float32) or not src.is_cuda:
        raise ValueError("src: bf16 or fp32 [rows, width] on the GPU")
    if not src.is_contiguous():
        raise ValueError("src: contiguous")
    rows, width = src.shape
    codes = torch.empty((rows, width // 2), dtype=torch.uint8, device=src.device)
    scales = torch.empty((width // 256, LIB.dit_mx_rows(rows), 8), dtype=torch.uint8,
                         device=src.device)
    dt = DIT_BF16 if src.dtype == torch.bfloat16 else DIT_F32
    _check(LIB.dit_quantize_mxfp4(_ptr(src), dt, width, rows, width, _ptr(codes), _ptr(scales),
                                  _stream(stream)))
    return codes, scales


def dit_linear_mxfp4(xq, w_q, b: Optional[torch.Tensor], out: torch.Tensor, stream=None):
    """W4A4 y = x W^T + b; xq, w_q: (codes, scales) pairs from dit_quantize_mxfp4;
    out fp32 or bf16 [M, N]."""
    xc, xs = xq
    wc, ws = w_q
    M, N, K = xc.shape[0], wc.shape[0], xc.shape[1] * 2
    if wc.shape[1] * 2 != K or tuple(out.shape) != (M, N):
        raise ValueError("dit_linear_mxfp4: shape mismatch")
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out: fp32 or bf16")
    if b is not None:
        _need(b, torch.float32, (N,), "b")
    yd = DIT_F32 if out.dtype == torch.float32 else DIT_BF16
    _check(LIB.dit_linear_mxfp4(_ptr(xc), _ptr(xs), M, K, _ptr(wc), _ptr(ws), _ptr(b), N,
                                _ptr(out), yd, _stream(stream)))
    return out


def dit_linear_forward(x: torch.Tensor, w: torch.Tensor, b: torch.Tensor,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = x W^T + b: x [M, K] bf16, w [N, K] bf16, b [N] fp32 -> y [M, N] (fp32 or bf16)."""
    M, K = x.shape
    N = w.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    _need(w, torch.bfloat16, (N, K), "w")
    _need(b, torch.float32, (N,), "b")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if tuple(out.shape) != (M, N) or out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out: fp32 or bf16 [M, N]")
    lin = DitLinear(_ptr(w), _ptr(b), None)
    yd = DIT_F32 if out.dtype == torch.float32 else DIT_BF16
    _check(LIB.dit_linear_forward(_ptr(x), M, K, ctypes.byref(lin), N, _ptr(out), yd, _stream(stream)))
    return out


def _lin(w: torch.Tensor, b: torch.Tensor, w_scale: Optional[torch.Tensor] = None,
         w_mx: Optional[torch.Tensor] = None) -> DitLinear:
    """bf16 layer (w_scale None), e4m3 layer (w uint8 codes, w_scale fp32 [out]) or
    MXFP4 layer (w uint8 E2M1 codes [out, in / 2], w_mx its E8M0 block scales)."""
    if b.dtype != torch.float32 or not (w.is_cuda and b.is_cuda):
        raise ValueError("linear: bias fp32, tensors on the GPU")
    if w_mx is not None:
        N, K2 = w.shape
        if w.dtype != torch.uint8 or w_mx.dtype != torch.uint8 or \
                tuple(w_mx.shape) != (2 * K2 // 256, LIB.dit_mx_rows(N), 8):
            raise ValueError("linear: mxfp4 layer needs E2M1 codes and their block scales")
        return DitLinear(_ptr(w), _ptr(b), None, _ptr(w_mx))
    if w_scale is None:
        if w.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("linear: bf16 (or fp32) weight expected")
    elif w.dtype not in (torch.uint8, torch.float8_e4m3fn) or w_scale.dtype != torch.float32 \
            or tuple(w_scale.shape) != (w.shape[0],):
        raise ValueError("linear: fp8 layer needs e4m3 codes and an fp32 scale per output")
    return DitLinear(_ptr(w), _ptr(b), _ptr(w_scale), None)


def _lin_of(p: dict, name: str) -> DitLinear:
    return _lin(p[name + ".w"], p[name + ".b"], p.get(name + ".w_scale"), p.get(name + ".w_mx"))


def make_double_block(p: dict, prefix: str = "") -> DitBlock:
    """p: '<prefix>img.qkv.w' ... device tensors (weights bf16, biases fp32); an fp8
    layer also has '<name>.w_scale' and its '.w' holds the e4m3 codes."""
    blk = DitBlock()
    blk.kind = DIT_BLOCK_DOUBLE
    for i, s in enumerate(("img", "txt")):
        blk.qkv[i] = _lin_of(p, f"{prefix}{s}.qkv")
        blk.proj[i] = _lin_of(p, f"{prefix}{s}.proj")
        blk.mlp1[i] = _lin_of(p, f"{prefix}{s}.mlp1")
        blk.mlp2[i] = _lin_of(p, f"{prefix}{s}.mlp2")
    return blk


def make_single_block(p: dict, prefix: str = "") -> DitBlock:
    blk = DitBlock()
    blk.kind = DIT_BLOCK_SINGLE
    blk.lin1 = _lin_of(p, f"{prefix}lin1")
    blk.lin2 = _lin_of(p, f"{prefix}lin2")
    return blk


def quantize_block_params(p: dict, prefix: str = "", stream=None) -> dict:
    """Copy of p with every block linear under prefix replaced by its e4m3 codes
    and per-output-channel scales (computed by dit_quantize_rows on the GPU)."""
    out = dict(p)
    for name in list(p):
        if not name.startswith(prefix) or not name.endswith(".w") or ".mod." in name:
            continue
        codes, scale = dit_quantize_rows(p[name], stream)
        out[name] = codes
        out[name + "_scale"] = scale
    return out


def quantize_block_params_mx(p: dict, prefix: str = "", stream=None) -> dict:
    """Copy of p with every block linear under prefix replaced by its MXFP4 (E2M1)
    codes and E8M0 block scales '<name>.w_mx' (dit_quantize_mxfp4 on the GPU)."""
    out = dict(p)
    for name in list(p):
        if not name.startswith(prefix) or not name.endswith(".w") or ".mod." in name:
            continue
        codes, scales = dit_quantize_mxfp4(p[name], stream)
        out[name] = codes
        out[name + "_mx"] = scales
    return out


def dit_block_forward(dims: DitDims, blk: DitBlock, x: torch.Tensor, mod: torch.Tensor,
                      rope: torch.Tensor, ws: torch.Tensor, mod_bstride: Optional[int] = None,
                      dtype: int = DIT_BF16, stream=None) -> torch.Tensor:
    """x [B, L, D] (fp32 or bf16) updated in place; mod [B or 1, k, D] fp32.
    dtype DIT_BF16; DIT_FP8 for a block built from quantize_block_params(); DIT_MXFP4 or
    DIT_MXFP4_FP8ATTN (e4m3 attention) for one built from quantize_block_params_mx()."""
    L = dims.Lt + dims.grid_h * dims.grid_w
    if tuple(x.shape) != (dims.B, L, dims.D) or x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"x: expected fp32/bf16 {(dims.B, L, dims.D)}, got {x.dtype} {tuple(x.shape)}")
    nk = 12 if blk.kind == DIT_BLOCK_DOUBLE else 3
    if mod.dtype != torch.float32 or mod.shape[-2:] != (nk, dims.D) or mod.shape[0] not in (1, dims.B):
        raise ValueError(f"mod: expected fp32 [B or 1, {nk}, {dims.D}]")
    if mod_bstride is None:
        mod_bstride = 0 if mod.shape[0] == 1 else nk * dims.D
    xd = DIT_F32 if x.dtype == torch.float32 else DIT_BF16
    _check(LIB.dit_block_forward(ctypes.byref(dims), ctypes.byref(blk), dtype, _ptr(x), xd,
                                 _ptr(mod), int(mod_bstride), _ptr(rope), _ptr(ws), ws.numel(),
                                 _stream(stream)))
    return x


def fbcache_should_skip(x_after: torch.Tensor, x_before: torch.Tensor,
                        anchor: Optional[torch.Tensor], staging: torch.Tensor, Lt: int,
                        threshold: float, has_anchor: bool, ws: torch.Tensor, stream=None):
    """x_after [B, Lt+Li, D] fp32; x_before, anchor, staging [B, Li, D] fp32.  -> (rel, skip)."""
    B, Li, D = x_before.shape
    _need(x_after, torch.float32, (B, Lt + Li, D), "x_after")
    _need(x_before, torch.float32, (B, Li, D), "x_before")
    _need(staging, torch.float32, (B, Li, D), "staging")
    if anchor is not None:
        _need(anchor, torch.float32, (B, Li, D), "anchor")
    rel = c_double()
    skip = c_int()
    _check(LIB.fbcache_should_skip(_ptr(x_after), _ptr(x_before), _ptr(anchor), _ptr(staging),
                                   B, Lt, Li, D, float(threshold), int(bool(has_anchor)), _ptr(ws),
                                   ws.numel(), _stream(stream), ctypes.byref(rel),
                                   ctypes.byref(skip)))
    return rel.value, bool(skip.value)


class GPUModel:
    """Device copy of a whole model plus the ctypes struct that points into it.

    params: name -> tensor in the enumeration of ``dit_inputs.param_specs``
    (weights bf16, biases any float dtype; moved to the GPU here).
    """

    def __init__(self, dims, B: int, Lt: int, grid_h: int, grid_w: int, params: dict,
                 guidance: float = 0.0, device="cuda", dtype: int = DIT_BF16):
        self.dims_py = dims
        D = dims.D
        self.n_double, self.n_single = dims.n_double, dims.n_single
        self.t = {}
        wdt = torch.float32 if dtype == DIT_F32 else torch.bfloat16
        for name, t in params.items():
            if name.rsplit(".", 1)[-1].startswith("b"):      # b, b1, b2: biases
                self.t[name] = t.to(device=device, dtype=torch.float32).contiguous()
            elif name.endswith(".mod.w"):
                continue
            else:
                self.t[name] = t.to(device=device, dtype=wdt).contiguous()
        # stacked modulation weights in the order the library expects
        order = []
        for j in range(self.n_double):
            order += [f"double{j}.img.mod", f"double{j}.txt.mod"]
        order += [f"single{j}.mod" for j in range(self.n_single)]
        order += ["final.mod"]
        self.mod_w = torch.cat([params[n + ".w"].to(device=device, dtype=wdt)
                                for n in order]).contiguous()
        self.mod_b = torch.cat([self.t[n + ".b"] for n in order]).contiguous()
        self.n_mod = self.mod_w.shape[0]
        assert self.n_mod == (12 * self.n_double + 3 * self.n_single + 2) * D
        if dtype == DIT_FP8:
            # block linears in e4m3 with per-channel scales; the rest stays bf16
            q = {}
            for pre in [f"double{j}." for j in range(self.n_double)] + \
                       [f"single{j}." for j in range(self.n_single)]:
                q.update(quantize_block_params({n: t for n, t in self.t.items()
                                                if n.startswith(pre)}, pre))
            for n, t in q.items():
                self.t[n] = t
        elif dtype in (DIT_MXFP4, DIT_MXFP4_FP8ATTN):
            # block linears W4A4 in MXFP4; the rest stays bf16
            q = {}
            for pre in [f"double{j}." for j in range(self.n_double)] + \
                       [f"single{j}." for j in range(self.n_single)]:
                q.update(quantize_block_params_mx({n: t for n, t in self.t.items()
                                                   if n.startswith(pre)}, pre))
            for n, t in q.items():
                self.t[n] = t
        elif dtype not in (DIT_BF16, DIT_F32):
            raise ValueError(f"model dtype {dtype}")
        self.dtype = dtype
        blocks = [make_double_block(self.t, f"double{j}.") for j in range(self.n_double)]
        blocks += [make_single_block(self.t, f"single{j}.") for j in range(self.n_single)]
        self._blocks = (DitBlock * max(1, len(blocks)))(*blocks)
        m = DitModel()
        m.dims = dims_of(B, Lt, grid_h, grid_w, D, dims.H, dims.F)
        m.n_double, m.n_single = self.n_double, self.n_single
        m.blocks = ctypes.cast(self._blocks, POINTER(DitBlock))
        m.time1 = _lin(self.t["time.w1"], self.t["time.b1"])
        m.time2 = _lin(self.t["time.w2"], self.t["time.b2"])
        m.img_in = _lin(self.t["img_in.w"], self.t["img_in.b"])
        m.final_out = _lin(self.t["final.out.w"], self.t["final.out.b"])
        m.mod = _lin(self.mod_w, self.mod_b)
        m.C_in = dims.C_in
        m.guidance = float(guidance)
        m.dtype = dtype
        self.model = m


def dit_modulation(gm: GPUModel, sigmas: Sequence[float], out: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    n = len(sigmas)
    if out is None:
        out = torch.empty((n, gm.n_mod), dtype=torch.float32, device="cuda")
    _need(out, torch.float32, (n, gm.n_mod), "out")
    if ws is None:
        ws = workspace(gm.model.dims, DIT_WS_MODULATION, n)
    sig = (c_double * n)(*[float(s) for s in sigmas])
    _check(LIB.dit_modulation(ctypes.byref(gm.model), sig, n, _ptr(out), _ptr(ws), ws.numel(),
                              _stream(stream)))
    return out


def block_views(dd: DitDims, ws: torch.Tensor) -> dict:
    """Tensor views of a block workspace's intermediates (see dit_block_views in
    include/dit.h), as torch tensors sharing the workspace's memory."""
    v = DitBlockViews()
    _check(LIB.dit_block_views_of(ctypes.byref(dd), _ptr(ws), ws.numel(), ctypes.byref(v)))
    B, L, D, H, F = dd.B, dd.Lt + dd.grid_h * dd.grid_w, dd.D, dd.H, dd.F
    d = D // H
    base = ws.data_ptr()

    def view(ptr, dtype, shape):
        n = 1
        for s_ in shape:
            n *= s_
        es = torch.empty((), dtype=dtype).element_size()
        off = ptr - base
        return ws[off:off + n * es].view(dtype).view(shape)

    rows = B * L
    return {
        "ln": view(v.ln, torch.bfloat16, (rows, D)),
        "ln8": view(v.ln8, torch.uint8, (rows, D)),
        "ln_scale": view(v.ln_scale, torch.float32, (rows,)),
        "q": view(v.q, torch.bfloat16, (B, H, L, d)),
        "k": view(v.k, torch.bfloat16, (B, H, L, d)),
        "v": view(v.v, torch.bfloat16, (B, H, L, d)),
        "q8": view(v.q8, torch.uint8, (B, H, L, d)),
        "k8": view(v.k8, torch.uint8, (B, H, L, d)),
        "v8": view(v.v8, torch.uint8, (B, H, L, d)),
        "qkv_scale": view(v.qkv_scale, torch.float32, (3, B, H)),
        "cat": view(v.cat, torch.bfloat16, (rows, D + F)),
        "cat8": view(v.cat8, torch.uint8, (rows, D + F)),
        "att_scale": view(v.att_scale, torch.float32, (rows,)),
        "hid_scale": view(v.hid_scale, torch.float32, (rows,)),
    }


def dit_modulation_static(gm: GPUModel, sigmas: Sequence[float], out: torch.Tensor,
                          stream=None) -> torch.Tensor:
    """dit_modulation without a workspace: the library's static device scratch
    holds the intermediates.  ``out`` is caller-allocated (fp32 [n, N_mod])."""
    n = len(sigmas)
    _need(out, torch.float32, (n, gm.n_mod), "out")
    sig = (c_double * n)(*[float(s) for s in sigmas])
    _check(LIB.dit_modulation_static(ctypes.byref(gm.model), sig, n, _ptr(out), _stream(stream)))
    return out


class FBCache:
    """Caller-held First-Block-Cache state (device buffers + the ctypes struct)."""

    def __init__(self, B: int, Li: int, D: int, threshold: float, enabled: bool = True,
                 device="cuda", warmup_steps: int = 0, max_skips: int = 0):
        self.anchor = torch.zeros((B, Li, D), dtype=torch.float32, device=device)
        self.cached = torch.zeros((B, Li, D), dtype=torch.float32, device=device)
        self.c = DitFBCache(int(enabled), float(threshold), 0, _ptr(self.anchor), _ptr(self.cached),
                            int(warmup_steps), int(max_skips), 0, 0)

    @property
    def has_anchor(self) -> bool:
        return bool(self.c.has_anchor)

    @property
    def steps_done(self) -> int:
        return int(self.c.steps_done)

    @property
    def skip_run(self) -> int:
        return int(self.c.skip_run)


def dit_denoise_step(gm: GPUModel, mod_step: torch.Tensor, txt: torch.Tensor,
                     latents: torch.Tensor, sigma: float, sigma_next: float,
                     cache: Optional[FBCache], ws: torch.Tensor, stream=None):
    """One Euler step in place on latents [Li, C_in] fp32; txt bf16 (fp32 for an fp32
    model).  -> (rel, skipped)."""
    dm = gm.model.dims
    Li = dm.grid_h * dm.grid_w
    _need(mod_step, torch.float32, (gm.n_mod,), "mod_step")
    _need(txt, torch.float32 if gm.dtype == DIT_F32 else torch.bfloat16, (dm.B, dm.Lt, dm.D),
          "txt")
    _need(latents, torch.float32, (Li, gm.model.C_in), "latents")
    info = DitStepInfo()
    cp = ctypes.byref(cache.c) if cache is not None else None
    _check(LIB.dit_denoise_step(ctypes.byref(gm.model), _ptr(mod_step), _ptr(txt), _ptr(latents),
                                float(sigma), float(sigma_next), cp, _ptr(ws), ws.numel(),
                                _stream(stream), ctypes.byref(info)))
    return info.rel, bool(info.skipped)


def step_at_workspace(gm: GPUModel, device=None) -> torch.Tensor:
    """A device workspace of dit_step_at_workspace_bytes(model) bytes."""
    nb = int(LIB.dit_step_at_workspace_bytes(ctypes.byref(gm.model)))
    if nb == 0:
        raise ValueError("dit_step_at_workspace_bytes rejected the model")
    return torch.empty(nb, dtype=torch.uint8, device=device or "cuda")


def dit_denoise_step_at(gm: GPUModel, txt: torch.Tensor, latents: torch.Tensor, step: int,
                        sigmas: Sequence[float], cache: Optional[FBCache], ws: torch.Tensor,
                        stream=None):
    """Step `step` of the schedule `sigmas` (n_steps + 1 entries) in place on latents,
    computing that step's modulation vectors itself.  -> (rel, skipped)."""
    dm = gm.model.dims
    Li = dm.grid_h * dm.grid_w
    _need(txt, torch.float32 if gm.dtype == DIT_F32 else torch.bfloat16, (dm.B, dm.Lt, dm.D),
          "txt")
    _need(latents, torch.float32, (Li, gm.model.C_in), "latents")
    n = len(sigmas) - 1
    sig = (c_double * len(sigmas))(*[float(x) for x in sigmas])
    info = DitStepInfo()
    cp = ctypes.byref(cache.c) if cache is not None else None
    _check(LIB.dit_denoise_step_at(ctypes.byref(gm.model), _ptr(latents), _ptr(txt), int(step), n,
                                   sig, cp, _ptr(ws), ws.numel(), _stream(stream),
                                   ctypes.byref(info)))
    return info.rel, bool(info.skipped)


class LoopGraph:
    """A denoise loop captured as one HIP graph per step and replayed with the
    First-Block-Cache decision kept on the device (dit_loop_graph_*).

    mod_all [n_steps, N_mod] fp32 (dit_modulation over sigmas[:-1]); sigmas: the
    n_steps + 1 schedule; txt, latents as for dit_denoise_step; cache: FBCache or
    None.  The workspace and loop state are allocated here and kept with the
    graph, as are references to every tensor it points into."""

    def __init__(self, gm: GPUModel, mod_all: torch.Tensor, txt: torch.Tensor,
                 latents: torch.Tensor, sigmas: Sequence[float], cache: Optional[FBCache] = None,
                 stream=None):
        n = len(sigmas) - 1
        dm = gm.model.dims
        Li = dm.grid_h * dm.grid_w
        _need(mod_all, torch.float32, (n, gm.n_mod), "mod_all")
        _need(txt, torch.float32 if gm.dtype == DIT_F32 else torch.bfloat16, (dm.B, dm.Lt, dm.D),
              "txt")
        _need(latents, torch.float32, (Li, gm.model.C_in), "latents")
        self.n_steps = n
        self.ws = workspace(dm, DIT_WS_STEP)
        nb = LIB.dit_loop_state_bytes(ctypes.byref(gm.model), n)
        if nb == 0:
            raise ValueError("dit_loop_state_bytes rejected the model or step count")
        self.state = torch.empty(nb, dtype=torch.uint8, device=latents.device)
        self._keep = (gm, mod_all, txt, latents, cache)
        self.cache = cache
        sig = (c_double * (n + 1))(*[float(x) for x in sigmas])
        h = c_void_p()
        cp = ctypes.byref(cache.c) if cache is not None else None
        _check(LIB.dit_loop_graph_create(ctypes.byref(gm.model), _ptr(mod_all), _ptr(txt),
                                         _ptr(latents), sig, n, cp, _ptr(self.ws), self.ws.numel(),
                                         _ptr(self.state), self.state.numel(), _stream(stream),
                                         ctypes.byref(h)))
        self.h = h
        self.launched = 0

    def run(self, n: Optional[int] = None, stream=None) -> None:
        """Enqueue n replays (default: the rest of the loop); returns at once."""
        if n is None:
            n = self.n_steps - self.launched
        _check(LIB.dit_loop_graph_run(self.h, int(n), _stream(stream)))
        self.launched += int(n)

    def sync(self, stream=None):
        """Wait for the replays; -> (steps completed, [(rel, skipped)] per step).
        The FBCache's counters are updated."""
        n = self.n_steps
        info = (DitStepInfo * n)()
        done = c_int(0)
        cp = ctypes.byref(self.cache.c) if self.cache is not None else None
        _check(LIB.dit_loop_graph_sync(self.h, cp, info, n, _stream(stream), ctypes.byref(done)))
        return int(done.value), [(info[i].rel, bool(info[i].skipped)) for i in range(n)]

    def reset(self, first_step: int = 0, stream=None) -> None:
        """Restart at first_step with the FBCache's current counters."""
        cp = ctypes.byref(self.cache.c) if self.cache is not None else None
        _check(LIB.dit_loop_graph_reset(self.h, cp, int(first_step), _stream(stream)))
        self.launched = int(first_step)

    def close(self) -> None:
        if getattr(self, "h", None) is not None and self.h.value is not None:
            torch.cuda.synchronize()
            _check(LIB.dit_loop_graph_destroy(self.h))
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------ launch timing

class KernelTimer:
    """HIP events recorded by libdit around launches of the selected sites.

    Events are created through the HIP runtime (libamdhip64) directly, so they
    bracket the kernels on whatever stream the library launches them on.
    """

    def __init__(self, sites: Sequence[str], capacity: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [POINTER(c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [POINTER(c_float), c_void_p, c_void_p]
        self.hip.hipEventDestroy.argtypes = [c_void_p]
        self.capacity = capacity
        self.start = (c_void_p * capacity)()
        self.stop = (c_void_p * capacity)()
        self.sites = (c_int * capacity)()
        for i in range(capacity):
            for arr in (self.start, self.stop):
                ev = c_void_p()
                if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                    raise DitError(DIT_ERR_HIP, "hipEventCreate failed")
                arr[i] = ev
        mask = 0
        for s_ in sites:
            mask |= 1 << SITES.index(s_)
        self.t = DitKernelTimer(mask, capacity, 0, self.sites,
                                ctypes.cast(self.start, POINTER(c_void_p)),
                                ctypes.cast(self.stop, POINTER(c_void_p)))

    def __enter__(self):
        self.t.count = 0
        _check(LIB.dit_set_kernel_timer(ctypes.byref(self.t)))
        return self

    def __exit__(self, *exc):
        _check(LIB.dit_set_kernel_timer(None))

    def durations_ms(self):
        """[(site name, ms)] of the recorded launches (call after synchronising)."""
        out = []
        for i in range(self.t.count):
            ms = c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.start[i], self.stop[i]) != 0:
                raise DitError(DIT_ERR_HIP, "hipEventElapsedTime failed")
            out.append((SITES[self.sites[i]], ms.value))
        return out

    def close(self):
        for i in range(self.capacity):
            self.hip.hipEventDestroy(self.start[i])
            self.hip.hipEventDestroy(self.stop[i])
