"""Seeded synthetic inputs for the DiT denoise step.

This module is shared by the CPU oracle and the HIP path. It holds shapes and
random-number plumbing only: no step of the method's arithmetic lives here.

Every tensor is drawn with its own ``torch.Generator('cpu')`` seed from a
standard normal in fp32, multiplied by its standard deviation, and then rounded
(round-to-nearest-even, torch's own cast) to the storage dtype.  Both sides read
the same rounded values, so input rounding is never counted as error.

Seed plan:
  * 0            latents (the initial noise)
  * 1            text tokens
  * 2            block activations (the joint residual stream in block tests)
  * 3            per-block modulation vectors (block tests)
  * 1000 + k     the k-th parameter tensor in the fixed enumeration of
                 :func:`param_specs`
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterator, List, Tuple

import torch

SEED_LATENTS = 0
SEED_TEXT = 1
SEED_ACT = 2
SEED_MOD = 3
SEED_PARAM_BASE = 1000

WEIGHT_STD = 0.02
MOD_STD = 0.1

FREQ_DIM = 256          # width of the sinusoidal timestep embedding
LATENT_CHANNELS = 16    # latent channels before 2x2 patching
PATCH = 2
C_IN = LATENT_CHANNELS * PATCH * PATCH   # 64 patch features per image token

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Dims:
    """Model widths."""
    D: int            # hidden size
    H: int            # attention heads
    F: int            # MLP hidden size
    n_double: int     # double-stream blocks
    n_single: int     # single-stream blocks
    C_in: int = C_IN

    @property
    def d(self) -> int:
        return self.D // self.H


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: model widths, token counts, loop settings."""
    name: str
    dims: Dims
    B: int                  # batch rows (2 = CFG pos/neg pair)
    grid_h: int             # patch-grid rows
    grid_w: int             # patch-grid columns
    Lt: int                 # text tokens
    dtype: str              # storage / compute dtype of the path: f32, bf16, fp8
    steps: int = 0
    shift: float = 1.0
    threshold: float = 0.0  # First-Block-Cache threshold (0 = never skip)
    guidance: float = 0.0   # CFG scale (B == 2 only)

    @property
    def Li(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def L(self) -> int:
        return self.Lt + self.Li

    @property
    def image_px(self) -> int:
        # patch 2 on a latent that is 1/8 of the image side
        return self.grid_h * PATCH * 8


FLUX_BLOCK = Dims(D=3072, H=24, F=12288, n_double=1, n_single=0)
FLUX_FULL = Dims(D=3072, H=24, F=12288, n_double=19, n_single=38)
TINY = Dims(D=256, H=4, F=1024, n_double=2, n_single=0)

WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 model, 4 Euler steps, 16x16 grid + 32 text tokens
    "tiny_fp32": Workload("tiny_fp32", TINY, B=1, grid_h=16, grid_w=16, Lt=32,
                          dtype="f32", steps=4, shift=1.0),
    # one FLUX-shaped double-stream block at 1024px
    "block_1024": Workload("block_1024", FLUX_BLOCK, B=1, grid_h=64, grid_w=64,
                           Lt=512, dtype="bf16"),
    # one block at 2048px, CFG pair
    "block_2048_cfg": Workload("block_2048_cfg", FLUX_BLOCK, B=2, grid_h=128,
                               grid_w=128, Lt=512, dtype="bf16"),
    # full 19+38 model, 1024px, 28 Euler steps, shift 3, FBC 0.12
    "flux_1024_28step": Workload("flux_1024_28step", FLUX_FULL, B=1, grid_h=64,
                                 grid_w=64, Lt=512, dtype="bf16", steps=28,
                                 shift=3.0, threshold=0.12),
    # fp8 W8A8, 2048px, CFG 3.5, 50 steps, FBC 0.2
    "flux_2048_fp8_cfg": Workload("flux_2048_fp8_cfg", FLUX_FULL, B=2,
                                  grid_h=128, grid_w=128, Lt=512, dtype="fp8",
                                  steps=50, shift=3.0, threshold=0.2,
                                  guidance=3.5),
}


def storage_dtype(dtype: str) -> torch.dtype:
    """Storage dtype of weights and activations (fp8 models keep bf16 masters)."""
    return _DTYPES.get(dtype, torch.bfloat16)


def randn(shape, seed: int, std: float = 1.0, dtype: str = "bf16") -> torch.Tensor:
    """N(0, std^2) on the CPU from its own seed, rounded to ``dtype``."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(storage_dtype(dtype))


def device_randn(shape, seed: int, std: float, device, dtype=torch.bfloat16) -> torch.Tensor:
    """Same distribution drawn by torch's device generator (fast, large models).

    Used only where no CPU oracle reads the values (throughput runs).
    """
    g = torch.Generator(device=device).manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    t.mul_(std)
    return t.to(dtype)


# ---------------------------------------------------------------------------
# parameter enumeration (shapes follow torch.nn.Linear: W is [out, in])
# ---------------------------------------------------------------------------

def double_block_specs(dims: Dims, prefix: str) -> List[Tuple[str, Tuple[int, ...]]]:
    D, F = dims.D, dims.F
    out = []
    for s in ("img", "txt"):
        p = f"{prefix}.{s}"
        out += [(f"{p}.mod.w", (6 * D, D)), (f"{p}.mod.b", (6 * D,)),
                (f"{p}.qkv.w", (3 * D, D)), (f"{p}.qkv.b", (3 * D,)),
                (f"{p}.proj.w", (D, D)), (f"{p}.proj.b", (D,)),
                (f"{p}.mlp1.w", (F, D)), (f"{p}.mlp1.b", (F,)),
                (f"{p}.mlp2.w", (D, F)), (f"{p}.mlp2.b", (D,))]
    return out


def single_block_specs(dims: Dims, prefix: str) -> List[Tuple[str, Tuple[int, ...]]]:
    D, F = dims.D, dims.F
    return [(f"{prefix}.mod.w", (3 * D, D)), (f"{prefix}.mod.b", (3 * D,)),
            (f"{prefix}.lin1.w", (3 * D + F, D)), (f"{prefix}.lin1.b", (3 * D + F,)),
            (f"{prefix}.lin2.w", (D, D + F)), (f"{prefix}.lin2.b", (D,))]


def param_specs(dims: Dims) -> List[Tuple[str, Tuple[int, ...]]]:
    """The fixed enumeration of every parameter tensor of the model."""
    D = dims.D
    specs = [("time.w1", (D, FREQ_DIM)), ("time.b1", (D,)),
             ("time.w2", (D, D)), ("time.b2", (D,)),
             ("img_in.w", (D, dims.C_in)), ("img_in.b", (D,))]
    for j in range(dims.n_double):
        specs += double_block_specs(dims, f"double{j}")
    for j in range(dims.n_single):
        specs += single_block_specs(dims, f"single{j}")
    specs += [("final.mod.w", (2 * D, D)), ("final.mod.b", (2 * D,)),
              ("final.out.w", (dims.C_in, D)), ("final.out.b", (dims.C_in,))]
    return specs


def iter_params(dims: Dims, dtype: str, only_prefix: str = None) -> Iterator[Tuple[str, torch.Tensor]]:
    """Yield (name, tensor) for every parameter, seeded 1000 + enumeration index."""
    for k, (name, shape) in enumerate(param_specs(dims)):
        if only_prefix is not None and not name.startswith(only_prefix):
            continue
        yield name, randn(shape, SEED_PARAM_BASE + k, WEIGHT_STD, dtype)


def block_params(dims: Dims, dtype: str, kind: str = "double") -> Dict[str, torch.Tensor]:
    """Parameters of one stand-alone block (block tests); seeds 1000 + k."""
    specs = double_block_specs(dims, "blk") if kind == "double" else single_block_specs(dims, "blk")
    return {name[4:]: randn(shape, SEED_PARAM_BASE + k, WEIGHT_STD, dtype)
            for k, (name, shape) in enumerate(specs)}


def block_inputs(w: Workload, kind: str = "double", batch_mod: bool = True) -> Dict[str, torch.Tensor]:
    """Joint activations x [B, L, D] ~ N(0,1) and modulation vectors ~ N(0, 0.1).

    Double blocks take 12 vectors per batch row (image 6 then text 6), single
    blocks 3.  With ``batch_mod`` every batch row gets its own vectors.
    """
    D = w.dims.D
    nmod = 12 if kind == "double" else 3
    x = randn((w.B, w.L, D), SEED_ACT, 1.0, w.dtype)
    mb = w.B if batch_mod else 1
    mod = randn((mb, nmod, D), SEED_MOD, MOD_STD, "f32")
    return {"x": x, "mod": mod}


def latents(w: Workload) -> torch.Tensor:
    """Initial noise in token layout [1, Li, C_in], fp32 (shared by a CFG pair)."""
    return randn((1, w.Li, w.dims.C_in), SEED_LATENTS, 1.0, "f32")


def text_tokens(w: Workload) -> torch.Tensor:
    """Text-encoder output stand-in [B, Lt, D]; CFG rows differ (pos, neg)."""
    return randn((w.B, w.Lt, w.dims.D), SEED_TEXT, 1.0, w.dtype)
