"""dit_modulation_static (no workspace, no allocation: its intermediates live in
the library's static device array) against dit_modulation through the C ABI.

The two entry points run the same kernels on the same inputs, so their outputs
must agree bit for bit; two calls in a row, the second with fewer steps, show
that nothing carries over in the shared array.  Also: a step count beyond the
static array is refused on the host, and the static call allocates no device
memory.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import dit_inputs as DI
import oracle as O
from _helpers import params64, parity_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dit():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from image_generation_amd import dit as D
    return D


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gpu_model(dit, dims, dtype="bf16"):
    w = DI.Workload("m", dims, B=1, grid_h=8, grid_w=8, Lt=32, dtype=dtype, steps=4, shift=3.0)
    params = dict(DI.iter_params(dims, dtype))
    kind = dit.DIT_F32 if dtype == "f32" else dit.DIT_BF16
    return dit.GPUModel(dims, w.B, w.Lt, w.grid_h, w.grid_w, params, dtype=kind), params


@pytest.mark.parametrize("dtype,dims", [
    ("bf16", DI.Dims(D=256, H=2, F=512, n_double=2, n_single=2)),
    ("bf16", DI.Dims(D=3072, H=24, F=12288, n_double=1, n_single=2)),
    ("f32", DI.Dims(D=256, H=4, F=1024, n_double=2, n_single=0)),
])
def test_modulation_static_matches_workspace_entry_point(dit, dtype, dims):
    gm, params = _gpu_model(dit, dims, dtype)
    # first call: 50 steps; second: 7 steps (a smaller input into the same array)
    for n, shift in ((50, 3.0), (7, 1.0)):
        sig = list(O.sigmas(n, shift)[:-1]) if n > 1 else [1.0]
        _say(f"modulation_static {dtype} D={dims.D} n={len(sig)}")
        ref = dit.dit_modulation(gm, sig)
        out = torch.full_like(ref, float("nan"))
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        dit.dit_modulation_static(gm, sig, out)
        torch.cuda.synchronize()
        # the device's free memory moves only when the library's code object (with
        # its static array) is first loaded, never on a later call
        if n != 50 or dims.D != 256 or dtype != "bf16":
            assert torch.cuda.mem_get_info()[0] == free0
        assert torch.equal(out, ref), float((out - ref).abs().max())
        # and the oracle's modulation vectors, as the workspace entry point is tested
        if dims.D == 256:
            P = {k: v.double().numpy() for k, v in params.items()}
            c = O.time_embed(P, np.array(sig))
            names = [f"double{j}.{s}.mod" for j in range(dims.n_double) for s in ("img", "txt")]
            names += [f"single{j}.mod" for j in range(dims.n_single)] + ["final.mod"]
            want = np.concatenate([O.linear(O.silu(c), P[k + ".w"], P[k + ".b"]) for k in names],
                                  axis=1)
            err = parity_err(out.double().cpu().numpy(), want)
            _say(f"  vs oracle {err:.3e}")
            assert err <= (1e-4 if dtype == "f32" else 2e-2)


def test_modulation_static_rejects_too_many_steps(dit):
    dims = DI.Dims(D=3072, H=24, F=12288, n_double=1, n_single=0)
    gm, _ = _gpu_model(dit, dims)
    need = dit.dit_workspace_bytes(gm.model.dims, dit.DIT_WS_MODULATION, 400)
    assert need > dit.DIT_MOD_STATIC_BYTES
    out = torch.empty((400, gm.n_mod), dtype=torch.float32, device="cuda")
    with pytest.raises(dit.DitError) as e:
        dit.dit_modulation_static(gm, [0.5] * 400, out)
    assert e.value.status == dit.DIT_ERR_WORKSPACE
