"""Tolerances and comparison helpers for GPU-vs-oracle parity.

Bars (element by element against the fp64 oracle on the same rounded inputs):
  * bf16 / fp16 inputs: max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <= 2e-3;
  * fp32 inputs: max |gpu - oracle| <= 1e-4;
  * cache contents and indices: bit-exact.
"""
import numpy as np
import torch

TOL = {torch.bfloat16: (2e-2, 2e-3), torch.float16: (2e-2, 2e-3), torch.float32: (1e-4, None)}


def to64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def assert_close(gpu, ref, dtype, what=""):
    g, r = to64(gpu), to64(ref)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    assert np.isfinite(g).all(), f"{what}: non-finite values in the GPU output"
    err = np.abs(g - r)
    max_abs = float(err.max()) if err.size else 0.0
    mean_abs = float(err.mean()) if err.size else 0.0
    tmax, tmean = TOL[dtype]
    assert max_abs <= tmax, f"{what}: max abs err {max_abs:.3g} > {tmax} (mean {mean_abs:.3g})"
    if tmean is not None:
        assert mean_abs <= tmean, f"{what}: mean abs err {mean_abs:.3g} > {tmean} (max {max_abs:.3g})"
    return max_abs, mean_abs
