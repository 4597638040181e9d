"""Shared helpers for the GPU parity tests (tolerances and reporting)."""

import sys

import numpy as np
import torch

# Tolerances of the parity bar: fp32 max |err| <= 1e-5; bf16 (fp32
# accumulate) max |err| <= 1e-2 and mean |err| <= 1e-3; indexing bit-exact.
F32_MAX = 1e-5
BF16_MAX = 1e-2
BF16_MEAN = 1e-3

DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def errors(out, ref):
    e = np.abs(np.asarray(out, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    return float(e.max()) if e.size else 0.0, float(e.mean()) if e.size else 0.0


def check(out, ref, dtype, what=""):
    mx, mean = errors(out, ref)
    say(f"  {what}: max |err| {mx:.3e}  mean |err| {mean:.3e}")
    assert np.all(np.isfinite(np.asarray(out, dtype=np.float64))), f"{what}: non-finite output"
    if dtype == torch.float32:
        assert mx <= F32_MAX, f"{what}: max err {mx:.3e} > {F32_MAX}"
    else:
        assert mx <= BF16_MAX, f"{what}: max err {mx:.3e} > {BF16_MAX}"
        assert mean <= BF16_MEAN, f"{what}: mean err {mean:.3e} > {BF16_MEAN}"
    return mx, mean
