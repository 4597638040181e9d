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


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    x = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(x)) - 7)


def check_bf16_output(out, ref, what=""):
    """A bf16 output against the exact value at the bf16 bar: max |err| <=
    1e-2 on every element with |O| < 4, mean |err| <= 1e-3 over all.  Where
    |O| >= 4 no bf16 number is guaranteed within 1e-2 of the exact value
    (half an ulp there is 1/64), so those elements must be faithfully
    rounded: one of the two bf16 neighbours of the exact value, i.e. less
    than one ulp away."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out - ref)
    small = np.abs(ref) < 4.0
    mx = float(err[small].max()) if small.any() else 0.0
    big = ~small
    worst = float((err[big] / bf16_ulp(ref[big])).max()) if big.any() else 0.0
    say(f"  {what}: max |err| {mx:.3e} where |O| < 4, mean |err| {err.mean():.3e}; "
        f"{int(big.sum())} elements with |O| >= 4, worst err/ulp {worst:.3f}")
    assert mx <= BF16_MAX, f"{what}: max err {mx:.3e} > {BF16_MAX} where |O| < 4"
    assert err.mean() <= BF16_MEAN, f"{what}: mean err {err.mean():.3e} > {BF16_MEAN}"
    assert worst < 1.0, f"{what}: an element with |O| >= 4 is not faithfully rounded ({worst:.3f} ulp)"


def check_stored(out, exact, dtype, what=""):
    """Values the method computes in fp32 and stores in `dtype` (rotated q
    and k): compared with the exact fp64 value.  bf16 storage: at most half a
    bf16 ulp of the exact value plus the fp32 arithmetic error (<= 1e-5 here),
    since an absolute 1e-2 is finer than bf16 spacing once |x| >= 4.  fp32:
    the fp32 bar."""
    out = np.asarray(out, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    err = np.abs(out - exact)
    if dtype == torch.float32:
        bound = np.full_like(exact, F32_MAX)
    else:
        bound = 0.5 * bf16_ulp(np.abs(exact) + 1e-5) + 1e-5
    worst = float((err / bound).max()) if err.size else 0.0
    say(f"  {what}: max |err| {err.max():.3e}  worst err/bound {worst:.3f}")
    assert np.all(err <= bound), f"{what}: error above the storage bound ({worst:.3f} of it)"
