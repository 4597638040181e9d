"""Fused residual add + RMSNorm (attn_residual_rms_norm) against the fp64
oracle: the updated residual bit-exact (both sides round the float32 sum to
the stored dtype), the normalised rows within the storage bound of the
exact value."""

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_05_amd as mi
from tests.gpu_util import DEV, check, check_stored, f64, say
from workloads import normal, rng, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def inputs(seed, rows, hidden, dtype):
    g = rng(seed)
    x = normal(g, (rows, hidden), dtype)
    r = normal(g, (rows, hidden), dtype)
    w = (1.0 + 0.1 * normal(g, (hidden,), torch.float32)).to(dtype)
    return x, r, w


# (seed, rows, hidden, dtype): the 1536-wide hidden state of the tutorial's
# serving model over the mixed step's 4224 new tokens; a ragged width
# (partial lane chunks); the widest and narrowest widths; fp32
SHAPES = [(81, 4224, 1536, torch.bfloat16), (82, 37, 1000, torch.bfloat16), (83, 9, 8192, torch.bfloat16),
          (84, 5, 8, torch.bfloat16), (85, 37, 1000, torch.float32), (86, 130, 4096, torch.float32)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[1]}x{s[2]}_{s[3]}" for s in SHAPES])
def test_residual_rms_norm(shape):
    seed, rows, hidden, dtype = shape
    say(f"case: residual rmsnorm {rows}x{hidden} {dtype}")
    x, r, w = inputs(seed, rows, hidden, dtype)
    y, h = mi.attn_residual_rms_norm(x.to(DEV), r.to(DEV), w.to(DEV), eps=1e-6)
    torch.cuda.synchronize()
    ry, rh = oracle.residual_rms_norm(to_f64(x), to_f64(r), to_f64(w), eps=1e-6, bf16=dtype == torch.bfloat16)
    assert np.array_equal(f64(h.cpu()), rh), "updated residual must be bit-exact"
    if dtype == torch.float32:
        check(f64(y.cpu()), ry, dtype, "rmsnorm y")
    else:
        check_stored(f64(y.cpu()), ry, dtype, "rmsnorm y")


def test_in_place_residual_and_zero_rows():
    """residual_out may be the residual tensor itself; a row whose sum is
    zero normalises to zero."""
    say("case: residual rmsnorm in place")
    x, r, w = inputs(87, 64, 1536, torch.bfloat16)
    x[5] = 0.0
    r[5] = 0.0
    xd, rd, wd = x.to(DEV), r.to(DEV), w.to(DEV)
    y1, h1 = mi.attn_residual_rms_norm(xd, rd, wd)
    y2, h2 = mi.attn_residual_rms_norm(xd, rd, wd, residual_out=rd)
    torch.cuda.synchronize()
    assert h2.data_ptr() == rd.data_ptr()
    assert torch.equal(h1.view(torch.int16), rd.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.all(y1[5] == 0)
