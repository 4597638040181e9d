"""CPU oracle for the fused residual add + RMS normalisation.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only the tests and the benchmark call it.  It shares no code with the HIP
library.

Source: the tutorial "Fast Attention Kernels and Operator Fusion"
(Machine Learning Mastery), §Operator Fusion, its residual RMSNorm example:
the residual is added to the input, each row is divided by the root mean
square of the sum (eps under the root, default 1e-6) and scaled elementwise
by a weight vector; the function returns the normalised rows and the updated
residual (the sum).

Readings:
  * The updated residual is stored in the input dtype, so it is the sum
    rounded once to that dtype; the sum itself is taken in float32 before
    that rounding, as the example's elementwise add of two bf16 tensors
    does.  Where that rounding decides a stored value both sides decide it
    in float32.
  * The mean of squares and the normalised output are float64 here, from
    the stored sum.  The example also rounds the reciprocal root and the
    products to the input dtype; those are intermediate roundings of its
    library calls, not part of the definition, and the tolerance covers the
    single rounding of the stored output.
"""

from __future__ import annotations

import numpy as np

from .attention import round_bf16

__all__ = ["residual_rms_norm"]


def residual_rms_norm(x, residual, weight, eps=1e-6, bf16=True):
    """(normalised [N, H], updated residual [N, H]) in float64.

    x, residual: [N, H]; weight: [H] (float64 arrays holding the exact input
    values).  bf16: the updated residual is rounded to bfloat16 (else it is
    the float32 sum)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(residual, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    h = (x.astype(np.float32) + r.astype(np.float32)).astype(np.float64)   # the float32 sum
    if bf16:
        h = round_bf16(h)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * w, h
